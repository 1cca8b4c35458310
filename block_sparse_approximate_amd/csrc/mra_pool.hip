// mra_pool.hip — step 1 pooling ([MRA] "第一步"): the masked mean of Q, K
// (and V in full mode) over each 32-token block, the valid-token count of
// each block, and the per-block mask word.
//
// Canonical fp32 order (the same as the CPU oracle's): for every channel the
// sum starts at +0.0f and adds the valid tokens t = 0..31 of the block in
// order; the mean is that sum divided by (float)count, correctly rounded;
// an empty block pools to zeros.  Built with -ffp-contract=off.
//
// Mapping (wave64): a wave pools 8 blocks of one tensor; each group of 8
// lanes owns one block and each lane 8 consecutive channels, so every load
// instruction reads 8 full 128-byte token rows (bf16, d = 64).  The sum over
// tokens stays inside one lane, which keeps the canonical order.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kBlocksPerWave = 8;
constexpr int kBlocksPerWG = kBlocksPerWave * (kPoolThreads / 64);

template <int DT>  // 0 = fp32, 1 = bf16
__device__ __forceinline__ void load8(const void* base, size_t elem, float (&x)[8]) {
    if constexpr (DT == 1) {
        const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    } else {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
        const float4 a = p[0], b = p[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <int DT>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(Params p, int ntens, int total_tiles,
                                                            int zero_words) {
    // Clear the selection histogram and the per-head counters for the next
    // stage (stream order makes this visible to it).
    {
        const int gt = blockIdx.x * kPoolThreads + threadIdx.x;
        const int stride = gridDim.x * kPoolThreads;
        if (gt == 0) *p.error = 0;
        for (int w = gt; w < zero_words; w += stride) {
            if (w < p.BH * kHistBins) p.hist[w] = 0u;
            else p.done[w - p.BH * kHistBins] = 0u;
        }
    }
    const int lane = threadIdx.x & 63;
    const int tile = blockIdx.x * kBlocksPerWG + (threadIdx.x >> 6) * kBlocksPerWave + (lane >> 3);
    if (tile >= total_tiles) return;
    const int sub = lane & 7;                 // channels sub*8 .. sub*8+7
    const int per_tensor = p.BH * p.nb;
    const int tens = tile / per_tensor;
    const int rem = tile - tens * per_tensor;
    const int bh = rem / p.nb;
    const int blk = rem - bh * p.nb;
    const int b = bh / p.H;

    uint32_t bits = 0xFFFFFFFFu;
    if (p.mask) {
        const uint4* mp = reinterpret_cast<const uint4*>(p.mask + (size_t)b * p.N + (size_t)blk * kBlock);
        const uint4 m0 = mp[0], m1 = mp[1];
        const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        bits = 0;
#pragma unroll
        for (int t = 0; t < 32; t++)
            bits |= (((mw[t >> 2] >> (8 * (t & 3))) & 0xFFu) != 0 ? 1u : 0u) << t;
    }
    const int count = __popc(bits);
    if (tens == 0 && (bh % p.H) == 0 && sub == 0) {
        p.cnt[b * p.nb + blk] = count;
        p.mbits[b * p.nb + blk] = bits;
    }

    const void* src = tens == 0 ? p.q : (tens == 1 ? p.k : p.v);
    float* dst = tens == 0 ? p.qhat : (tens == 1 ? p.khat : p.vhat);
    const size_t row0 = ((size_t)bh * p.N + (size_t)blk * kBlock) * kHeadDim + sub * 8;

    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; c++) acc[c] = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; half++) {
        float x[16][8];
#pragma unroll
        for (int t = 0; t < 16; t++) load8<DT>(src, row0 + (size_t)(half * 16 + t) * kHeadDim, x[t]);
#pragma unroll
        for (int t = 0; t < 16; t++) {
            if ((bits >> (half * 16 + t)) & 1u) {
#pragma unroll
                for (int c = 0; c < 8; c++) acc[c] = acc[c] + x[t][c];
            }
        }
    }
    float outv[8];
    const float fc = (float)count;
#pragma unroll
    for (int c = 0; c < 8; c++) outv[c] = count > 0 ? acc[c] / fc : 0.0f;
    float4* o = reinterpret_cast<float4*>(dst + ((size_t)bh * p.nb + blk) * kHeadDim + sub * 8);
    o[0] = make_float4(outv[0], outv[1], outv[2], outv[3]);
    o[1] = make_float4(outv[4], outv[5], outv[6], outv[7]);
}

}  // namespace

hipError_t launch_pool(const Params& p, hipStream_t s) {
    const int ntens = p.mode == 0 ? 3 : 2;
    const int total_tiles = ntens * p.BH * p.nb;
    const int grid = (total_tiles + kBlocksPerWG - 1) / kBlocksPerWG;
    const int zero_words = p.BH * kHistBins + p.BH;
    if (p.d != kHeadDim) return hipErrorInvalidValue;
    if (p.dtype == 1)
        hipLaunchKernelGGL(pool_kernel<1>, dim3(grid), dim3(kPoolThreads), 0, s, p, ntens, total_tiles,
                           zero_words);
    else
        hipLaunchKernelGGL(pool_kernel<0>, dim3(grid), dim3(kPoolThreads), 0, s, p, ntens, total_tiles,
                           zero_words);
    return hipGetLastError();
}

}  // namespace mra
