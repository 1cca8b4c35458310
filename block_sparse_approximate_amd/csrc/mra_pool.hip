// mra_pool.hip — step 1 pooling ([MRA] "第一步"): the masked mean of Q, K
// (and V in full mode) over each 32-token block, the valid-token count of
// each block, and the per-block mask word.
//
// Canonical fp32 order (the same as the CPU oracle's): for every channel the
// sum starts at +0.0f and adds the valid tokens t = 0..31 of the block in
// order; the mean is that sum divided by (float)count, correctly rounded;
// an empty block pools to zeros.  Built with -ffp-contract=off.
//
// Mapping: a workgroup of kPoolThreads threads pools kPoolThreads / (d / 2)
// consecutive blocks of one tensor and head (one thread per block and
// channel pair), which are one contiguous run of token rows; all workgroups
// of a head run on the same XCD.  Every thread first issues all of its
// 16-byte loads of that run (fully coalesced, one round trip), stores them in
// LDS, and then each thread sums two channels of one block over its 32 rows
// in token order.  (Workgroups of 1024 threads and 128 KiB of staging were
// measured slower at N = 4096 with three tensors: one workgroup per CU left
// part of the grid for a second round.)
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kPoolMaxThreads = 256;
constexpr int kPoolTileBytes = 64 * 1024;    // LDS staging per workgroup, at most
// blocks per workgroup (one thread per block and channel pair): as many as
// fill the staging tile, up to kPoolMaxThreads threads
__host__ __device__ constexpr int pool_blocks(int dt, int hd) {
    return (kPoolTileBytes / (kBlock * hd * (dt == 1 ? 2 : 4))) * (hd / 2) > kPoolMaxThreads
               ? kPoolMaxThreads / (hd / 2)
               : kPoolTileBytes / (kBlock * hd * (dt == 1 ? 2 : 4));
}
__host__ __device__ constexpr int pool_threads(int dt, int hd) { return pool_blocks(dt, hd) * (hd / 2); }

template <int DT, int HD>  // DT: 0 = fp32, 1 = bf16; HD: channels per head
__global__ __launch_bounds__(kPoolMaxThreads) void pool_kernel(Params p, int ntens, int groups_per_head,
                                                               size_t zero_words) {
    constexpr int kPoolThreads = pool_threads(DT, HD);
    constexpr int kPoolBlocks = pool_blocks(DT, HD);
    constexpr int kEs = DT == 1 ? 2 : 4;              // bytes per element
    constexpr int kBlockBytes = kBlock * HD * kEs;    // 4 to 16 KiB
    constexpr int kLoads = kPoolBlocks * kBlockBytes / 16 / kPoolThreads;
    extern __shared__ __align__(16) unsigned char tile[];   // kPoolBlocks * kBlockBytes

    // Clear the selection histogram and candidate counts for the next stages
    // (stream order makes this visible to them).
    {
        const size_t gt = (size_t)blockIdx.x * kPoolThreads + threadIdx.x;
        const size_t stride = (size_t)gridDim.x * kPoolThreads;
        if (gt == 0) {
            p.error[0] = 0;
            p.error[1] = p.save_stats;   // the backward checks that the statistics were kept
        }
        for (size_t w = gt; w < zero_words; w += stride) p.hist[w] = 0u;
        if (gt < p.BH) p.ncand[(size_t)gt * kCandStride] = 0u;
    }
    // workgroup g runs on XCD g % 8; every workgroup of head bh goes to XCD
    // bh % 8, the XCD whose L2 the later stages of that head use
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_head = ntens * groups_per_head;
    const int hm = slot / per_head;
    const int rem = slot - hm * per_head;
    const int tens = rem / groups_per_head;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return;
    const int blk0 = (rem - tens * groups_per_head) * kPoolBlocks;
    const int nblk = min(kPoolBlocks, p.nb - blk0);
    const int b = bh / p.H;
    const int tid = threadIdx.x;

    const unsigned char* src = static_cast<const unsigned char*>(tens == 0 ? p.q : (tens == 1 ? p.k : p.v)) +
                               ((size_t)bh * p.N + (size_t)blk0 * kBlock) * HD * kEs;
    uint4 v[kLoads];
#pragma unroll
    for (int e = 0; e < kLoads; e++) {
        const int off = (tid + e * kPoolThreads) * 16;
        v[e] = off < nblk * kBlockBytes ? *reinterpret_cast<const uint4*>(src + off) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < kLoads; e++) *reinterpret_cast<uint4*>(tile + (tid + e * kPoolThreads) * 16) = v[e];

    // thread -> (block bk, channel pair cp)
    const int bk = tid / (HD / 2), cp = tid % (HD / 2);
    const int blk = blk0 + bk;
    uint32_t bits = 0xFFFFFFFFu;
    if (p.mask && bk < nblk) {
        const uint4* mp = reinterpret_cast<const uint4*>(p.mask + (size_t)b * p.N + (size_t)blk * kBlock);
        const uint4 m0 = mp[0], m1 = mp[1];
        const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        bits = 0;
#pragma unroll
        for (int t = 0; t < 32; t++) bits |= (((mw[t >> 2] >> (8 * (t & 3))) & 0xFFu) != 0 ? 1u : 0u) << t;
    }
    __syncthreads();
    if (bk >= nblk) return;
    const int count = __popc(bits);
    if (tens == 0 && (bh % p.H) == 0 && cp == 0) {
        p.cnt[b * p.nb + blk] = count;
        p.mbits[b * p.nb + blk] = bits;
    }
    float a0 = 0.0f, a1 = 0.0f;
    const unsigned char* col = tile + bk * kBlockBytes + cp * 2 * kEs;
#pragma unroll
    for (int t = 0; t < kBlock; t++) {
        float x0, x1;
        if constexpr (DT == 1) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(col + t * HD * kEs);
            x0 = __uint_as_float(w << 16);
            x1 = __uint_as_float(w & 0xFFFF0000u);
        } else {
            const float2 w = *reinterpret_cast<const float2*>(col + t * HD * kEs);
            x0 = w.x;
            x1 = w.y;
        }
        if ((bits >> t) & 1u) {
            a0 = a0 + x0;
            a1 = a1 + x1;
        }
    }
    const float fc = (float)count;
    float* dst = tens == 0 ? p.qhat : (tens == 1 ? p.khat : p.vhat);
    *reinterpret_cast<float2*>(dst + ((size_t)bh * p.nb + blk) * HD + 2 * cp) =
        count > 0 ? make_float2(a0 / fc, a1 / fc) : make_float2(0.0f, 0.0f);
}

}  // namespace

template <int DT, int HD>
static hipError_t launch_pool_dt(const Params& p, hipStream_t s, int ntens, int groups_per_head, size_t zero_words) {
    constexpr size_t kLds = (size_t)pool_blocks(DT, HD) * kBlock * HD * (DT == 1 ? 2 : 4);
    static const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&pool_kernel<DT, HD>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (a != hipSuccess) return a;
    const int grid = 8 * ((p.BH + 7) / 8) * ntens * groups_per_head;
    hipLaunchKernelGGL((pool_kernel<DT, HD>), dim3(grid), dim3(pool_threads(DT, HD)), kLds, s, p, ntens,
                       groups_per_head, zero_words);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_pool_t(const Params& p, hipStream_t s) {
    const int ntens = p.mode == 0 ? 3 : 2;
    const int pb = p.dtype == 1 ? pool_blocks(1, HD) : pool_blocks(0, HD);
    const int groups_per_head = (p.nb + pb - 1) / pb;
    const size_t zero_words = (size_t)p.BH * kHistBins;
    return p.dtype == 1 ? launch_pool_dt<1, HD>(p, s, ntens, groups_per_head, zero_words)
                        : launch_pool_dt<0, HD>(p, s, ntens, groups_per_head, zero_words);
}

hipError_t launch_pool(const Params& p, hipStream_t s) {
    if (p.d == 64) return launch_pool_t<64>(p, s);
    if (p.d == 128) return launch_pool_t<128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mra
