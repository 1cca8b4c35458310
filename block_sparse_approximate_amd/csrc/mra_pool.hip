// mra_pool.hip — step 1 pooling ([MRA] "第一步"): the masked mean of Q, K
// (and V in full mode, unless the logits launch pools it) over each 32-token
// block, the valid-token count of each block, and the per-block mask word.
//
// Mapping: a workgroup is one pooling unit (pool_unit in mra_pool_unit.h):
// kPoolThreads / (d / 2) consecutive blocks of one tensor and head, one
// thread per block and channel pair; all workgroups of a head run on the
// same XCD.  (Workgroups of 1024 threads and 128 KiB of staging were
// measured slower at N = 4096 with three tensors: one workgroup per CU left
// part of the grid for a second round.)
#include "mra_pool_unit.h"

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
    extern __shared__ __align__(16) unsigned char tile[];   // kPoolBlocks blocks

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
        if (gt < p.BH) {
            p.ncand[(size_t)gt * kCandStride] = 0u;       // pre-marked candidates
            p.ncand[(size_t)gt * kCandStride + 1] = 0u;   // workgroups of the head whose logits are stored
            p.ncand[(size_t)gt * kCandStride + 2] = 0u;   // workgroups of the head whose V pooling is stored
        }
    }
    // workgroup g runs on XCD g % 8; every workgroup of head bh goes to XCD
    // bh % 8, the XCD whose L2 the later stages of that head use
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_head = ntens * groups_per_head;
    const int hm = slot / per_head;
    const int rem = slot - hm * per_head;
    const int tens = rem / groups_per_head;
    const int bh = xcd + 8 * hm;
    const int blk0 = (rem - tens * groups_per_head) * kPoolBlocks;
    pool_unit<DT, HD, kPoolBlocks>(p, tens, bh, blk0, bh < p.BH, (int)threadIdx.x, tile);
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
    const int ntens = p.mode == 0 && !p.v_in_logits ? 3 : 2;
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
