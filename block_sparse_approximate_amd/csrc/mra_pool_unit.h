// mra_pool_unit.h — one unit of step 1 pooling ([MRA] "第一步"): the masked
// mean over each 32-token block of kBlocks consecutive blocks of one tensor
// and head.  The pooling kernel runs it for Q and K (and V where V is not
// folded into the logits launch); the logits launch runs it for V beside its
// logits workgroups.
//
// Canonical fp32 order (the same as the CPU oracle's): for every channel the
// sum starts at +0.0f and adds the valid tokens t = 0..31 of the block in
// order; the mean is that sum divided by (float)count, correctly rounded;
// an empty block pools to zeros.  Translation units that include this header
// are built with -ffp-contract=off.
#pragma once
#include "mra_common.h"

namespace mra {

// A unit is kBlocks * (HD / 2) threads (t = 0 ..), one per block and channel
// pair.  They first issue all of their 16-byte loads of the unit's blocks
// (one contiguous run of token rows, fully coalesced, one round trip) and
// store them in the staging tile, then each sums two channels of one block
// over its 32 rows in token order.  The caller's workgroup reaches the one
// barrier inside with all of its threads; inactive threads (active false,
// e.g. a unit past the last head) load and write nothing.
template <int DT, int HD, int kBlocks>
__device__ __forceinline__ void pool_unit(const Params& p, int tens, int bh, int blk0, bool active, int t,
                                          unsigned char* tile) {
    constexpr int kThreads = kBlocks * (HD / 2);
    constexpr int kEs = DT == 1 ? 2 : 4;              // bytes per element
    constexpr int kBlockBytes = kBlock * HD * kEs;    // 4 to 16 KiB
    constexpr int kLoads = kBlocks * kBlockBytes / 16 / kThreads;
    active = active && t < kThreads;
    const int nblk = active ? min(kBlocks, p.nb - blk0) : 0;
    const int b = active ? bh / p.H : 0;

    const unsigned char* src = static_cast<const unsigned char*>(tens == 0 ? p.q : (tens == 1 ? p.k : p.v)) +
                               ((size_t)bh * p.N + (size_t)blk0 * kBlock) * HD * kEs;
    uint4 v[kLoads];
#pragma unroll
    for (int e = 0; e < kLoads; e++) {
        const int off = (t + e * kThreads) * 16;
        v[e] = off < nblk * kBlockBytes ? *reinterpret_cast<const uint4*>(src + off) : make_uint4(0, 0, 0, 0);
    }
    if (active) {
#pragma unroll
        for (int e = 0; e < kLoads; e++) *reinterpret_cast<uint4*>(tile + (t + e * kThreads) * 16) = v[e];
    }

    // thread -> (block bk, channel pair cp)
    const int bk = t / (HD / 2), cp = t % (HD / 2);
    const int blk = blk0 + bk;
    uint32_t bits = 0xFFFFFFFFu;
    if (p.mask && bk < nblk) {
        const uint4* mp = reinterpret_cast<const uint4*>(p.mask + (size_t)b * p.N + (size_t)blk * kBlock);
        const uint4 m0 = mp[0], m1 = mp[1];
        const uint32_t mw[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
        bits = 0;
#pragma unroll
        for (int x = 0; x < 32; x++) bits |= (((mw[x >> 2] >> (8 * (x & 3))) & 0xFFu) != 0 ? 1u : 0u) << x;
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
    for (int x = 0; x < kBlock; x++) {
        float x0, x1;
        if constexpr (DT == 1) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(col + x * HD * kEs);
            x0 = __uint_as_float(w << 16);
            x1 = __uint_as_float(w & 0xFFFF0000u);
        } else {
            const float2 w = *reinterpret_cast<const float2*>(col + x * HD * kEs);
            x0 = w.x;
            x1 = w.y;
        }
        if ((bits >> x) & 1u) {
            a0 = a0 + x0;
            a1 = a1 + x1;
        }
    }
    const float fc = (float)count;
    float* dst = tens == 0 ? p.qhat : (tens == 1 ? p.khat : p.vhat);
    *reinterpret_cast<float2*>(dst + ((size_t)bh * p.nb + blk) * HD + 2 * cp) =
        count > 0 ? make_float2(a0 / fc, a1 / fc) : make_float2(0.0f, 0.0f);
}

// V pooling in the logits launch: units of kVUnitBytes of staging, two per
// workgroup of that launch.
constexpr int kVUnitBytes = 32 * 1024;
__host__ __device__ constexpr int v_unit_blocks(int dt, int hd) { return kVUnitBytes / (kBlock * hd * (dt == 1 ? 2 : 4)); }
constexpr int kVUnitsPerGroup = 2;
constexpr int kVUnitStride = 256;   // threads set aside per unit (a unit uses 128 or 256 of them)

}  // namespace mra
