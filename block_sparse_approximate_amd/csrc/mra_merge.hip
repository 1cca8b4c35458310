// mra_merge.hip — step 4 ([MRA] "第四步"): the low-resolution attention on
// the unselected blocks (full mode) and the merge of high- and
// low-resolution partial results through a shared row maximum.
//
// lowres_kernel: for block row i of head bh,
//   W_ij = cnt_j * exp(S_ij - m_i)  for j not selected in row i, cnt_j > 0
//   lo_o[i] = sum_j W_ij vhat_j,  lo_l[i] = sum_j W_ij          (fp32)
// m_i is the row max of the low-res logits, so every weight is <= cnt_j.
// Each pooled block stands for cnt_j keys, hence the cnt_j factor; with
// block-constant queries and keys this makes full mode equal dense attention.
// A workgroup takes 8 block rows and streams vhat through LDS in tiles of
// 32 key blocks, so vhat is read once per 8 rows.
//
// merge_kernel: block rows whose selection did not fit one attention work
// item.  For each query token t of row i it joins the partials
// (O_c, m_c, l_c) of the row's items and, in full mode, the low-res part:
//   M = max(m_c, m_i);  out_t = (sum_c O_c 2^(m_c-M) + lo_o[i] e^(m_i-M))
//                              / (sum_c l_c 2^(m_c-M) + lo_l[i] e^(m_i-M))
// (high-res maxima are kept in log2 units); 0 when the denominator is 0 or
// the token is padding.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kLoRows = 8;
constexpr int kLoTile = 32;
constexpr int kLoThreads = 256;

__global__ __launch_bounds__(kLoThreads) void lowres_kernel(Params p) {
    __shared__ __align__(16) float vt[kLoTile][kHeadDim];
    __shared__ float wt[kLoRows][kLoTile];
    const int nb = p.nb, words = p.words;
    const int tiles = (nb + kLoRows - 1) / kLoRows;
    const int bh = blockIdx.x / tiles;
    const int row0 = (blockIdx.x - bh * tiles) * kLoRows;
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const int r = tid >> 5;             // row of this thread (0..7)
    const int c2 = (tid & 31) * 2;      // two channels
    const int i = row0 + r;
    const float* S = p.logits + (size_t)bh * nb * nb;
    const float* vh = p.vhat + (size_t)bh * nb * kHeadDim;
    const uint32_t* bits = p.selbits + (size_t)bh * nb * words;
    const int* cnt = p.cnt + (size_t)b * nb;
    float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
    for (int j0 = 0; j0 < nb; j0 += kLoTile) {
        __syncthreads();
        for (int x = tid; x < kLoTile * (kHeadDim / 4); x += kLoThreads) {
            const int jj = x / (kHeadDim / 4), c4 = (x % (kHeadDim / 4)) * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j0 + jj < nb) v = *reinterpret_cast<const float4*>(vh + (size_t)(j0 + jj) * kHeadDim + c4);
            *reinterpret_cast<float4*>(&vt[jj][c4]) = v;
        }
        {
            const int jj = tid & 31, j = j0 + jj;
            float w = 0.f;
            if (i < nb && j < nb) {
                const bool sel = (bits[(size_t)i * words + (j >> 5)] >> (j & 31)) & 1u;
                const int cj = cnt[j];
                if (!sel && cj > 0)
                    w = (float)cj * __builtin_amdgcn_exp2f((S[(size_t)i * nb + j] - p.rowmax[(size_t)bh * nb + i]) * kLog2e);
            }
            wt[r][jj] = w;
        }
        __syncthreads();
#pragma unroll 8
        for (int jj = 0; jj < kLoTile; jj++) {
            const float w = wt[r][jj];
            const float2 v = *reinterpret_cast<const float2*>(&vt[jj][c2]);
            acc0 = __builtin_fmaf(w, v.x, acc0);
            acc1 = __builtin_fmaf(w, v.y, acc1);
            lsum += w;
        }
    }
    if (i < nb) {
        *reinterpret_cast<float2*>(p.lo_o + ((size_t)bh * nb + i) * kHeadDim + c2) = make_float2(acc0, acc1);
        if (c2 == 0) p.lo_l[(size_t)bh * nb + i] = lsum;
    }
}

constexpr int kMergeRows = 4;  // block rows per workgroup, one wave each

template <int DT>
__global__ __launch_bounds__(64 * kMergeRows) void merge_kernel(Params p) {
    const int nb = p.nb;
    const int tiles = (nb + kMergeRows - 1) / kMergeRows;
    const int bh = blockIdx.x / tiles;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int i = (blockIdx.x - bh * tiles) * kMergeRows + wave;
    if (i >= nb) return;
    const int* ip = p.item_ptr + (size_t)bh * (nb + 1);
    const int first = max(ip[i], 0);
    const int nit = min(ip[i + 1] - first, p.max_items - first);
    if (nit <= 1) return;  // finished by the attention kernel
    const int b = bh / p.H;
    const int t = lane & 31;          // token within the block
    const int half = lane >> 5;       // channels half*32 .. half*32+31
    const bool valid = (p.mbits[(size_t)b * nb + i] >> t) & 1u;
    float M2 = -__builtin_inff();
    const size_t pbase = (size_t)bh * p.max_items + first;
    for (int c = 0; c < nit; c++) M2 = fmaxf(M2, p.part_ml[(pbase + c) * 64 + t]);
    float mi2 = -__builtin_inff();
    if (p.mode == 0) {
        mi2 = p.rowmax[(size_t)bh * nb + i] * kLog2e;
        M2 = fmaxf(M2, mi2);
    }
    float acc[32];
#pragma unroll
    for (int e = 0; e < 32; e++) acc[e] = 0.f;
    float den = 0.f;
    if (M2 != -__builtin_inff()) {
        for (int c = 0; c < nit; c++) {
            const float mc = p.part_ml[(pbase + c) * 64 + t];
            const float lc = p.part_ml[(pbase + c) * 64 + 32 + t];
            const float f = __builtin_amdgcn_exp2f(mc - M2);
            den += lc * f;
            const float4* po = reinterpret_cast<const float4*>(p.part_o + ((pbase + c) * kBlock + t) * kHeadDim + 32 * half);
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const float4 v = po[q];
                acc[4 * q] += v.x * f;
                acc[4 * q + 1] += v.y * f;
                acc[4 * q + 2] += v.z * f;
                acc[4 * q + 3] += v.w * f;
            }
        }
        if (p.mode == 0) {
            const float f = __builtin_amdgcn_exp2f(mi2 - M2);
            den += p.lo_l[(size_t)bh * nb + i] * f;
            const float4* lo = reinterpret_cast<const float4*>(p.lo_o + ((size_t)bh * nb + i) * kHeadDim + 32 * half);
#pragma unroll
            for (int q = 0; q < 8; q++) {
                const float4 v = lo[q];
                acc[4 * q] += v.x * f;
                acc[4 * q + 1] += v.y * f;
                acc[4 * q + 2] += v.z * f;
                acc[4 * q + 3] += v.w * f;
            }
        }
    }
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    const size_t orow = ((size_t)bh * p.N + (size_t)i * kBlock + t) * kHeadDim + 32 * half;
    if constexpr (DT == 1) {
        uint16_t* o = static_cast<uint16_t*>(p.out) + orow;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            uint4 pk;
            pk.x = (uint32_t)float_to_bf16(acc[8 * q] * inv) | ((uint32_t)float_to_bf16(acc[8 * q + 1] * inv) << 16);
            pk.y = (uint32_t)float_to_bf16(acc[8 * q + 2] * inv) | ((uint32_t)float_to_bf16(acc[8 * q + 3] * inv) << 16);
            pk.z = (uint32_t)float_to_bf16(acc[8 * q + 4] * inv) | ((uint32_t)float_to_bf16(acc[8 * q + 5] * inv) << 16);
            pk.w = (uint32_t)float_to_bf16(acc[8 * q + 6] * inv) | ((uint32_t)float_to_bf16(acc[8 * q + 7] * inv) << 16);
            reinterpret_cast<uint4*>(o)[q] = pk;
        }
    } else {
        float* o = static_cast<float*>(p.out) + orow;
#pragma unroll
        for (int q = 0; q < 8; q++)
            reinterpret_cast<float4*>(o)[q] =
                make_float4(acc[4 * q] * inv, acc[4 * q + 1] * inv, acc[4 * q + 2] * inv, acc[4 * q + 3] * inv);
    }
}

}  // namespace

hipError_t launch_lowres(const Params& p, hipStream_t s) {
    const int tiles = (p.nb + kLoRows - 1) / kLoRows;
    hipLaunchKernelGGL(lowres_kernel, dim3(p.BH * tiles), dim3(kLoThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_merge(const Params& p, hipStream_t s) {
    const int tiles = (p.nb + kMergeRows - 1) / kMergeRows;
    if (p.dtype == 1)
        hipLaunchKernelGGL(merge_kernel<1>, dim3(p.BH * tiles), dim3(64 * kMergeRows), 0, s, p);
    else
        hipLaunchKernelGGL(merge_kernel<0>, dim3(p.BH * tiles), dim3(64 * kMergeRows), 0, s, p);
    return hipGetLastError();
}

}  // namespace mra
