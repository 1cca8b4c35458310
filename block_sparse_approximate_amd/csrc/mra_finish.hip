// mra_finish.hip — step 4 ([MRA] "第四步"): the low-resolution attention on
// the unselected blocks (full mode) and the merge of high- and
// low-resolution results through a shared row maximum and normaliser.
//
// Low-resolution part of block row i of head bh:
//   W_ij = cnt_j * exp(S_ij - m_i)  for j not selected in row i, cnt_j > 0
//   lo_o = sum_j W_ij vhat_j,  lo_l = sum_j W_ij                    (fp32)
// m_i is the row max of the low-res logits, so every weight is <= cnt_j.
// Each pooled block stands for cnt_j keys, hence the cnt_j factor; with
// block-constant queries and keys this makes full mode equal dense attention.
//
// Merge, per query token t of row i, with high-res maxima kept in log2
// units and M the largest of the maxima involved:
//   out_t = (sum_c O_c 2^(m_c - M) + lo_o 2^(m_i log2e - M))
//         / (sum_c l_c 2^(m_c - M) + lo_l 2^(m_i log2e - M))
// where (O_c, m_c, l_c) are the high-res results of the row's segments; 0
// when the denominator is 0 or the token is padding.
//
// One launch, two kinds of workgroup:
//   * full mode only: a workgroup takes 8 block rows, computes their
//     low-res parts (walking the key blocks in tiles of 64 with the next
//     tile's loads in flight, so vhat is read once per 8 rows) and merges
//     them into the rows that one attention segment finished (their O/l is
//     already in `out`, their max and sum in the side buffer);
//   * a workgroup per row listed by the selector (no selected block, or
//     several segments): it computes that row's low-res part itself (full
//     mode) and joins the segments' partials.
// The two kinds touch disjoint rows.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kThreads = 256;
constexpr int kLoRows = 8;
constexpr int kLoTile = 64;
constexpr int kBatch = 8;   // segments whose loads are in flight together

// ------------------------------------------------------------ 8-row tiles
template <int DT>
__device__ void rows_tile(const Params& p, int bh, int row0) {
    __shared__ __align__(16) float vt[kLoTile][kHeadDim];
    __shared__ float wt[kLoRows][kLoTile];
    __shared__ __align__(16) float lo[kLoRows][kHeadDim];
    __shared__ float ll[kLoRows];
    const int nb = p.nb, words = p.words;
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const int r = tid >> 5;             // row of this thread in the multiply (0..7)
    const int c2 = (tid & 31) * 2;      // two channels
    const float* S = p.logits + (size_t)bh * nb * nb;
    const float* vh = p.vhat + (size_t)bh * nb * kHeadDim;
    const uint32_t* bits = p.selbits + (size_t)bh * nb * words;
    const int* cnt = p.cnt + (size_t)b * nb;

    // each thread weighs two cells of a tile: (wr, wj) and (wr + 4, wj)
    const int wj = tid & 63, wr = tid >> 6;
    float mrow[2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const int i = row0 + wr + 4 * e;
        mrow[e] = i < nb ? p.rowmax[(size_t)bh * nb + i] : 0.f;
    }
    float sv[2];
    uint32_t sb[2];
    int cv;
    float4 vv[4];
    auto fetch = [&](int j0) {
        const int j = j0 + wj;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int i = row0 + wr + 4 * e;
            const bool ok = i < nb && j < nb;
            sv[e] = ok ? S[(size_t)i * nb + j] : 0.f;
            sb[e] = ok ? bits[(size_t)i * words + (j >> 5)] : 0xFFFFFFFFu;
        }
        cv = j < nb ? cnt[j] : 0;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int x = tid + e * kThreads;    // float4 index in the tile
            const int jj = x >> 4, c4 = (x & 15) * 4;
            vv[e] = (j0 + jj < nb) ? *reinterpret_cast<const float4*>(vh + (size_t)(j0 + jj) * kHeadDim + c4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    fetch(0);
    float acc0 = 0.f, acc1 = 0.f, lsum = 0.f;
    for (int j0 = 0; j0 < nb; j0 += kLoTile) {
        __syncthreads();
        const int j = j0 + wj;
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const bool sel = (sb[e] >> (j & 31)) & 1u;
            wt[wr + 4 * e][wj] = (!sel && cv > 0) ? (float)cv * __builtin_amdgcn_exp2f((sv[e] - mrow[e]) * kLog2e)
                                                  : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int x = tid + e * kThreads;
            *reinterpret_cast<float4*>(&vt[x >> 4][(x & 15) * 4]) = vv[e];
        }
        __syncthreads();
        if (j0 + kLoTile < nb) fetch(j0 + kLoTile);   // in flight during the multiply
#pragma unroll 8
        for (int jj = 0; jj < kLoTile; jj++) {
            const float w = wt[r][jj];
            const float2 v = *reinterpret_cast<const float2*>(&vt[jj][c2]);
            acc0 = __builtin_fmaf(w, v.x, acc0);
            acc1 = __builtin_fmaf(w, v.y, acc1);
            lsum += w;
        }
    }
    lo[r][c2] = acc0;
    lo[r][c2 + 1] = acc1;
    if (c2 == 0) ll[r] = lsum;
    __syncthreads();

    // merge into the rows one segment finished: thread = (row, token)
    const int t = tid & 31;
    const int i = row0 + r;
    if (i >= nb) return;
    const int* ip = p.item_ptr + (size_t)bh * (nb + 1);
    if (ip[i + 1] - ip[i] != 1) return;   // joined by a per-row workgroup
    const bool valid = (p.mbits[(size_t)b * nb + i] >> t) & 1u;
    const size_t tok = (size_t)bh * p.N + (size_t)i * kBlock + t;
    const float2 ml = *reinterpret_cast<const float2*>(p.side_ml + tok * 2);
    const float mi2 = p.rowmax[(size_t)bh * nb + i] * kLog2e;
    const float M2 = fmaxf(ml.x, mi2);
    float a = 0.f, bw = 0.f;
    if (M2 != -__builtin_inff()) {
        a = __builtin_amdgcn_exp2f(ml.x - M2) * ml.y;   // O/l was stored: scale back by l
        bw = __builtin_amdgcn_exp2f(mi2 - M2);
    }
    const float den = (M2 != -__builtin_inff() ? __builtin_amdgcn_exp2f(ml.x - M2) : 0.f) * ml.y + ll[r] * bw;
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    if constexpr (DT == 1) {
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + tok * kHeadDim);
        uint4 in[8];
#pragma unroll
        for (int q = 0; q < 8; q++) in[q] = o[q];
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const uint32_t w4[4] = {in[q].x, in[q].y, in[q].z, in[q].w};
            uint32_t res[4];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int c = 8 * q + 2 * e;
                const float x0 = __uint_as_float(w4[e] << 16), x1 = __uint_as_float(w4[e] & 0xFFFF0000u);
                const float y0 = (x0 * a + lo[r][c] * bw) * inv, y1 = (x1 * a + lo[r][c + 1] * bw) * inv;
                res[e] = (uint32_t)float_to_bf16(y0) | ((uint32_t)float_to_bf16(y1) << 16);
            }
            o[q] = make_uint4(res[0], res[1], res[2], res[3]);
        }
    } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + tok * kHeadDim);
        float4 in[16];
#pragma unroll
        for (int q = 0; q < 16; q++) in[q] = o[q];
#pragma unroll
        for (int q = 0; q < 16; q++) {
            const int c = 4 * q;
            o[q] = make_float4((in[q].x * a + lo[r][c] * bw) * inv, (in[q].y * a + lo[r][c + 1] * bw) * inv,
                               (in[q].z * a + lo[r][c + 2] * bw) * inv, (in[q].w * a + lo[r][c + 3] * bw) * inv);
        }
    }
}

// ------------------------------------------------------------ listed rows
template <int DT>
__device__ void merge_row(const Params& p, int bh, int i) {
    __shared__ float wl[512];
    __shared__ float red[4][kHeadDim + 1];
    __shared__ __align__(16) float lo[kHeadDim];
    __shared__ float ll;
    const int nb = p.nb;
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    float mi2 = -__builtin_inff();
    if (p.mode == 0) {
        // the row's low-res part, computed here
        const float* S = p.logits + ((size_t)bh * nb + i) * nb;
        const uint32_t* bits = p.selbits + ((size_t)bh * nb + i) * p.words;
        const int* cnt = p.cnt + (size_t)b * nb;
        const float m = p.rowmax[(size_t)bh * nb + i];
        mi2 = m * kLog2e;
        for (int j = tid; j < nb; j += kThreads) {
            const bool sel = (bits[j >> 5] >> (j & 31)) & 1u;
            const int cj = cnt[j];
            wl[j] = (!sel && cj > 0) ? (float)cj * __builtin_amdgcn_exp2f((S[j] - m) * kLog2e) : 0.f;
        }
        __syncthreads();
        const int c = tid & 63, g = tid >> 6;
        const float* vh = p.vhat + (size_t)bh * nb * kHeadDim;
        float acc = 0.f;
        for (int j = g; j < nb; j += 4) acc = __builtin_fmaf(wl[j], vh[(size_t)j * kHeadDim + c], acc);
        red[g][c] = acc;
        __syncthreads();
        if (tid < kHeadDim) lo[tid] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
        if (tid == 0) {
            float s = 0.f;
            for (int j = 0; j < nb; j++) s += wl[j];
            ll = s;
        }
        __syncthreads();
    }

    const int* ip = p.item_ptr + (size_t)bh * (nb + 1);
    const int first = max(ip[i], 0);
    const int nit = max(0, min(ip[i + 1] - first, p.max_items - first));
    const int t = tid >> 3;              // token within the block
    const int cg = (tid & 7) * 8;        // channels cg .. cg+7
    const bool valid = (p.mbits[(size_t)b * nb + i] >> t) & 1u;
    const size_t pbase = (size_t)bh * p.max_items + first;

    float M2 = mi2;
    for (int c0 = 0; c0 < nit; c0 += kBatch) {
        float mc[kBatch];
#pragma unroll
        for (int c = 0; c < kBatch; c++) mc[c] = c0 + c < nit ? p.part_ml[(pbase + c0 + c) * 64 + t] : -__builtin_inff();
#pragma unroll
        for (int c = 0; c < kBatch; c++) M2 = fmaxf(M2, mc[c]);
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) acc[e] = 0.f;
    float den = 0.f;
    if (M2 != -__builtin_inff()) {
        for (int c0 = 0; c0 < nit; c0 += kBatch) {
            float mc[kBatch], lc[kBatch];
            float4 oa[kBatch], ob[kBatch];
#pragma unroll
            for (int c = 0; c < kBatch; c++) {
                const bool ok = c0 + c < nit;
                const size_t it = pbase + c0 + c;
                mc[c] = ok ? p.part_ml[it * 64 + t] : -__builtin_inff();
                lc[c] = ok ? p.part_ml[it * 64 + 32 + t] : 0.f;
                const float4* po = reinterpret_cast<const float4*>(p.part_o + (it * kBlock + t) * kHeadDim + cg);
                oa[c] = ok ? po[0] : make_float4(0.f, 0.f, 0.f, 0.f);
                ob[c] = ok ? po[1] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int c = 0; c < kBatch; c++) {
                const float f = __builtin_amdgcn_exp2f(mc[c] - M2);
                den += lc[c] * f;
                acc[0] += oa[c].x * f; acc[1] += oa[c].y * f; acc[2] += oa[c].z * f; acc[3] += oa[c].w * f;
                acc[4] += ob[c].x * f; acc[5] += ob[c].y * f; acc[6] += ob[c].z * f; acc[7] += ob[c].w * f;
            }
        }
        if (p.mode == 0) {
            const float f = __builtin_amdgcn_exp2f(mi2 - M2);
            den += ll * f;
#pragma unroll
            for (int e = 0; e < 8; e++) acc[e] += lo[cg + e] * f;
        }
    }
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    const size_t orow = ((size_t)bh * p.N + (size_t)i * kBlock + t) * kHeadDim + cg;
    if constexpr (DT == 1) {
        uint4 pk;
        pk.x = (uint32_t)float_to_bf16(acc[0] * inv) | ((uint32_t)float_to_bf16(acc[1] * inv) << 16);
        pk.y = (uint32_t)float_to_bf16(acc[2] * inv) | ((uint32_t)float_to_bf16(acc[3] * inv) << 16);
        pk.z = (uint32_t)float_to_bf16(acc[4] * inv) | ((uint32_t)float_to_bf16(acc[5] * inv) << 16);
        pk.w = (uint32_t)float_to_bf16(acc[6] * inv) | ((uint32_t)float_to_bf16(acc[7] * inv) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow) = pk;
    } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow);
        o[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
        o[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void finish_kernel(Params p, int tiles) {
    const int nb = p.nb;
    const int per_head = (nb + kLoRows - 1) / kLoRows;
    if ((int)blockIdx.x < tiles) {
        const int bh = blockIdx.x / per_head;
        rows_tile<DT>(p, bh, (blockIdx.x - bh * per_head) * kLoRows);
        return;
    }
    const int g = blockIdx.x - tiles;
    const int bh = g / nb, s = g - bh * nb;
    if (s >= p.n_merge[bh]) return;
    const int i = min(max(p.merge_rows[(size_t)bh * nb + s], 0), nb - 1);
    merge_row<DT>(p, bh, i);
}

}  // namespace

hipError_t launch_finish(const Params& p, hipStream_t s) {
    const int tiles = p.mode == 0 ? p.BH * ((p.nb + kLoRows - 1) / kLoRows) : 0;
    const int grid = tiles + p.BH * p.nb;
    if (p.dtype == 1)
        hipLaunchKernelGGL(finish_kernel<1>, dim3(grid), dim3(kThreads), 0, s, p, tiles);
    else
        hipLaunchKernelGGL(finish_kernel<0>, dim3(grid), dim3(kThreads), 0, s, p, tiles);
    return hipGetLastError();
}

}  // namespace mra
