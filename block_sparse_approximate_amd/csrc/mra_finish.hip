// mra_finish.hip — step 4 ([MRA] "第四步") for the block rows the attention
// kernel cannot finish alone: rows with no selected block, and rows whose
// selection was cut into several segments.  (A row that is one segment is
// finished, low-res merge included, by the attention kernel.)
//
// For a listed block row i of head bh (its descriptor: row, first segment,
// number of segments):
//   * full mode: the row's low-resolution part without its selected blocks,
//       lo = lo_all_i - sum_{j in sel(i)} w_ij vhat_j,
//       ll = ll_all_i - sum_{j in sel(i)} w_ij,
//     where lo_all, ll_all (every key block) come from the low-res sums and
//     the two sums over sel(i) from the segments' partials;
//   * the join, per query token t, with high-res maxima in log2 units and M
//     the largest of the maxima involved:
//       out_t = (sum_c O_c 2^(m_c - M) + lo 2^(m_i log2e - M))
//             / (sum_c l_c 2^(m_c - M) + ll 2^(m_i log2e - M))
//     over the row's segments c (O_c, m_c, l_c from the attention kernel);
//     the low-res terms only in full mode; 0 when the denominator is 0 or
//     the token is padding.
// A workgroup of 256 threads takes listed rows of one head in turn.
#include "mra_common.h"

namespace mra {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;       // segments whose loads are in flight together
// Workgroups per head: about kGridTarget in all (many small heads share few
// rows to join each; a few long heads can have hundreds), 4 to 32 per head,
// and never more than the head's block rows.
constexpr int kGridTarget = 512;
__host__ __device__ inline int row_slots(int nb, int BH) {
    int s = kGridTarget / BH;
    s = s < 4 ? 4 : (s > 32 ? 32 : s);
    return nb < s ? nb : s;
}

// One listed row, from its descriptor (row i, first segment, segments).
// Every load the row needs is issued before the first wait; the segments are
// joined in one pass with a running maximum.
template <int DT, int HD>
__device__ void merge_row(const Params& p, int bh, int4 dsc, float* lo, float* ll_s) {
    constexpr int kCh = HD / 8;          // channels per thread
    constexpr int kF4 = kCh / 4;
    const int nb = p.nb;
    const int b = bh / p.H;
    const int tid = threadIdx.x;
    const int i = min(max(dsc.x, 0), nb - 1);
    const int first = max(dsc.y, 0);
    const int nit = max(0, min(dsc.z, p.max_items - first));
    const size_t pbase = (size_t)bh * p.max_items + first;
    const size_t row = (size_t)bh * nb + i;
    const bool full = p.mode == 0;
    const int t = tid >> 3;              // token within the block
    const int cg = (tid & 7) * kCh;      // channels cg .. cg + kCh - 1
    const uint32_t qm = p.mbits[(size_t)b * nb + i];
    float lo_in = 0.f, mrow = 0.f;
    if (full) {
        if (tid <= HD) lo_in = tid < HD ? p.lo_all[row * HD + tid] : p.ll_all[row];
        mrow = p.rowmax[row];
    }

    // high-res segments: running max M (log2 units), numerator acc, denominator den
    float M = -__builtin_inff(), den = 0.f, corr = 0.f;
    float acc[kCh];
#pragma unroll
    for (int e = 0; e < kCh; e++) acc[e] = 0.f;
    for (int c0 = 0; c0 < nit; c0 += kBatch) {
        float mc[kBatch], lc[kBatch], cc[kBatch];
        float4 oa[kBatch][kF4];
#pragma unroll
        for (int c = 0; c < kBatch; c++) {
            const bool ok = c0 + c < nit;
            const size_t it = pbase + (ok ? c0 + c : 0);
            mc[c] = ok ? p.part_ml[it * 64 + t] : -__builtin_inff();
            lc[c] = ok ? p.part_ml[it * 64 + 32 + t] : 0.f;
            cc[c] = (ok && full && tid <= HD) ? p.part_corr[it * corr_stride(HD) + tid] : 0.f;
            const float4* po = reinterpret_cast<const float4*>(p.part_o + (it * kBlock + t) * HD + cg);
#pragma unroll
            for (int x = 0; x < kF4; x++) oa[c][x] = ok ? po[x] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float Mb = M;
#pragma unroll
        for (int c = 0; c < kBatch; c++) Mb = fmaxf(Mb, mc[c]);
        if (Mb != -__builtin_inff()) {
            const float s = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
            den *= s;
#pragma unroll
            for (int e = 0; e < kCh; e++) acc[e] *= s;
#pragma unroll
            for (int c = 0; c < kBatch; c++) {
                const float f = mc[c] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mc[c] - Mb);
                den += lc[c] * f;
#pragma unroll
                for (int x = 0; x < kF4; x++) {
                    acc[4 * x] += oa[c][x].x * f;
                    acc[4 * x + 1] += oa[c][x].y * f;
                    acc[4 * x + 2] += oa[c][x].z * f;
                    acc[4 * x + 3] += oa[c][x].w * f;
                }
            }
            M = Mb;
        }
#pragma unroll
        for (int c = 0; c < kBatch; c++) corr += cc[c];
    }
    float Mu = M;   // the max that den and the probabilities are relative to
    if (full) {
        // the row's low-res part: lo_all minus the segments' corrections
        if (tid < HD) lo[tid] = lo_in - corr;
        else if (tid == HD) *ll_s = fmaxf(lo_in - corr, 0.f);
        __syncthreads();
        const float ll = *ll_s, mi2 = mrow * kLog2e;
        const float Mf = fmaxf(M, mi2);
        if (Mf != -__builtin_inff()) {
            const float s = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
            const float f = __builtin_amdgcn_exp2f(mi2 - Mf);
            den = den * s + ll * f;
            Mu = Mf;
#pragma unroll
            for (int e = 0; e < kCh; e++) acc[e] = acc[e] * s + lo[cg + e] * f;
        }
    }
    const bool valid = (qm >> t) & 1u;
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    const size_t orow = ((size_t)bh * p.N + (size_t)i * kBlock + t) * HD + cg;
    if ((tid & 7) == 0 && p.save_stats) {   // the token's softmax statistics, for the backward pass
        const size_t st = (size_t)bh * p.N + (size_t)i * kBlock + t;
        p.st_m[st] = Mu == -__builtin_inff() ? 0.f : Mu;
        p.st_linv[st] = inv;
    }
    if constexpr (DT == 1) {
#pragma unroll
        for (int x = 0; x < kCh / 8; x++) {
            const float* a = acc + 8 * x;
            uint4 pk;
            pk.x = (uint32_t)float_to_bf16(a[0] * inv) | ((uint32_t)float_to_bf16(a[1] * inv) << 16);
            pk.y = (uint32_t)float_to_bf16(a[2] * inv) | ((uint32_t)float_to_bf16(a[3] * inv) << 16);
            pk.z = (uint32_t)float_to_bf16(a[4] * inv) | ((uint32_t)float_to_bf16(a[5] * inv) << 16);
            pk.w = (uint32_t)float_to_bf16(a[6] * inv) | ((uint32_t)float_to_bf16(a[7] * inv) << 16);
            reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow)[x] = pk;
        }
    } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow);
#pragma unroll
        for (int x = 0; x < kF4; x++)
            o[x] = make_float4(acc[4 * x] * inv, acc[4 * x + 1] * inv, acc[4 * x + 2] * inv, acc[4 * x + 3] * inv);
    }
}

template <int DT, int HD>
__global__ __launch_bounds__(kThreads) void finish_kernel(Params p) {
    __shared__ __align__(16) float lo[HD];
    __shared__ float ll;
    const int nb = p.nb;
    const int slots = row_slots(nb, p.BH);
    const int bh = blockIdx.x / slots, slot = blockIdx.x - bh * slots;
    // the descriptor of this workgroup's first row is loaded with the count
    int4 dsc = slot < nb ? p.merge_rows[(size_t)bh * nb + slot] : make_int4(0, 0, 0, 0);
    const int nm = min(p.n_merge[bh], nb);
    for (int s = slot; s < nm; s += slots) {
        if (s != slot) dsc = p.merge_rows[(size_t)bh * nb + s];
        merge_row<DT, HD>(p, bh, dsc, lo, &ll);
        __syncthreads();   // lo and ll are reused by the next row
    }
}

}  // namespace

template <int HD>
static hipError_t launch_finish_t(const Params& p, hipStream_t s) {
    const int grid = p.BH * row_slots(p.nb, p.BH);
    if (p.dtype == 1)
        hipLaunchKernelGGL((finish_kernel<1, HD>), dim3(grid), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((finish_kernel<0, HD>), dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_finish(const Params& p, hipStream_t s) {
    if (p.d == 64) return launch_finish_t<64>(p, s);
    if (p.d == 128) return launch_finish_t<128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mra
