// mra_attn.hip — step 3 ([MRA] "第三步"): exact softmax attention on the
// selected 32x32 blocks, i.e. what the pages' sampled dense matmul, row max,
// sparse-dense matmul and reduce-sum do, in one pass with an online row max.
//
// Work item = (head, query block row i, chunk of at most kChunk selected key
// blocks); one wave64 per item.  Per key block j of the chunk:
//   S^T = K_j Q_i^T           4 x MFMA 32x32x16 bf16 (fp32: 32 x 32x32x2 f32)
//   online max / exp2 / sum   in registers: lane l holds query l%32 and 16 of
//                             its 32 keys, so row reductions need one swap
//                             with lane l^32
//   O^T += V_j^T P^T          V_j staged through LDS and read back transposed
//                             with ds_read_b64_tr_b16; P goes straight from
//                             the S^T accumulators into the B operand
// Computing S^T rather than S is what lets P stay in registers: the MFMA
// accumulator layout of S^T is the B-operand layout of P^T up to a fixed
// permutation of the key index, which V's LDS reads apply.
//
// A block row whose selection fits in one item is finished here: sparse
// mode writes O / l; full mode merges with the low-resolution part of the
// row ([MRA] "第四步") through the shared row maximum.  Longer rows write
// un-normalised partials (O, running max, sum) that the merge kernel joins.
//
// Workgroups are placed XCD-aware: workgroup g runs on XCD g % 8, and all
// items of head bh go to XCD bh % 8, so a head's K/V re-reads stay in one L2.
#include "mra_common.h"

namespace mra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kVStrideB = 80;   // bf16 elements per staged V row (64 + 16 pad: no bank conflicts)
constexpr int kVStrideF = 68;   // fp32 elements per staged V row

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// key index held by accumulator register r of a 32x32 MFMA tile in lane l
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

template <int DT>
struct Stage;

template <>
struct Stage<1> {  // bf16
    uint16_t v[32 * kVStrideB];
};
template <>
struct Stage<0> {  // fp32
    float v[32 * kVStrideF];
};

template <int DT>
__global__ __launch_bounds__(kThreads) void attn_kernel(Params p, int wg_per_head) {
    __shared__ __align__(16) Stage<DT> stage[kWaves];
    const int g = blockIdx.x;
    const int xcd = g & 7;
    const int slot = g >> 3;
    const int hm = slot / wg_per_head;
    const int w = slot - hm * wg_per_head;
    const int bh = xcd + 8 * hm;
    if (bh >= p.BH) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int item = w * kWaves + wave;
    if (item >= min(p.n_items[bh], p.max_items)) return;

    const int nb = p.nb;
    const int2 it = p.items[(size_t)bh * p.max_items + item];
    // indices read from memory are clamped so that no logic slip can address
    // outside the tensors
    const int i = min(max(it.x, 0), nb - 1), chunk = max(it.y, 0);
    const int* rp = p.row_ptr + (size_t)bh * (nb + 1);
    const int cbeg = rp[i] + chunk * kChunk;
    const int nblk = max(0, min(min(kChunk, rp[i + 1] - cbeg), (int)p.K - cbeg));
    const int* ip = p.item_ptr + (size_t)bh * (nb + 1);
    const bool single = (ip[i + 1] - ip[i]) == 1;
    const int b = bh / p.H;
    const int jcol = lane < nblk ? min(max(p.col[(size_t)bh * p.K + cbeg + lane], 0), nb - 1) : 0;
    const uint32_t* mb = p.mbits + (size_t)b * nb;
    const float scale2 = (1.0f / __builtin_sqrtf((float)p.d)) * kLog2e;
    const int n = lane & 31, h = lane >> 5;

    f32x16 o0, o1;
#pragma unroll
    for (int r = 0; r < 16; r++) { o0[r] = 0.f; o1[r] = 0.f; }
    float mrun = -__builtin_inff(), lsum = 0.f;

    const size_t head_off = (size_t)bh * p.N * kHeadDim;
    if constexpr (DT == 1) {
        const uint16_t* Qg = static_cast<const uint16_t*>(p.q) + head_off + (size_t)i * kBlock * kHeadDim;
        const uint16_t* Kg = static_cast<const uint16_t*>(p.k) + head_off;
        const uint16_t* Vg = static_cast<const uint16_t*>(p.v) + head_off;
        uint16_t* vs = stage[wave].v;
        bf16x8 qb[4];
#pragma unroll
        for (int kc = 0; kc < 4; kc++)
            qb[kc] = as_bf16x8(*reinterpret_cast<const uint4*>(Qg + n * kHeadDim + 16 * kc + 8 * h));
        // V tile loads: lane covers rows lane/8 + 8e, 16 bytes at column (lane%8)*8
        const int vrow = lane >> 3, vcol = (lane & 7) * 8;
        uint4 kn[4], vn[4];
        if (nblk > 0) {
            const int j = __shfl(jcol, 0, 64);
            const uint16_t* Kb = Kg + (size_t)j * kBlock * kHeadDim;
            const uint16_t* Vb = Vg + (size_t)j * kBlock * kHeadDim;
#pragma unroll
            for (int kc = 0; kc < 4; kc++) kn[kc] = *reinterpret_cast<const uint4*>(Kb + n * kHeadDim + 16 * kc + 8 * h);
#pragma unroll
            for (int e = 0; e < 4; e++) vn[e] = *reinterpret_cast<const uint4*>(Vb + (vrow + 8 * e) * kHeadDim + vcol);
        }
        for (int t = 0; t < nblk; t++) {
            const int j = __shfl(jcol, t, 64);
            uint4 kc_[4], vc_[4];
#pragma unroll
            for (int e = 0; e < 4; e++) { kc_[e] = kn[e]; vc_[e] = vn[e]; }
            if (t + 1 < nblk) {  // prefetch the next block while this one computes
                const int jn = __shfl(jcol, t + 1, 64);
                const uint16_t* Kb = Kg + (size_t)jn * kBlock * kHeadDim;
                const uint16_t* Vb = Vg + (size_t)jn * kBlock * kHeadDim;
#pragma unroll
                for (int kc = 0; kc < 4; kc++) kn[kc] = *reinterpret_cast<const uint4*>(Kb + n * kHeadDim + 16 * kc + 8 * h);
#pragma unroll
                for (int e = 0; e < 4; e++) vn[e] = *reinterpret_cast<const uint4*>(Vb + (vrow + 8 * e) * kHeadDim + vcol);
            }
            // S^T = K_j Q_i^T
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; r++) s[r] = 0.f;
#pragma unroll
            for (int kc = 0; kc < 4; kc++)
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kc_[kc]), qb[kc], s, 0, 0, 0);
            // stage V_j in LDS (this wave's region only)
#pragma unroll
            for (int e = 0; e < 4; e++) *reinterpret_cast<uint4*>(vs + (vrow + 8 * e) * kVStrideB + vcol) = vc_[e];
            // online softmax in log2 units
            const uint32_t kb = mb[j];
            float bm = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float x = ((kb >> acc_row(r, lane)) & 1u) ? s[r] * scale2 : -__builtin_inff();
                s[r] = x;
                bm = fmaxf(bm, x);
            }
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mnew = fmaxf(mrun, bm);
            const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
            const float alpha = fast_exp2(mrun - muse);
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                s[r] = fast_exp2(s[r] - muse);
                ps += s[r];
            }
            lsum = lsum * alpha + ps;
            mrun = mnew;
#pragma unroll
            for (int r = 0; r < 16; r++) { o0[r] *= alpha; o1[r] *= alpha; }
            bf16x8 pb[2];
#pragma unroll
            for (int kc2 = 0; kc2 < 2; kc2++)
#pragma unroll
                for (int e = 0; e < 8; e++) pb[kc2][e] = static_cast<__bf16>(s[8 * kc2 + e]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // O^T += V_j^T P^T ; A operand read transposed from LDS
            const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
            for (int kc2 = 0; kc2 < 2; kc2++) {
#pragma unroll
                for (int mt = 0; mt < 2; mt++) {
                    const int col = 32 * mt + 16 * (g16 & 1) + 4 * (s16 & 3);
                    const int row = 16 * kc2 + 4 * h + (s16 >> 2);
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vs + row * kVStrideB + col));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_i16x4*)(vs + (row + 8) * kVStrideB + col));
                    const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                                          hi[0], hi[1], hi[2], hi[3]};
                    const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
                    if (mt == 0) o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], o0, 0, 0, 0);
                    else o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc2], o1, 0, 0, 0);
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    } else {
        const float* Qg = static_cast<const float*>(p.q) + head_off + (size_t)i * kBlock * kHeadDim;
        const float* Kg = static_cast<const float*>(p.k) + head_off;
        const float* Vg = static_cast<const float*>(p.v) + head_off;
        float* vs = stage[wave].v;
        float qf[32];
#pragma unroll
        for (int c4 = 0; c4 < 8; c4++) {
            const float4 x = *reinterpret_cast<const float4*>(Qg + n * kHeadDim + 32 * h + 4 * c4);
            qf[4 * c4] = x.x; qf[4 * c4 + 1] = x.y; qf[4 * c4 + 2] = x.z; qf[4 * c4 + 3] = x.w;
        }
        const int vrow = lane >> 4, vcol = (lane & 15) * 4;
        for (int t = 0; t < nblk; t++) {
            const int j = __shfl(jcol, t, 64);
            const float* Kb = Kg + (size_t)j * kBlock * kHeadDim;
            const float* Vb = Vg + (size_t)j * kBlock * kHeadDim;
            float kf[32];
#pragma unroll
            for (int c4 = 0; c4 < 8; c4++) {
                const float4 x = *reinterpret_cast<const float4*>(Kb + n * kHeadDim + 32 * h + 4 * c4);
                kf[4 * c4] = x.x; kf[4 * c4 + 1] = x.y; kf[4 * c4 + 2] = x.z; kf[4 * c4 + 3] = x.w;
            }
            float4 vv[8];
#pragma unroll
            for (int e = 0; e < 8; e++) vv[e] = *reinterpret_cast<const float4*>(Vb + (vrow + 4 * e) * kHeadDim + vcol);
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; r++) s[r] = 0.f;
#pragma unroll
            for (int kc = 0; kc < 32; kc++) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[kc], qf[kc], s, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 8; e++) *reinterpret_cast<float4*>(vs + (vrow + 4 * e) * kVStrideF + vcol) = vv[e];
            const uint32_t kb = mb[j];
            float bm = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float x = ((kb >> acc_row(r, lane)) & 1u) ? s[r] * scale2 : -__builtin_inff();
                s[r] = x;
                bm = fmaxf(bm, x);
            }
            bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
            const float mnew = fmaxf(mrun, bm);
            const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
            const float alpha = fast_exp2(mrun - muse);
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                s[r] = fast_exp2(s[r] - muse);
                ps += s[r];
            }
            lsum = lsum * alpha + ps;
            mrun = mnew;
#pragma unroll
            for (int r = 0; r < 16; r++) { o0[r] *= alpha; o1[r] *= alpha; }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int kc = 0; kc < 16; kc++) {
                const int key = (kc >> 2) * 8 + 4 * h + (kc & 3);
                o0 = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * kVStrideF + n], s[kc], o0, 0, 0, 0);
                o1 = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * kVStrideF + 32 + n], s[kc], o1, 0, 0, 0);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }

    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    const int tok = i * kBlock + n;
    if (single) {
        // finish the row: sparse O/l, or full-mode merge with the low-res part
        const bool valid = (mb[i] >> n) & 1u;
        float a = 0.f, bw = 0.f, den = 0.f;
        const float* lo = nullptr;
        if (p.mode == 0) {
            const float mi2 = p.rowmax[(size_t)bh * nb + i] * kLog2e;
            const float M2 = fmaxf(mrun, mi2);
            if (M2 != -__builtin_inff()) {
                a = fast_exp2(mrun - M2);
                bw = fast_exp2(mi2 - M2);
            }
            const float ll = p.lo_l[(size_t)bh * nb + i];
            den = ltot * a + ll * bw;
            lo = p.lo_o + ((size_t)bh * nb + i) * kHeadDim;
        } else {
            a = 1.f;
            den = ltot;
        }
        const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
        const size_t orow = ((size_t)bh * p.N + tok) * kHeadDim;
#pragma unroll
        for (int mt = 0; mt < 2; mt++) {
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int d0 = 32 * mt + 8 * gq + 4 * h;
                float vals[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float ov = mt == 0 ? o0[4 * gq + e] : o1[4 * gq + e];
                    float num = ov * a;
                    if (p.mode == 0) num += lo[d0 + e] * bw;
                    vals[e] = num * inv;
                }
                if constexpr (DT == 1) {
                    uint2 pk;
                    pk.x = (uint32_t)float_to_bf16(vals[0]) | ((uint32_t)float_to_bf16(vals[1]) << 16);
                    pk.y = (uint32_t)float_to_bf16(vals[2]) | ((uint32_t)float_to_bf16(vals[3]) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + d0) = pk;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + d0) =
                        make_float4(vals[0], vals[1], vals[2], vals[3]);
                }
            }
        }
    } else {
        const size_t pidx = (size_t)bh * p.max_items + item;
        float* po = p.part_o + (pidx * kBlock + n) * kHeadDim;
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int d0 = 32 * mt + 8 * gq + 4 * h;
                const f32x16& oo = mt == 0 ? o0 : o1;
                *reinterpret_cast<float4*>(po + d0) =
                    make_float4(oo[4 * gq], oo[4 * gq + 1], oo[4 * gq + 2], oo[4 * gq + 3]);
            }
        if (h == 0) {
            p.part_ml[pidx * 64 + n] = mrun;
            p.part_ml[pidx * 64 + 32 + n] = ltot;
        }
    }
}

}  // namespace

hipError_t launch_attn(const Params& p, hipStream_t s) {
    const int wg_per_head = (p.max_items + kWaves - 1) / kWaves;
    const int head_slots = (p.BH + 7) / 8;
    const int grid = 8 * head_slots * wg_per_head;
    if (p.dtype == 1)
        hipLaunchKernelGGL(attn_kernel<1>, dim3(grid), dim3(kThreads), 0, s, p, wg_per_head);
    else
        hipLaunchKernelGGL(attn_kernel<0>, dim3(grid), dim3(kThreads), 0, s, p, wg_per_head);
    return hipGetLastError();
}

}  // namespace mra
