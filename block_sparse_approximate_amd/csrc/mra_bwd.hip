// mra_bwd.hip — gradients of the sparse-mode forward with respect to q, k
// and v ([MRA] "第三步": the block products are autograd functions whose
// backward reuses the same kernels on transposed block indices, so the
// selection of step 2 is a constant of the backward pass; in sparse mode the
// output is the high-resolution part alone, [MRA] "第四步").
//
// With the selection fixed, a valid query token t of block row i attends to
// the valid keys u of its selected blocks:
//   s_u = tau q_t . k_u,  P_u = 2^(s_u log2e - m_t) / l_t,  O_t = sum_u P_u v_u
// and for dO = dL/dO, D_t = dO_t . O_t:
//   dS_u = P_u (dO_t . v_u - D_t),  dq_t = tau sum_u dS_u k_u,
//   dk_u = tau sum_t dS_u q_t,      dv_u = sum_t P_u dO_t.
//
// Three kernels, in stream order after a forward call that left its
// selection in the workspace:
//   transpose_kernel  per head: the query-block rows that selected each key
//                     block (column lists of the selection bitmap, ascending)
//   dq_kernel         one wave per query block row i: pass 1 the row's max
//                     m_t and sum l_t (stored, with D_t, for dkv_kernel);
//                     pass 2 per selected block j:
//                       S^T = K_j Q_i^T, dP^T = V_j dO_i^T   (lane = query)
//                       dS^T = P^T (dP^T - D),  dQ^T += K_j^T dS^T
//   dkv_kernel        one wave per key block column j, over the rows i that
//                     selected it:
//                       S = Q_i K_j^T, dP = dO_i V_j^T       (lane = key)
//                       dV^T += dO_i^T P,  dK^T += Q_i^T dS
// Blocks are staged in the wave's LDS as 32 token rows; MFMA operands are
// read one row per lane, and a transposed operand (X^T with the contraction
// over the block's rows) with ds_read_b64_tr_b16 in the order of an
// accumulator's registers, so an accumulator (P, dS) feeds the next product
// straight from registers.  bf16 operands, fp32 accumulation.
#include "mra_common.h"

namespace mra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 2;             // per workgroup: 4 staged blocks per wave fit static LDS
constexpr int kThreads = kWaves * 64;
constexpr int kStr = 72;              // bf16 elements per staged token row (144 bytes)
constexpr int kTile = kBlock * kStr;  // one staged block
constexpr int kTrThreads = 512;       // transpose_kernel: one thread per key block (nb <= 512)

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// row index (within the 32 x 32 tile) held by accumulator register r in lane l
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A 32 x 64 bf16 block (row-major in memory) into the wave's LDS: lane l
// moves 16 bytes of token rows l / 8 + 8 x, channels 8 (l % 8) .. +7
// (whole 128-byte rows per 8 lanes).
__device__ __forceinline__ void stage(uint16_t* s, const uint16_t* g, int lane) {
    u32x4 r[4];
#pragma unroll
    for (int x = 0; x < 4; x++) r[x] = *reinterpret_cast<const u32x4*>(g + ((lane >> 3) + 8 * x) * kHeadDim + (lane & 7) * 8);
#pragma unroll
    for (int x = 0; x < 4; x++) *reinterpret_cast<u32x4*>(s + ((lane >> 3) + 8 * x) * kStr + (lane & 7) * 8) = r[x];
}

// MFMA operand piece kc of a staged block: row l % 32, channels 16 kc + 8 (l / 32) .. +7
__device__ __forceinline__ bf16x8 op(const uint16_t* s, int lane, int kc) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(s + (lane & 31) * kStr + 16 * kc + 8 * (lane >> 5)));
}

// A operand of X^T for rows (channels) 32 mt .. 32 mt + 31, contracting over
// the staged block's rows in the order that accumulator registers
// 8 kc2 .. 8 kc2 + 7 of lane l hold them (acc_row).
__device__ __forceinline__ bf16x8 op_t(const uint16_t* s, int lane, int kc2, int mt) {
    const int g16 = lane >> 4, s16 = lane & 15, h = lane >> 5;
    const int col = 32 * mt + 16 * (g16 & 1) + 4 * (s16 & 3);
    const int row = 16 * kc2 + 4 * h + (s16 >> 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + row * kStr + col));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + (row + 8) * kStr + col));
    const i16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, a8);
}

// accumulator registers 8 kc2 .. 8 kc2 + 7 as a bf16 B operand
__device__ __forceinline__ bf16x8 acc_op(const f32x16& a, int kc2) {
    bf16x8 b;
#pragma unroll
    for (int x = 0; x < 8; x++) b[x] = static_cast<__bf16>(a[8 * kc2 + x]);
    return b;
}

__device__ __forceinline__ f32x16 mm4(f32x16 c, const uint16_t* a, const uint16_t* b, int lane) {
#pragma unroll
    for (int kc = 0; kc < 4; kc++) c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op(a, lane, kc), op(b, lane, kc), c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.f;
    return z;
}

// A 32 x 64 result tile pair (channels 0..31 in a0, 32..63 in a1; lane l
// holds token row l % 32) times `scale` to bf16 memory at g.
__device__ __forceinline__ void store_rows(uint16_t* g, const f32x16& a0, const f32x16& a1, float scale, int lane) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const f32x16& a = mt == 0 ? a0 : a1;
            const int d0 = 32 * mt + 8 * gq + 4 * h;
            uint2 pk;
            pk.x = (uint32_t)float_to_bf16(a[4 * gq] * scale) | ((uint32_t)float_to_bf16(a[4 * gq + 1] * scale) << 16);
            pk.y = (uint32_t)float_to_bf16(a[4 * gq + 2] * scale) | ((uint32_t)float_to_bf16(a[4 * gq + 3] * scale) << 16);
            *reinterpret_cast<uint2*>(g + n * kHeadDim + d0) = pk;
        }
}

// ---------------------------------------------------------------- transpose
__global__ __launch_bounds__(kTrThreads) void transpose_kernel(Params p) {
    extern __shared__ __align__(16) uint32_t bits[];   // [nb, words]
    __shared__ int wsum[kTrThreads / 64 + 1];
    const int bh = blockIdx.x, nb = p.nb, words = p.words, tid = threadIdx.x;
    const uint32_t* gb = p.selbits + (size_t)bh * nb * words;
    for (int x = tid; x < nb * words; x += kTrThreads) bits[x] = gb[x];
    __syncthreads();
    const int j = tid;
    int c = 0;
    if (j < nb)
        for (int i = 0; i < nb; i++) c += (bits[i * words + (j >> 5)] >> (j & 31)) & 1u;
    // exclusive scan of the column counts over the workgroup
    const int lane = tid & 63, wave = tid >> 6;
    int x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int w = 0; w < kTrThreads / 64; w++) {
            const int t = wsum[w];
            wsum[w] = acc;
            acc += t;
        }
        wsum[kTrThreads / 64] = acc;
    }
    __syncthreads();
    int pos = wsum[wave] + x - c;
    int32_t* ptr = p.ct_ptr + (size_t)bh * (nb + 1);
    int32_t* rows = p.ct_row + (size_t)bh * p.K;
    if (j < nb) {
        ptr[j] = pos;
        for (int i = 0; i < nb; i++)
            if ((bits[i * words + (j >> 5)] >> (j & 31)) & 1u) {
                if (pos < p.K) rows[pos] = i;
                pos++;
            }
    }
    if (tid == 0) {
        ptr[nb] = wsum[kTrThreads / 64];
        if ((int64_t)wsum[kTrThreads / 64] != p.K) atomicOr(reinterpret_cast<unsigned int*>(p.error), 8u);
    }
}

// ---------------------------------------------------------------- dQ
__global__ __launch_bounds__(kThreads) void dq_kernel(Params p) {
    __shared__ __align__(16) uint16_t lds[kWaves][4][kTile];   // per wave: Q_i, dO_i, K_j, V_j
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = p.nb;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    if (g >= (int64_t)p.BH * nb) return;
    const int bh = (int)(g / nb), i = (int)(g - (int64_t)bh * nb), b = bh / p.H;
    const int n = lane & 31, h = lane >> 5;
    uint16_t* qs = lds[wave][0];
    uint16_t* dos = lds[wave][1];
    uint16_t* ks = lds[wave][2];
    uint16_t* vs = lds[wave][3];
    const size_t head = (size_t)bh * p.N * kHeadDim, rowoff = head + (size_t)i * kBlock * kHeadDim;
    const uint16_t* Q = static_cast<const uint16_t*>(p.q) + head;
    const uint16_t* Kh = static_cast<const uint16_t*>(p.k) + head;
    const uint16_t* Vh = static_cast<const uint16_t*>(p.v) + head;
    const uint16_t* dO = static_cast<const uint16_t*>(p.dout) + rowoff;
    const uint16_t* Of = static_cast<const uint16_t*>(p.fout) + rowoff;
    const float tau = 1.0f / __builtin_sqrtf((float)p.d);
    const float scale2 = tau * kLog2e;

    stage(qs, Q + (size_t)i * kBlock * kHeadDim, lane);
    stage(dos, dO, lane);
    // D_t = dO_t . O_t: lane (n, h) takes channels 32 h .. 32 h + 31 of token n
    float dpart = 0.f;
#pragma unroll
    for (int x = 0; x < 4; x++) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(dO + n * kHeadDim + 32 * h + 8 * x);
        const u32x4 o = *reinterpret_cast<const u32x4*>(Of + n * kHeadDim + 32 * h + 8 * x);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            dpart += bf16_to_float(a[e] & 0xFFFFu) * bf16_to_float(o[e] & 0xFFFFu);
            dpart += bf16_to_float(a[e] >> 16) * bf16_to_float(o[e] >> 16);
        }
    }
    const float D = dpart + __shfl_xor(dpart, 32, 64);
    const bool valid = (p.mbits[(size_t)b * nb + i] >> n) & 1u;
    const int32_t* rp = p.row_ptr + (size_t)bh * (nb + 1);
    const int e0 = max(rp[i], 0), e1 = min(rp[i + 1], (int)p.K);
    const int32_t* cols = p.col + (size_t)bh * p.K;
    wave_sync_lds();

    // pass 1: the row's max (log2 units) and sum over its selected valid keys
    float m = -__builtin_inff(), lpart = 0.f;
    for (int e = e0; e < e1; e++) {
        const int j = min(max(cols[e], 0), nb - 1);
        const uint32_t km = p.mbits[(size_t)b * nb + j];
        stage(ks, Kh + (size_t)j * kBlock * kHeadDim, lane);
        wave_sync_lds();
        f32x16 S = mm4(zero16(), ks, qs, lane);   // S^T: lane = query, registers = keys
        float bm = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 16; r++) {
            S[r] = ((km >> acc_row(r, lane)) & 1u) ? S[r] * scale2 : -__builtin_inff();
            bm = fmaxf(bm, S[r]);
        }
        bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
        const float mn = fmaxf(m, bm);
        if (mn != -__builtin_inff()) {
            float ps = 0.f;
#pragma unroll
            for (int r = 0; r < 16; r++) ps += __builtin_amdgcn_exp2f(S[r] - mn);
            lpart = lpart * __builtin_amdgcn_exp2f(m - mn) + ps;
            m = mn;
        }
        wave_sync_lds();
    }
    const float l = lpart + __shfl_xor(lpart, 32, 64);
    const float mu = m == -__builtin_inff() ? 0.f : m;
    const float linv = (valid && l > 0.f) ? 1.0f / l : 0.f;
    const float Dv = linv > 0.f ? D : 0.f;
    if (h == 0) {
        const size_t t = (size_t)bh * p.N + (size_t)i * kBlock + n;
        p.st_m[t] = mu;
        p.st_linv[t] = linv;
        p.st_d[t] = Dv;
    }

    // pass 2: dQ^T += K_j^T dS^T
    f32x16 dq0 = zero16(), dq1 = zero16();
    for (int e = e0; e < e1; e++) {
        const int j = min(max(cols[e], 0), nb - 1);
        const uint32_t km = p.mbits[(size_t)b * nb + j];
        stage(ks, Kh + (size_t)j * kBlock * kHeadDim, lane);
        stage(vs, Vh + (size_t)j * kBlock * kHeadDim, lane);
        wave_sync_lds();
        const f32x16 S = mm4(zero16(), ks, qs, lane);    // S^T
        const f32x16 dP = mm4(zero16(), vs, dos, lane);  // dP^T
        f32x16 dS;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float pv = ((km >> acc_row(r, lane)) & 1u) ? __builtin_amdgcn_exp2f(S[r] * scale2 - mu) * linv : 0.f;
            dS[r] = pv * (dP[r] - Dv);
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++) {
            const bf16x8 bs = acc_op(dS, kc2);
            dq0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(ks, lane, kc2, 0), bs, dq0, 0, 0, 0);
            dq1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(ks, lane, kc2, 1), bs, dq1, 0, 0, 0);
        }
        wave_sync_lds();
    }
    store_rows(static_cast<uint16_t*>(p.dq) + rowoff, dq0, dq1, tau, lane);
}

// ---------------------------------------------------------------- dK, dV
__global__ __launch_bounds__(kThreads) void dkv_kernel(Params p) {
    __shared__ __align__(16) uint16_t lds[kWaves][4][kTile];   // per wave: K_j, V_j, Q_i, dO_i
    __shared__ __align__(16) float st[kWaves][3][kBlock];      // per wave: m, 1/l, D of block i's tokens
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = p.nb;
    const int64_t g = (int64_t)blockIdx.x * kWaves + wave;
    if (g >= (int64_t)p.BH * nb) return;
    const int bh = (int)(g / nb), j = (int)(g - (int64_t)bh * nb), b = bh / p.H;
    const int n = lane & 31;
    uint16_t* ks = lds[wave][0];
    uint16_t* vs = lds[wave][1];
    uint16_t* qs = lds[wave][2];
    uint16_t* dos = lds[wave][3];
    const size_t head = (size_t)bh * p.N * kHeadDim, coloff = head + (size_t)j * kBlock * kHeadDim;
    const uint16_t* Q = static_cast<const uint16_t*>(p.q) + head;
    const uint16_t* dO = static_cast<const uint16_t*>(p.dout) + head;
    const float tau = 1.0f / __builtin_sqrtf((float)p.d);
    const float scale2 = tau * kLog2e;

    stage(ks, static_cast<const uint16_t*>(p.k) + coloff, lane);
    stage(vs, static_cast<const uint16_t*>(p.v) + coloff, lane);
    const bool kvalid = (p.mbits[(size_t)b * nb + j] >> n) & 1u;   // lane = key n
    const int32_t* cp = p.ct_ptr + (size_t)bh * (nb + 1);
    const int c0 = max(cp[j], 0), c1 = min(cp[j + 1], (int)p.K);
    const int32_t* rows = p.ct_row + (size_t)bh * p.K;
    const size_t sbase = (size_t)bh * p.N;

    f32x16 dk0 = zero16(), dk1 = zero16(), dv0 = zero16(), dv1 = zero16();
    for (int c = c0; c < c1; c++) {
        const int i = min(max(rows[c], 0), nb - 1);
        stage(qs, Q + (size_t)i * kBlock * kHeadDim, lane);
        stage(dos, dO + (size_t)i * kBlock * kHeadDim, lane);
        if (lane < kBlock) {
            const size_t t = sbase + (size_t)i * kBlock + lane;
            st[wave][0][lane] = p.st_m[t];
            st[wave][1][lane] = p.st_linv[t];
            st[wave][2][lane] = p.st_d[t];
        }
        wave_sync_lds();
        const f32x16 S = mm4(zero16(), qs, ks, lane);    // S: lane = key, registers = queries
        const f32x16 dP = mm4(zero16(), dos, vs, lane);  // dP
        f32x16 P, dS;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int q = acc_row(r, lane);
            const float pv = kvalid ? __builtin_amdgcn_exp2f(S[r] * scale2 - st[wave][0][q]) * st[wave][1][q] : 0.f;
            P[r] = pv;
            dS[r] = pv * (dP[r] - st[wave][2][q]);
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++) {
            const bf16x8 bp = acc_op(P, kc2), bs = acc_op(dS, kc2);
            dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(dos, lane, kc2, 0), bp, dv0, 0, 0, 0);
            dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(dos, lane, kc2, 1), bp, dv1, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(qs, lane, kc2, 0), bs, dk0, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t(qs, lane, kc2, 1), bs, dk1, 0, 0, 0);
        }
        wave_sync_lds();
    }
    store_rows(static_cast<uint16_t*>(p.dk) + coloff, dk0, dk1, tau, lane);
    store_rows(static_cast<uint16_t*>(p.dv) + coloff, dv0, dv1, 1.0f, lane);
}

}  // namespace

hipError_t launch_bwd(const Params& p, hipStream_t s) {
    if (p.dtype != 1 || p.d != kHeadDim || p.nb > kTrThreads) return hipErrorInvalidValue;
    const size_t tr_lds = (size_t)p.nb * p.words * 4;
    hipLaunchKernelGGL(transpose_kernel, dim3(p.BH), dim3(kTrThreads), tr_lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t waves = (int64_t)p.BH * p.nb;
    const unsigned grid = (unsigned)((waves + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(dq_kernel, dim3(grid), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dkv_kernel, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace mra
