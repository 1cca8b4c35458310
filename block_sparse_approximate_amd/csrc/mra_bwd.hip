// mra_bwd.hip — gradients of the forward with respect to q, k and v
// ([MRA] "第三步": the block products are autograd functions whose backward
// reuses the same kernels on transposed block indices, so the selection of
// step 2 is a constant of the backward pass; [MRA] "第四步": in full mode the
// low-resolution branch is ordinary tensor code and is differentiated too,
// down through the block means).
//
// With the selection fixed, a valid query token t of block row i attends to
// the valid keys u of its selected blocks:
//   s_u = tau q_t . k_u,  P_u = 2^(s_u log2e - m_t) / l_t,  O_t = sum_u P_u v_u
// (+ the low-res part in full mode, included in m_t and l_t) and for
// dO = dL/dO, D_t = dO_t . O_t:
//   dS_u = P_u (dO_t . v_u - D_t),  dq_t = tau sum_u dS_u k_u,
//   dk_u = tau sum_t dS_u q_t,      dv_u = sum_t P_u dO_t.
// Full mode adds, for the unselected non-empty cells (i, j) with forward
// weight w_ij = cnt_j 2^((S_ij - m_i) log2e), the low-res probability of
// token t, w_ij a_t with a_t = 2^(m_i log2e - m_t) / l_t.  Summed over the
// block's tokens this needs only
//   g_i = sum_t a_t dO_t,  c_i = sum_t a_t D_t,
//   e_ij = w_ij (g_i . vhat_j - c_i)       (gradient of the logit S_ij)
//   dqhat_i = tau sum_j e_ij khat_j,  dkhat_j = tau sum_i e_ij qhat_i,
//   dvhat_j = sum_i w_ij g_i,
// and a block mean hands its gradient to each valid token of the block
// divided by the block's count (added in the dq / dkv / reduce epilogues).
//
// The forward left in its workspace the selection and each token's softmax
// statistics (m_t in log2 units and 1 / l_t), so no statistics pass is
// needed.  The kernels, in stream order after that forward call:
//   plan_kernel    per head: the query-block rows that selected each key
//                  block (column lists of the selection bitmap, ascending),
//                  and both lists cut into chunks of at most kChunkB blocks
//                  (a row or column with none is one empty chunk)
//   lr_rows_kernel full mode: g_i, c_i, e_ij, w_ij and dqhat_i, one wave
//                  per block row over key-block tiles staged in LDS
//   lr_cols_kernel full mode: dkhat_j, dvhat_j, one wave per key block
//   dq_kernel      one wave per row chunk (query block i, some of its
//                  selected blocks j):
//                    S^T = K_j Q_i^T, dP^T = V_j dO_i^T   (lane = query)
//                    dS^T = P^T (dP^T - D),  dQ^T += K_j^T dS^T
//                  and D_t, stored for dkv_kernel
//   dkv_kernel     one wave per column chunk (key block j, some of the rows
//                  i that selected it):
//                    S = Q_i K_j^T, dP = dO_i V_j^T       (lane = key)
//                    dV^T += dO_i^T P,  dK^T += Q_i^T dS
//   reduce_kernel  rows and columns of several chunks: the chunks' fp32
//                  partials summed in chunk order (the result does not
//                  depend on scheduling); single-chunk rows and columns are
//                  written directly by their wave
// Chunks keep the work even: a prior makes some rows and columns hold every
// block of the head.
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

// Head sizes HD = 64 or 128 (template parameter of every kernel below).
// bf16 chunk kernels: 2 waves per workgroup for 64 channels, 1 for 128, so
// that each wave's 4 staged blocks fit static LDS.
__host__ __device__ constexpr int chunk_waves(int hd) { return hd == 64 ? 2 : 1; }
__host__ __device__ constexpr int str_b(int hd) { return hd + 8; }          // bf16 per staged token row
__host__ __device__ constexpr int tile_b(int hd) { return kBlock * str_b(hd); }
constexpr int kTrThreads = 512;       // plan_kernel: one thread per block row / column (nb <= 512)
constexpr int kChunkB = 8;            // selected blocks per backward work chunk

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ float bf16_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// key index held by accumulator register r of a 32x32 MFMA tile in lane l
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A 32 x HD bf16 block (row-major in memory) into the wave's LDS: lane l
// moves 16 bytes of token rows l / (HD / 8) + (512 / HD) x, channels
// 8 (l % (HD / 8)) .. +7 (whole token rows per HD / 8 lanes).
template <int HD>
__device__ __forceinline__ void load_blk(u32x4 (&r)[HD / 16], const uint16_t* g, int lane) {
    constexpr int kRowLanes = HD / 8, kRows = 64 / kRowLanes;
#pragma unroll
    for (int x = 0; x < HD / 16; x++)
        r[x] = *reinterpret_cast<const u32x4*>(g + (lane / kRowLanes + kRows * x) * HD + (lane % kRowLanes) * 8);
}
template <int HD>
__device__ __forceinline__ void store_blk(uint16_t* s, const u32x4 (&r)[HD / 16], int lane) {
    constexpr int kRowLanes = HD / 8, kRows = 64 / kRowLanes;
#pragma unroll
    for (int x = 0; x < HD / 16; x++)
        *reinterpret_cast<u32x4*>(s + (lane / kRowLanes + kRows * x) * str_b(HD) + (lane % kRowLanes) * 8) = r[x];
}
template <int HD>
__device__ __forceinline__ void stage(uint16_t* s, const uint16_t* g, int lane) {
    u32x4 r[HD / 16];
    load_blk<HD>(r, g, lane);
    store_blk<HD>(s, r, lane);
}

// MFMA operand piece kc of a staged block: row l % 32, channels 16 kc + 8 (l / 32) .. +7
template <int HD>
__device__ __forceinline__ bf16x8 op(const uint16_t* s, int lane, int kc) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(s + (lane & 31) * str_b(HD) + 16 * kc + 8 * (lane >> 5)));
}

// A operand of X^T for rows (channels) 32 mt .. 32 mt + 31, contracting over
// the staged block's rows in the order that accumulator registers
// 8 kc2 .. 8 kc2 + 7 of lane l hold them (acc_row).
template <int HD>
__device__ __forceinline__ bf16x8 op_t(const uint16_t* s, int lane, int kc2, int mt) {
    const int g16 = lane >> 4, s16 = lane & 15, h = lane >> 5;
    const int col = 32 * mt + 16 * (g16 & 1) + 4 * (s16 & 3);
    const int row = 16 * kc2 + 4 * h + (s16 >> 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + row * str_b(HD) + col));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(s + (row + 8) * str_b(HD) + col));
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

// C += A B^T over the HD channels of two staged blocks
template <int HD>
__device__ __forceinline__ f32x16 mmk(f32x16 c, const uint16_t* a, const uint16_t* b, int lane) {
#pragma unroll
    for (int kc = 0; kc < HD / 16; kc++)
        c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op<HD>(a, lane, kc), op<HD>(b, lane, kc), c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int r = 0; r < 16; r++) z[r] = 0.f;
    return z;
}

// A 32 x HD result (tile mt holds channels 32 mt .. 32 mt + 31; lane l holds
// token row l % 32) times `scale`, plus add[channel] * aw when add is given
// (a block mean's gradient share), to bf16 memory at g.
template <int HD>
__device__ __forceinline__ void store_rows(uint16_t* g, const f32x16 (&a)[HD / 32], float scale, int lane,
                                           const float* add = nullptr, float aw = 0.f) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const int d0 = 32 * mt + 8 * gq + 4 * h;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; e++) x[e] = a[mt][4 * gq + e] * scale;
            if (add) {
                const float4 ad = *reinterpret_cast<const float4*>(add + d0);
                x[0] += ad.x * aw; x[1] += ad.y * aw; x[2] += ad.z * aw; x[3] += ad.w * aw;
            }
            uint2 pk;
            pk.x = pack_bf16x2(x[0], x[1]);
            pk.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2*>(g + n * HD + d0) = pk;
        }
}

// D_t = dO_t . O_t for token n = lane % 32 of a block (rows of HD bf16
// channels): lane (n, h) sums channels HD / 2 h .. + HD / 2 - 1, then the halves.
template <int HD>
__device__ __forceinline__ float row_dot(const uint16_t* dO, const uint16_t* O, int lane) {
    const int n = lane & 31, h = lane >> 5;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < HD / 16; x++) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(dO + n * HD + (HD / 2) * h + 8 * x);
        const u32x4 o = *reinterpret_cast<const u32x4*>(O + n * HD + (HD / 2) * h + 8 * x);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            s += bf16_to_float(a[e] & 0xFFFFu) * bf16_to_float(o[e] & 0xFFFFu);
            s += bf16_to_float(a[e] >> 16) * bf16_to_float(o[e] >> 16);
        }
    }
    return s + __shfl_xor(s, 32, 64);
}

// Workgroup g runs on XCD g % 8.  With at least 8 heads, all workgroups of
// head bh go to XCD bh % 8 (the XCD's heads one after another), so the
// blocks a head re-reads stay in one L2; per_head = workgroups per head.
__device__ __forceinline__ bool head_slot(int BH, int per_head, int* bh, int* idx) {
    if (BH >= 8) {
        const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3, hl = k / per_head;
        *bh = xcd + 8 * hl;
        *idx = k - hl * per_head;
    } else {
        *bh = blockIdx.x / per_head;
        *idx = blockIdx.x - *bh * per_head;
    }
    return *bh < BH;
}

// The same grid for the chunk kernels, with the heads of an XCD interleaved:
// its workgroups take chunk group idx of each of its heads in turn, so that
// every head's first (longest) chunks start in the first round.
__device__ __forceinline__ bool head_slot_interleaved(int BH, int per_head, int* bh, int* idx) {
    if (BH >= 8) {
        const int hpx = (BH + 7) / 8;
        const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3, hl = k % hpx;
        *bh = xcd + 8 * hl;
        *idx = k / hpx;
    } else {
        *bh = blockIdx.x % BH;
        *idx = blockIdx.x / BH;
    }
    return *bh < BH && *idx < per_head;
}

inline unsigned head_grid(int BH, int per_head) {
    return (unsigned)(BH >= 8 ? 8 * (int64_t)((BH + 7) / 8) * per_head : (int64_t)BH * per_head);
}

// D_t for fp32 rows: lane (n, h) sums channels HD / 2 h .. + HD / 2 - 1 of token n.
template <int HD>
__device__ __forceinline__ float row_dot32(const float* dO, const float* O, int lane) {
    const int n = lane & 31, h = lane >> 5;
    float s = 0.f;
#pragma unroll
    for (int x = 0; x < HD / 8; x++) {
        const float4 a = *reinterpret_cast<const float4*>(dO + n * HD + (HD / 2) * h + 4 * x);
        const float4 o = *reinterpret_cast<const float4*>(O + n * HD + (HD / 2) * h + 4 * x);
        s += a.x * o.x + a.y * o.y + a.z * o.z + a.w * o.w;
    }
    return s + __shfl_xor(s, 32, 64);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------- plan
// exclusive scan of one value per thread over the plan workgroup; *total gets the sum
template <typename T>
__device__ __forceinline__ T plan_scan(T v, T* wsum, T* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    T x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        T acc = 0;
        for (int w = 0; w < kTrThreads / 64; w++) {
            const T t = wsum[w];
            wsum[w] = acc;
            acc += t;
        }
        wsum[kTrThreads / 64] = acc;
    }
    __syncthreads();
    const T ex = wsum[wave] + x - v;
    *total = wsum[kTrThreads / 64];
    __syncthreads();
    return ex;
}

__global__ __launch_bounds__(kTrThreads) void plan_kernel(Params p) {
    extern __shared__ __align__(16) uint32_t cbits[];   // [nb, words]: column j's bitmap over block rows,
                                                        // then [nb] each column's list start
    __shared__ uint64_t wsum[kTrThreads / 64 + 1];
    const int bh = blockIdx.x, nb = p.nb, words = p.words, x = threadIdx.x;
    const int K = (int)p.K, maxch = p.bwd_maxch;
    const uint32_t* gb = p.selbits + (size_t)bh * nb * words;   // row i's bitmap over key blocks
    // transpose the bitmap, one (column j, 32-row word wi) per item; the
    // threads of a wave share wi and read the same row words
    for (int it = x; it < nb * words; it += kTrThreads) {
        const int wi = it / nb, j = it - wi * nb;
        const int i0 = 32 * wi, rows = min(32, nb - i0);
        uint32_t w[32];   // all 32 row words in flight at once
#pragma unroll
        for (int r = 0; r < 32; r++) w[r] = r < rows ? gb[(size_t)(i0 + r) * words + (j >> 5)] : 0u;
        uint32_t m = 0;
#pragma unroll
        for (int r = 0; r < 32; r++) m |= ((w[r] >> (j & 31)) & 1u) << r;
        cbits[j * words + wi] = m;
    }
    __syncthreads();
    const bool on = x < nb;
    // thread x: block row x and key block column x
    int ccount = 0;
    if (on)
        for (int wi = 0; wi < words; wi++) ccount += __popc(cbits[x * words + wi]);
    const int32_t* rp = p.row_ptr + (size_t)bh * (nb + 1);
    const int e0 = on ? min(max(rp[x], 0), K) : 0, e1 = on ? min(max(rp[x + 1], e0), K) : 0;
    const int nr = on ? max(1, (e1 - e0 + kChunkB - 1) / kChunkB) : 0;
    const int nc = on ? max(1, (ccount + kChunkB - 1) / kChunkB) : 0;
    // two scans of packed fields: column counts, row chunks and column chunks
    // (21 bits each: totals stay below K + nb + K / kChunkB < 2^21), then
    // the rows and columns of several chunks (16 bits each, totals <= nb)
    constexpr uint64_t kM21 = (1u << 21) - 1;
    uint64_t t1, t2;
    const uint64_t s1 = plan_scan<uint64_t>((uint64_t)ccount | ((uint64_t)nr << 21) | ((uint64_t)nc << 42), wsum, &t1);
    const uint64_t s2 = plan_scan<uint64_t>((uint64_t)(nr > 1 ? 1 : 0) | ((uint64_t)(nc > 1 ? 1 : 0) << 16), wsum, &t2);
    const int cpos = (int)(s1 & kM21), rbase = (int)((s1 >> 21) & kM21), cbase = (int)(s1 >> 42);
    const int tot_c = (int)(t1 & kM21), tot_r = (int)((t1 >> 21) & kM21), tot_cc = (int)(t1 >> 42);
    const int rm = (int)(s2 & 0xFFFFu), cm = (int)(s2 >> 16);
    const int tot_rm = (int)(t2 & 0xFFFFu), tot_cm = (int)(t2 >> 16);
    int32_t* cptr = p.ct_ptr + (size_t)bh * (nb + 1);
    int32_t* crow = p.ct_row + (size_t)bh * K;
    int4* rch = p.bwd_rch + (size_t)bh * maxch;
    int4* cch = p.bwd_cch + (size_t)bh * maxch;
    int* cstart = reinterpret_cast<int*>(cbits + nb * words);
    // The chunk lists go longest first (the chunk kernels' waves take them
    // in list order, so the long ones start in the first round and the
    // short ones fill in behind them): a count of chunks per length, its
    // scan from the longest length down, then each thread's chunks placed
    // in their length's range.  A chunk keeps its partial slot (slot = its
    // index among its row's or column's chunks, from rbase / cbase), so the
    // order changes only which wave computes it when.
    __shared__ int lcnt[2][kChunkB + 1], lnext[2][kChunkB + 1];
    if (x < 2 * (kChunkB + 1)) (&lcnt[0][0])[x] = 0;
    __syncthreads();
    const int rlast = on ? (e1 - e0) - kChunkB * (nr - 1) : 0;   // length of the row's last chunk
    const int clast = on ? ccount - kChunkB * (nc - 1) : 0;
    if (on) {
        if (nr > 1) atomicAdd(&lcnt[0][kChunkB], nr - 1);
        atomicAdd(&lcnt[0][rlast], 1);
        if (nc > 1) atomicAdd(&lcnt[1][kChunkB], nc - 1);
        atomicAdd(&lcnt[1][clast], 1);
    }
    __syncthreads();
    if (x < 2) {
        int acc = 0;
        for (int L = kChunkB; L >= 0; L--) {
            lnext[x][L] = acc;
            acc += lcnt[x][L];
        }
    }
    __syncthreads();
    if (on) {
        cptr[x] = cpos;
        cstart[x] = cpos;
        const int rf = nr > 1 ? atomicAdd(&lnext[0][kChunkB], nr - 1) : 0, rl = atomicAdd(&lnext[0][rlast], 1);
        for (int c = 0; c < nr; c++) {
            const int at = c + 1 < nr ? rf + c : rl;
            if (at < maxch)
                rch[at] = make_int4(x, e0 + c * kChunkB, min(e0 + (c + 1) * kChunkB, e1), nr > 1 ? rbase + c : -1);
        }
        const int c0 = cpos, c1 = min(cpos + ccount, K);
        const int cf = nc > 1 ? atomicAdd(&lnext[1][kChunkB], nc - 1) : 0, cl = atomicAdd(&lnext[1][clast], 1);
        for (int c = 0; c < nc; c++) {
            const int at = c + 1 < nc ? cf + c : cl;
            if (at < maxch)
                cch[at] = make_int4(x, c0 + c * kChunkB, min(c0 + (c + 1) * kChunkB, c1), nc > 1 ? cbase + c : -1);
        }
        if (nr > 1) p.bwd_rmul[(size_t)bh * nb + rm] = make_int4(x, rbase, nr, 0);
        if (nc > 1) p.bwd_cmul[(size_t)bh * nb + cm] = make_int4(x, cbase, nc, 0);
    }
    // column lists (ascending rows), one thread per selected cell c in
    // column order: its column is the last whose list starts at or before
    // c, its row the bit of rank c - start among the column's set bits
    __syncthreads();
    const int ncell = min(tot_c, K);
    for (int c = x; c < ncell; c += kTrThreads) {
        int lo = 0, hi = nb - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (cstart[mid] <= c) lo = mid;
            else hi = mid - 1;
        }
        const uint32_t* cw = cbits + lo * words;
        int r = c - cstart[lo], wi = 0;
        uint32_t bits = cw[0];
        int cn = __popc(bits);
        while (r >= cn && wi + 1 < words) {
            r -= cn;
            bits = cw[++wi];
            cn = __popc(bits);
        }
        int pos = 0;
#pragma unroll
        for (int half = 16; half > 0; half >>= 1) {
            const uint32_t low = bits & ((1u << half) - 1u);
            const int cl = __popc(low);
            if (r >= cl) {
                r -= cl;
                bits >>= half;
                pos += half;
            } else {
                bits = low;
            }
        }
        crow[c] = 32 * wi + pos;
    }
    if (x == 0) {
        cptr[nb] = tot_c;
        p.bwd_count[bh] = make_int4(min(tot_r, maxch), min(tot_cc, maxch), tot_rm, tot_cm);
        // a static layout fills row_ptr[nb] of the stream's capacity K
        const int want = p.attn_dyn ? min(rp[nb], K) : K;
        if (tot_c != want || tot_r > maxch || tot_cc > maxch) atomicOr(reinterpret_cast<unsigned int*>(p.error), 8u);
        // the forward must have kept each token's softmax statistics
        if (p.error[1] != 1) atomicOr(reinterpret_cast<unsigned int*>(p.error), 16u);
    }
}

// A wave's 32 x HD fp32 partial (tile mt: channels 32 mt .. 32 mt + 31; lane
// l holds token row l % 32) to a contiguous [32, HD] slot.
template <int HD>
__device__ __forceinline__ void store_part(float* g, const f32x16 (&a)[HD / 32], int lane) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++)
            *reinterpret_cast<float4*>(g + n * HD + 32 * mt + 8 * gq + 4 * h) =
                make_float4(a[mt][4 * gq], a[mt][4 * gq + 1], a[mt][4 * gq + 2], a[mt][4 * gq + 3]);
}

// ---------------------------------------------------------------- low-res (full mode)
constexpr int kLrWaves = 8;            // block rows (columns) per workgroup, one per wave
constexpr int kLrThreads = kLrWaves * 64;
constexpr int kLrTile = 64;            // key blocks (query blocks) per staged tile
// dynamic LDS of the low-res kernels (128-channel tiles exceed static LDS)
__host__ __device__ constexpr size_t lr_rows_lds(int hd) {
    return ((size_t)kLrTile * (hd + 4) + (size_t)kLrTile * (hd + 1) + (size_t)kLrWaves * (hd + 1) +
            2 * kLrWaves * (kLrTile + 1) + kLrWaves * kBlock) * 4;
}
__host__ __device__ constexpr size_t lr_cols_lds(int hd) {
    return (2 * (size_t)kLrTile * hd + 2 * kLrWaves * kLrTile) * 4;
}

// Workgroup (bh, rows i0 .. i0 + 7), wave w takes row i = i0 + w:
//   phase 1: a_t, D_t of the row's tokens; g_i (lane = channel, and channel
//            + 64 for 128-channel heads), c_i
//   phase 2: per tile of kLrTile key blocks (vhat, khat staged): wave = row,
//            lane = j forms w_ij (the forward's weight, 0 for selected or
//            empty cells); then on the matrix core T = G Vhat^T (waves 0..3,
//            16 key blocks each), e_ij = w_ij (T_ij - c_i), and
//            dqhat += E Khat (wave w: channels 16 w ..).  E and W go out
//            transposed ([j][i], 8 consecutive rows per j).
template <int DT, int HD>
__global__ __launch_bounds__(kLrThreads) void lr_rows_kernel(Params p) {
    constexpr int kCx = HD / 64;   // channels per lane
    // kt [kLrTile][HD + 4] first (16-byte stores), then vt [kLrTile][HD + 1], gs [kLrWaves][HD + 1], es and
    // ws [kLrWaves][kLrTile + 1], al [kLrWaves][kBlock]; the padded strides spread the MFMA operand reads
    // (16 rows or keys by 4 columns a read) over the banks
    extern __shared__ __align__(16) float lrs[];
    float (*kt)[HD + 4] = reinterpret_cast<float (*)[HD + 4]>(lrs);
    float (*vt)[HD + 1] = reinterpret_cast<float (*)[HD + 1]>(lrs + kLrTile * (HD + 4));
    float (*gs)[HD + 1] = reinterpret_cast<float (*)[HD + 1]>(lrs + kLrTile * (HD + 4) + kLrTile * (HD + 1));
    float (*es)[kLrTile + 1] = reinterpret_cast<float (*)[kLrTile + 1]>(lrs + kLrTile * (HD + 4) + kLrTile * (HD + 1) +
                                                                        kLrWaves * (HD + 1));
    float (*ws)[kLrTile + 1] = es + kLrWaves;
    float (*al)[kBlock] = reinterpret_cast<float (*)[kBlock]>(ws + kLrWaves);
    const int nb = p.nb, groups = (nb + kLrWaves - 1) / kLrWaves;
    int bh, grp;
    if (!head_slot(p.BH, groups, &bh, &grp)) return;
    const int i0 = grp * kLrWaves;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int i = i0 + wave, b = bh / p.H;
    const bool act = i < nb;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const size_t hrow = (size_t)bh * nb + (act ? i : 0);
    const float mi = p.rowmax[hrow];

    // a tile's inputs, one tile ahead: vhat and khat rows, and this lane's
    // logit, key count and selection word for the weight of (row, key block)
    const float* S = p.logits + hrow * nb;
    const uint32_t* sbits = p.selbits + hrow * p.words;
    const int32_t* cnt = p.cnt + (size_t)b * nb;
    const float* vh = p.vhat + (size_t)bh * nb * HD;
    const float* kh = p.khat + (size_t)bh * nb * HD;
    constexpr int kTL = kLrTile * (HD / 4) / kLrThreads;   // float4s of a tile per thread and tensor
    float4 tv[kTL], tk[kTL];
    float tS = 0.f;
    int tc = 0;
    uint32_t tb = 0xFFFFFFFFu;
    auto fetch_tile = [&](int j0) {
#pragma unroll
        for (int e = 0; e < kTL; e++) {
            const int x = tid + e * kLrThreads, j = j0 + x / (HD / 4), c4 = (x % (HD / 4)) * 4;
            tv[e] = j < nb ? *reinterpret_cast<const float4*>(vh + (size_t)j * HD + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
            tk[e] = j < nb ? *reinterpret_cast<const float4*>(kh + (size_t)j * HD + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const int j = j0 + lane;
        tS = act && j < nb ? S[j] : 0.f;
        tc = j < nb ? cnt[j] : 0;
        tb = act && j < nb ? sbits[j >> 5] : 0xFFFFFFFFu;
    };
    fetch_tile(0);

    float ci = 0.f;
    if (act) {
        const size_t rowoff = ((size_t)bh * p.N + (size_t)i * kBlock) * HD;
        const int n = lane & 31, h = lane >> 5;
        // dO at this lane's channels for every token of the row, loaded with the
        // row's first loads: g_i below then needs no further round trip
        float dv[kCx][kBlock];
#pragma unroll
        for (int x = 0; x < kCx; x++) {
#pragma unroll
            for (int u = 0; u < kBlock; u++) {
                if constexpr (DT == 1)
                    dv[x][u] = bf16_to_float(static_cast<const uint16_t*>(p.dout)[rowoff + u * HD + lane + 64 * x]);
                else
                    dv[x][u] = static_cast<const float*>(p.dout)[rowoff + u * HD + lane + 64 * x];
            }
        }
        float D;
        if constexpr (DT == 1)
            D = row_dot<HD>(static_cast<const uint16_t*>(p.dout) + rowoff,
                            static_cast<const uint16_t*>(p.fout) + rowoff, lane);
        else
            D = row_dot32<HD>(static_cast<const float*>(p.dout) + rowoff, static_cast<const float*>(p.fout) + rowoff,
                              lane);
        const size_t t = (size_t)bh * p.N + (size_t)i * kBlock + n;
        const float mu = p.st_m[t], linv = p.st_linv[t];
        const float a = linv > 0.f ? __builtin_amdgcn_exp2f(mi * kLog2e - mu) * linv : 0.f;
        if (h == 0) al[wave][n] = a;
        ci = wave_sum(h == 0 ? a * D : 0.f);
        wave_sync_lds();
#pragma unroll
        for (int x = 0; x < kCx; x++) {
            const int c = lane + 64 * x;
            float g = 0.f;
#pragma unroll
            for (int u = 0; u < kBlock; u++) g += al[wave][u] * dv[x][u];
            gs[wave][c] = g;
            p.bwd_g[hrow * HD + c] = g;
        }
        if (lane == 0) p.bwd_c[hrow] = ci;
    } else {
#pragma unroll
        for (int x = 0; x < kCx; x++) gs[wave][lane + 64 * x] = 0.f;   // rows past the head: T = 0
    }
    if (lane == 0) al[wave][0] = ci;   // al is free now: row c_i for the tile products

    // the tile products on v_mfma_f32_16x16x4f32 (16-row tiles, rows 8 .. 15
    // zero): A lane l holds X[l % 16][k = l / 16], B lane l holds Y[k = l / 16]
    // [l % 16], accumulator e of lane l is row 4 (l / 16) + e, column l % 16
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int l16 = lane & 15, k4 = lane >> 4;
    f32x4 dq = {0.f, 0.f, 0.f, 0.f};   // wave w < HD / 16: dqhat of channels 16 w .. 16 w + 15
    for (int j0 = 0; j0 < nb; j0 += kLrTile) {
        __syncthreads();   // every wave is done with the previous tile
#pragma unroll
        for (int e = 0; e < kTL; e++) {
            const int x = tid + e * kLrThreads, r = x / (HD / 4), c4 = (x % (HD / 4)) * 4;
            vt[r][c4] = tv[e].x; vt[r][c4 + 1] = tv[e].y; vt[r][c4 + 2] = tv[e].z; vt[r][c4 + 3] = tv[e].w;
            *reinterpret_cast<float4*>(&kt[r][c4]) = tk[e];
        }
        // w_ij of the tile (wave = row, lane = key block)
        {
            const int j = j0 + lane;
            ws[wave][lane] = (act && j < nb && !((tb >> (j & 31)) & 1u)) ? lowres_weight(tS, mi, tc) : 0.f;
        }
        if (j0 + kLrTile < nb) fetch_tile(j0 + kLrTile);   // in flight during this tile
        __syncthreads();
        // T = G Vhat^T (waves 0 .. 3: 16 key blocks each), then e_ij = w_ij (T_ij - c_i)
        if (wave < kLrTile / 16) {
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k0 = 0; k0 < HD; k0 += 4) {
                const float a = l16 < kLrWaves ? gs[l16][k0 + k4] : 0.f;
                t = __builtin_amdgcn_mfma_f32_16x16x4f32(a, vt[16 * wave + l16][k0 + k4], t, 0, 0, 0);
            }
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int r = 4 * k4 + e;
                if (r < kLrWaves) es[r][16 * wave + l16] = ws[r][16 * wave + l16] * (t[e] - al[r][0]);
            }
        }
        __syncthreads();
        // dqhat += E Khat (wave w < HD / 16: channels 16 w .. 16 w + 15)
        if (wave < HD / 16) {
#pragma unroll 8
            for (int k0 = 0; k0 < kLrTile; k0 += 4) {
                const float a = l16 < kLrWaves ? es[l16][k0 + k4] : 0.f;
                dq = __builtin_amdgcn_mfma_f32_16x16x4f32(a, kt[k0 + k4][16 * wave + l16], dq, 0, 0, 0);
            }
        }
        __syncthreads();   // the tile's e and w of every row
        if (tid < 2 * kLrTile) {
            const int u = tid & (kLrTile - 1), j = j0 + u;
            if (j < nb) {
                float* dst = (tid < kLrTile ? p.bwd_et : p.bwd_wt) + ((size_t)bh * nb + j) * nb + i0;
                const float (*src)[kLrTile + 1] = tid < kLrTile ? es : ws;
                for (int r = 0; r < kLrWaves && i0 + r < nb; r++) dst[r] = src[r][u];
            }
        }
    }
    if (wave < HD / 16) {
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int r = 4 * k4 + e;
            if (r < kLrWaves && i0 + r < nb) p.bwd_dqh[((size_t)bh * nb + i0 + r) * HD + 16 * wave + l16] = tau * dq[e];
        }
    }
}

// Workgroup (bh, key blocks j0 .. j0 + 7), wave w takes column j = j0 + w,
// lane = channel (and channel + 64): dvhat_j = sum_i w_ij g_i,
// dkhat_j = tau sum_i e_ij qhat_i over tiles of kLrTile query blocks (g and
// qhat staged, shared by the waves).
template <int HD>
__global__ __launch_bounds__(kLrThreads) void lr_cols_kernel(Params p) {
    constexpr int kCx = HD / 64;
    // gt, qt [kLrTile][HD], then es, ws [kLrWaves][kLrTile]
    extern __shared__ __align__(16) float lrs[];
    float (*gt)[HD] = reinterpret_cast<float (*)[HD]>(lrs);
    float (*qt)[HD] = gt + kLrTile;
    float (*es)[kLrTile] = reinterpret_cast<float (*)[kLrTile]>(lrs + 2 * kLrTile * HD);
    float (*ws)[kLrTile] = es + kLrWaves;
    const int nb = p.nb, groups = (nb + kLrWaves - 1) / kLrWaves;
    int bh, grp;
    if (!head_slot(p.BH, groups, &bh, &grp)) return;
    const int j0 = grp * kLrWaves;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int j = j0 + wave;
    const bool act = j < nb;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const float* gh = p.bwd_g + (size_t)bh * nb * HD;
    const float* qh = p.qhat + (size_t)bh * nb * HD;
    const size_t col = ((size_t)bh * nb + (act ? j : 0)) * nb;
    float dv[kCx], dk[kCx];
#pragma unroll
    for (int x = 0; x < kCx; x++) dv[x] = dk[x] = 0.f;
    // a tile's inputs, one tile ahead: g and qhat rows, and this lane's e and w
    constexpr int kTL = kLrTile * (HD / 4) / kLrThreads;   // float4s of a tile per thread and tensor
    float4 tg[kTL], tq[kTL];
    float te = 0.f, tw = 0.f;
    auto fetch_tile = [&](int r0) {
#pragma unroll
        for (int e = 0; e < kTL; e++) {
            const int x = tid + e * kLrThreads, i = r0 + x / (HD / 4), c4 = (x % (HD / 4)) * 4;
            tg[e] = i < nb ? *reinterpret_cast<const float4*>(gh + (size_t)i * HD + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
            tq[e] = i < nb ? *reinterpret_cast<const float4*>(qh + (size_t)i * HD + c4) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const int i = r0 + lane;
        te = act && i < nb ? p.bwd_et[col + i] : 0.f;
        tw = act && i < nb ? p.bwd_wt[col + i] : 0.f;
    };
    fetch_tile(0);
    for (int r0 = 0; r0 < nb; r0 += kLrTile) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kTL; e++) {
            const int x = tid + e * kLrThreads, r = x / (HD / 4), c4 = (x % (HD / 4)) * 4;
            *reinterpret_cast<float4*>(&gt[r][c4]) = tg[e];
            *reinterpret_cast<float4*>(&qt[r][c4]) = tq[e];
        }
        es[wave][lane] = te;
        ws[wave][lane] = tw;
        if (r0 + kLrTile < nb) fetch_tile(r0 + kLrTile);   // in flight during this tile
        __syncthreads();
        if (act) {
#pragma unroll
            for (int x = 0; x < kCx; x++)
#pragma unroll 16
                for (int u = 0; u < kLrTile; u++) {
                    dv[x] += ws[wave][u] * gt[u][lane + 64 * x];
                    dk[x] += es[wave][u] * qt[u][lane + 64 * x];
                }
        }
    }
    if (act) {
#pragma unroll
        for (int x = 0; x < kCx; x++) {
            p.bwd_dvh[col / nb * HD + lane + 64 * x] = dv[x];
            p.bwd_dkh[col / nb * HD + lane + 64 * x] = tau * dk[x];
        }
    }
}

// ---------------------------------------------------------------- dQ
template <int HD>
__global__ __launch_bounds__(64 * chunk_waves(HD)) void dq_kernel(Params p) {
    constexpr int kWaves = chunk_waves(HD), kKV = HD / 16, kMT = HD / 32;
    __shared__ __align__(16) uint16_t lds[kWaves][4][tile_b(HD)];   // per wave: Q_i, dO_i, K_j, V_j
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = p.nb, maxch = p.bwd_maxch;
    int bh, wg;
    if (!head_slot_interleaved(p.BH, (maxch + kWaves - 1) / kWaves, &bh, &wg)) return;
    const int cid = wg * kWaves + wave;
    if (cid >= p.bwd_count[bh].x) return;
    const int4 dsc = p.bwd_rch[(size_t)bh * maxch + cid];
    const int i = min(max(dsc.x, 0), nb - 1), b = bh / p.H;
    const int e0 = max(dsc.y, 0), e1 = min(dsc.z, (int)p.K);
    const int n = lane & 31, h = lane >> 5;
    uint16_t* qs = lds[wave][0];
    uint16_t* dos = lds[wave][1];
    uint16_t* ks = lds[wave][2];
    uint16_t* vs = lds[wave][3];
    const size_t head = (size_t)bh * p.N * HD, rowoff = head + (size_t)i * kBlock * HD;
    const uint16_t* Kh = static_cast<const uint16_t*>(p.k) + head;
    const uint16_t* Vh = static_cast<const uint16_t*>(p.v) + head;
    const uint16_t* dO = static_cast<const uint16_t*>(p.dout) + rowoff;
    const uint16_t* Of = static_cast<const uint16_t*>(p.fout) + rowoff;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const float scale2 = tau * kLog2e;

    // the next block's K and V rows and mask word travel in registers while
    // the current block is computed; the first block's are issued before
    // the row's own loads
    const int32_t* cols = p.col + (size_t)bh * p.K;
    u32x4 kr[kKV], vr[kKV];
    uint32_t kmn = 0;
    if (e0 < e1) {
        const int j = min(max(cols[e0], 0), nb - 1);
        load_blk<HD>(kr, Kh + (size_t)j * kBlock * HD, lane);
        load_blk<HD>(vr, Vh + (size_t)j * kBlock * HD, lane);
        kmn = p.mbits[(size_t)b * nb + j];
    }
    stage<HD>(qs, static_cast<const uint16_t*>(p.q) + rowoff, lane);
    stage<HD>(dos, dO, lane);
    const float dfull = row_dot<HD>(dO, Of, lane);
    const size_t t = (size_t)bh * p.N + (size_t)i * kBlock + n;
    const float mu = p.st_m[t], linv = p.st_linv[t];
    const bool qv = linv > 0.f;   // padded and keyless query tokens take no gradient
    const float Dv = qv ? dfull : 0.f;
    if (h == 0) p.st_d[t] = Dv;   // every chunk of the row writes the same value
    wave_sync_lds();

    f32x16 dq[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) dq[mt] = zero16();
    for (int e = e0; e < e1; e++) {
        const uint32_t km = kmn;
        store_blk<HD>(ks, kr, lane);
        store_blk<HD>(vs, vr, lane);
        if (e + 1 < e1) {
            const int j = min(max(cols[e + 1], 0), nb - 1);
            load_blk<HD>(kr, Kh + (size_t)j * kBlock * HD, lane);
            load_blk<HD>(vr, Vh + (size_t)j * kBlock * HD, lane);
            kmn = p.mbits[(size_t)b * nb + j];
        }
        wave_sync_lds();
        const f32x16 S = mmk<HD>(zero16(), ks, qs, lane);    // S^T: lane = query, registers = keys
        const f32x16 dP = mmk<HD>(zero16(), vs, dos, lane);  // dP^T
        f32x16 dS;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float pv = (qv && ((km >> acc_row(r, lane)) & 1u)) ? __builtin_amdgcn_exp2f(S[r] * scale2 - mu) * linv : 0.f;
            dS[r] = pv * (dP[r] - Dv);
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++) {
            const bf16x8 bs = acc_op(dS, kc2);
#pragma unroll
            for (int mt = 0; mt < kMT; mt++)
                dq[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t<HD>(ks, lane, kc2, mt), bs, dq[mt], 0, 0, 0);
        }
        wave_sync_lds();
    }
    if (dsc.w < 0) {
        const float* add = nullptr;
        float aw = 0.f;
        if (p.mode == 0) {   // the token's share of dqhat_i
            add = p.bwd_dqh + ((size_t)bh * nb + i) * HD;
            aw = ((p.mbits[(size_t)b * nb + i] >> n) & 1u) ? 1.0f / (float)p.cnt[(size_t)b * nb + i] : 0.f;
        }
        store_rows<HD>(static_cast<uint16_t*>(p.dq) + rowoff, dq, tau, lane, add, aw);
    } else store_part<HD>(p.bwd_part_dq + ((size_t)bh * maxch + min(dsc.w, maxch - 1)) * kBlock * HD, dq, lane);
}

// ---------------------------------------------------------------- dK, dV
template <int HD>
__global__ __launch_bounds__(64 * chunk_waves(HD)) void dkv_kernel(Params p) {
    constexpr int kWaves = chunk_waves(HD), kKV = HD / 16, kMT = HD / 32;
    __shared__ __align__(16) uint16_t lds[kWaves][4][tile_b(HD)];   // per wave: K_j, V_j, Q_i, dO_i
    __shared__ __align__(16) float st[kWaves][3][kBlock];      // per wave: m, 1/l, D of block i's tokens
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nb = p.nb, maxch = p.bwd_maxch;
    int bh, wg;
    if (!head_slot_interleaved(p.BH, (maxch + kWaves - 1) / kWaves, &bh, &wg)) return;
    const int cid = wg * kWaves + wave;
    if (cid >= p.bwd_count[bh].y) return;
    const int4 dsc = p.bwd_cch[(size_t)bh * maxch + cid];
    const int j = min(max(dsc.x, 0), nb - 1), b = bh / p.H;
    const int c0 = max(dsc.y, 0), c1 = min(dsc.z, (int)p.K);
    const int n = lane & 31;
    uint16_t* ks = lds[wave][0];
    uint16_t* vs = lds[wave][1];
    uint16_t* qs = lds[wave][2];
    uint16_t* dos = lds[wave][3];
    const size_t head = (size_t)bh * p.N * HD, coloff = head + (size_t)j * kBlock * HD;
    const uint16_t* Q = static_cast<const uint16_t*>(p.q) + head;
    const uint16_t* dO = static_cast<const uint16_t*>(p.dout) + head;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const float scale2 = tau * kLog2e;

    const int32_t* rows = p.ct_row + (size_t)bh * p.K;
    const size_t sbase = (size_t)bh * p.N;
    // the next row block's Q and dO rows and statistics travel in registers
    // while the current one is computed; the first one's are issued before
    // the column's own loads
    u32x4 qr[kKV], gr[kKV];
    float sm = 0.f, sl = 0.f, sd = 0.f;
    auto fetch = [&](int c) {
        const int i = min(max(rows[c], 0), nb - 1);
        load_blk<HD>(qr, Q + (size_t)i * kBlock * HD, lane);
        load_blk<HD>(gr, dO + (size_t)i * kBlock * HD, lane);
        const size_t t = sbase + (size_t)i * kBlock + (lane & 31);
        sm = p.st_m[t];
        sl = p.st_linv[t];
        sd = p.st_d[t];
    };
    if (c0 < c1) {   // a column with no selected row needs neither its K nor its V
        fetch(c0);
        stage<HD>(ks, static_cast<const uint16_t*>(p.k) + coloff, lane);
        stage<HD>(vs, static_cast<const uint16_t*>(p.v) + coloff, lane);
    }
    const bool kvalid = (p.mbits[(size_t)b * nb + j] >> n) & 1u;   // lane = key n

    f32x16 dk[kMT], dv[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) dk[mt] = dv[mt] = zero16();
    for (int c = c0; c < c1; c++) {
        store_blk<HD>(qs, qr, lane);
        store_blk<HD>(dos, gr, lane);
        if (lane < kBlock) {
            st[wave][0][lane] = sm;
            st[wave][1][lane] = sl;
            st[wave][2][lane] = sd;
        }
        if (c + 1 < c1) fetch(c + 1);
        wave_sync_lds();
        const f32x16 S = mmk<HD>(zero16(), qs, ks, lane);    // S: lane = key, registers = queries
        const f32x16 dP = mmk<HD>(zero16(), dos, vs, lane);  // dP
        f32x16 P, dS;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int q = acc_row(r, lane);
            const float li = st[wave][1][q];
            const float pv = (kvalid && li > 0.f) ? __builtin_amdgcn_exp2f(S[r] * scale2 - st[wave][0][q]) * li : 0.f;
            P[r] = pv;
            dS[r] = pv * (dP[r] - st[wave][2][q]);
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++) {
            const bf16x8 bp = acc_op(P, kc2), bs = acc_op(dS, kc2);
#pragma unroll
            for (int mt = 0; mt < kMT; mt++) {
                dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t<HD>(dos, lane, kc2, mt), bp, dv[mt], 0, 0, 0);
                dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op_t<HD>(qs, lane, kc2, mt), bs, dk[mt], 0, 0, 0);
            }
        }
        wave_sync_lds();
    }
    if (dsc.w < 0) {
        const float* addk = nullptr;
        const float* addv = nullptr;
        float aw = 0.f;
        if (p.mode == 0) {   // the key's share of dkhat_j, dvhat_j
            addk = p.bwd_dkh + ((size_t)bh * nb + j) * HD;
            addv = p.bwd_dvh + ((size_t)bh * nb + j) * HD;
            aw = kvalid ? 1.0f / (float)p.cnt[(size_t)b * nb + j] : 0.f;
        }
        store_rows<HD>(static_cast<uint16_t*>(p.dk) + coloff, dk, tau, lane, addk, aw);
        store_rows<HD>(static_cast<uint16_t*>(p.dv) + coloff, dv, 1.0f, lane, addv, aw);
    } else {
        const size_t slot = ((size_t)bh * maxch + min(dsc.w, maxch - 1)) * kBlock * HD;
        store_part<HD>(p.bwd_part_dk + slot, dk, lane);
        store_part<HD>(p.bwd_part_dv + slot, dv, lane);
    }
}

// ---------------------------------------------------------------- fp32 chunks
// The same products on fp32 operands with v_mfma_f32_32x32x2f32 (32 token
// rows of HD channels per staged block, row stride HD + 1 so that lanes
// reading a column of different rows fall on different banks; the staged
// blocks of 128-channel heads exceed static LDS, so these kernels take
// dynamic LDS).  For a
// product over the channels lane l takes row l % 32, channel 2 s + l / 32 at
// step s, for A and B alike.  For a product over the block's tokens, the
// accumulator of the previous product is the B operand: at step s lane l
// gives its register s, the token acc_row(s, l), and the A operand is read
// transposed from the staged block at that same token.
__host__ __device__ constexpr int str32(int hd) { return hd + 1; }   // fp32 per staged token row
__host__ __device__ constexpr int tile32(int hd) { return kBlock * str32(hd); }
// LDS of the fp32 chunk kernels: 4 staged blocks, then (dkv) 3 x 32 statistics
__host__ __device__ constexpr size_t lds32_bytes(int hd) { return (4 * (size_t)tile32(hd) + 3 * kBlock) * 4; }

template <int HD>
__device__ __forceinline__ void load_blk32(float4 (&r)[HD / 8], const float* g, int lane) {
    constexpr int kRowLanes = HD / 4, kRows = 64 / kRowLanes;
#pragma unroll
    for (int x = 0; x < HD / 8; x++)
        r[x] = *reinterpret_cast<const float4*>(g + (lane / kRowLanes + kRows * x) * HD + (lane % kRowLanes) * 4);
}
template <int HD>
__device__ __forceinline__ void store_blk32(float* s, const float4 (&r)[HD / 8], int lane) {
    constexpr int kRowLanes = HD / 4, kRows = 64 / kRowLanes;
#pragma unroll
    for (int x = 0; x < HD / 8; x++) {
        float* d = s + (lane / kRowLanes + kRows * x) * str32(HD) + (lane % kRowLanes) * 4;
        d[0] = r[x].x; d[1] = r[x].y; d[2] = r[x].z; d[3] = r[x].w;
    }
}
// C += A B^T over the HD channels: A, B staged blocks (rows = the result's rows / columns)
template <int HD>
__device__ __forceinline__ f32x16 mm32(f32x16 c, const float* a, const float* b, int lane) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll 8
    for (int st = 0; st < HD / 2; st++)
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[n * str32(HD) + 2 * st + h], b[n * str32(HD) + 2 * st + h], c, 0,
                                                 0, 0);
    return c;
}
// C[channel][col] += sum_t X[t][32 mt + channel] acc[t][col] over the block's 32 tokens
template <int HD>
__device__ __forceinline__ f32x16 mm32_t(f32x16 c, const float* x, const f32x16& acc, int mt, int lane) {
    const int m = lane & 31;
#pragma unroll
    for (int st = 0; st < 16; st++)
        c = __builtin_amdgcn_mfma_f32_32x32x2f32(x[acc_row(st, lane) * str32(HD) + 32 * mt + m], acc[st], c, 0, 0, 0);
    return c;
}
// result tiles (lane = token, registers = channels) times scale, plus add, to fp32 rows
template <int HD>
__device__ __forceinline__ void store_rows32(float* g, const f32x16 (&a)[HD / 32], float scale, int lane,
                                             const float* add, float aw) {
    const int n = lane & 31, h = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const int d0 = 32 * mt + 8 * gq + 4 * h;
            float4 x = make_float4(a[mt][4 * gq] * scale, a[mt][4 * gq + 1] * scale, a[mt][4 * gq + 2] * scale,
                                   a[mt][4 * gq + 3] * scale);
            if (add) {
                const float4 ad = *reinterpret_cast<const float4*>(add + d0);
                x.x += ad.x * aw; x.y += ad.y * aw; x.z += ad.z * aw; x.w += ad.w * aw;
            }
            *reinterpret_cast<float4*>(g + n * HD + d0) = x;
        }
}

template <int HD>
__global__ __launch_bounds__(64) void dq32_kernel(Params p) {
    extern __shared__ __align__(16) float lds32[];   // Q_i, dO_i, K_j, V_j: lds32_bytes(HD)
    constexpr int kMT = HD / 32;
    const int lane = threadIdx.x & 63;
    const int nb = p.nb, maxch = p.bwd_maxch;
    int bh, cid;
    if (!head_slot_interleaved(p.BH, maxch, &bh, &cid)) return;
    if (cid >= p.bwd_count[bh].x) return;
    const int4 dsc = p.bwd_rch[(size_t)bh * maxch + cid];
    const int i = min(max(dsc.x, 0), nb - 1), b = bh / p.H;
    const int e0 = max(dsc.y, 0), e1 = min(dsc.z, (int)p.K);
    const int n = lane & 31, h = lane >> 5;
    float* qs = lds32;
    float* dos = lds32 + tile32(HD);
    float* ks = lds32 + 2 * tile32(HD);
    float* vs = lds32 + 3 * tile32(HD);
    const size_t head = (size_t)bh * p.N * HD, rowoff = head + (size_t)i * kBlock * HD;
    const float* Kh = static_cast<const float*>(p.k) + head;
    const float* Vh = static_cast<const float*>(p.v) + head;
    const float* dO = static_cast<const float*>(p.dout) + rowoff;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const float scale2 = tau * kLog2e;
    const int32_t* cols = p.col + (size_t)bh * p.K;
    float4 r[HD / 8];
    load_blk32<HD>(r, static_cast<const float*>(p.q) + rowoff, lane);
    store_blk32<HD>(qs, r, lane);
    load_blk32<HD>(r, dO, lane);
    store_blk32<HD>(dos, r, lane);
    const float dfull = row_dot32<HD>(dO, static_cast<const float*>(p.fout) + rowoff, lane);
    const size_t t = (size_t)bh * p.N + (size_t)i * kBlock + n;
    const float mu = p.st_m[t], linv = p.st_linv[t];
    const bool qv = linv > 0.f;
    const float Dv = qv ? dfull : 0.f;
    if (h == 0) p.st_d[t] = Dv;
    f32x16 dq[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) dq[mt] = zero16();
    for (int e = e0; e < e1; e++) {
        const int j = min(max(cols[e], 0), nb - 1);
        const uint32_t km = p.mbits[(size_t)b * nb + j];
        load_blk32<HD>(r, Kh + (size_t)j * kBlock * HD, lane);
        store_blk32<HD>(ks, r, lane);
        load_blk32<HD>(r, Vh + (size_t)j * kBlock * HD, lane);
        store_blk32<HD>(vs, r, lane);
        wave_sync_lds();
        const f32x16 S = mm32<HD>(zero16(), ks, qs, lane);     // S^T: lane = query, registers = keys
        const f32x16 dP = mm32<HD>(zero16(), vs, dos, lane);   // dP^T
        f32x16 dS;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            const float pv = (qv && ((km >> acc_row(rr, lane)) & 1u)) ? __builtin_amdgcn_exp2f(S[rr] * scale2 - mu) * linv : 0.f;
            dS[rr] = pv * (dP[rr] - Dv);
        }
#pragma unroll
        for (int mt = 0; mt < kMT; mt++) dq[mt] = mm32_t<HD>(dq[mt], ks, dS, mt, lane);   // dQ^T += K^T dS^T
        wave_sync_lds();
    }
    if (dsc.w < 0) {
        const float* add = nullptr;
        float aw = 0.f;
        if (p.mode == 0) {
            add = p.bwd_dqh + ((size_t)bh * nb + i) * HD;
            aw = ((p.mbits[(size_t)b * nb + i] >> n) & 1u) ? 1.0f / (float)p.cnt[(size_t)b * nb + i] : 0.f;
        }
        store_rows32<HD>(static_cast<float*>(p.dq) + rowoff, dq, tau, lane, add, aw);
    } else store_part<HD>(p.bwd_part_dq + ((size_t)bh * maxch + min(dsc.w, maxch - 1)) * kBlock * HD, dq, lane);
}

template <int HD>
__global__ __launch_bounds__(64) void dkv32_kernel(Params p) {
    // K_j, V_j, Q_i, dO_i, then m, 1/l, D of block i's tokens: lds32_bytes(HD)
    extern __shared__ __align__(16) float lds32[];
    constexpr int kMT = HD / 32;
    float (*st)[kBlock] = reinterpret_cast<float (*)[kBlock]>(lds32 + 4 * tile32(HD));
    const int lane = threadIdx.x & 63;
    const int nb = p.nb, maxch = p.bwd_maxch;
    int bh, cid;
    if (!head_slot_interleaved(p.BH, maxch, &bh, &cid)) return;
    if (cid >= p.bwd_count[bh].y) return;
    const int4 dsc = p.bwd_cch[(size_t)bh * maxch + cid];
    const int j = min(max(dsc.x, 0), nb - 1), b = bh / p.H;
    const int c0 = max(dsc.y, 0), c1 = min(dsc.z, (int)p.K);
    const int n = lane & 31;
    float* ks = lds32;
    float* vs = lds32 + tile32(HD);
    float* qs = lds32 + 2 * tile32(HD);
    float* dos = lds32 + 3 * tile32(HD);
    const size_t head = (size_t)bh * p.N * HD, coloff = head + (size_t)j * kBlock * HD;
    const float* Q = static_cast<const float*>(p.q) + head;
    const float* dO = static_cast<const float*>(p.dout) + head;
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const float scale2 = tau * kLog2e;
    const int32_t* rows = p.ct_row + (size_t)bh * p.K;
    const size_t sbase = (size_t)bh * p.N;
    float4 r[HD / 8];
    load_blk32<HD>(r, static_cast<const float*>(p.k) + coloff, lane);
    store_blk32<HD>(ks, r, lane);
    load_blk32<HD>(r, static_cast<const float*>(p.v) + coloff, lane);
    store_blk32<HD>(vs, r, lane);
    const bool kvalid = (p.mbits[(size_t)b * nb + j] >> n) & 1u;   // lane = key n
    f32x16 dk[kMT], dv[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) dk[mt] = dv[mt] = zero16();
    for (int c = c0; c < c1; c++) {
        const int i = min(max(rows[c], 0), nb - 1);
        load_blk32<HD>(r, Q + (size_t)i * kBlock * HD, lane);
        store_blk32<HD>(qs, r, lane);
        load_blk32<HD>(r, dO + (size_t)i * kBlock * HD, lane);
        store_blk32<HD>(dos, r, lane);
        if (lane < kBlock) {
            const size_t t = sbase + (size_t)i * kBlock + lane;
            st[0][lane] = p.st_m[t];
            st[1][lane] = p.st_linv[t];
            st[2][lane] = p.st_d[t];
        }
        wave_sync_lds();
        const f32x16 S = mm32<HD>(zero16(), qs, ks, lane);     // S: lane = key, registers = queries
        const f32x16 dP = mm32<HD>(zero16(), dos, vs, lane);
        f32x16 P, dS;
#pragma unroll
        for (int rr = 0; rr < 16; rr++) {
            const int q = acc_row(rr, lane);
            const float li = st[1][q];
            const float pv = (kvalid && li > 0.f) ? __builtin_amdgcn_exp2f(S[rr] * scale2 - st[0][q]) * li : 0.f;
            P[rr] = pv;
            dS[rr] = pv * (dP[rr] - st[2][q]);
        }
#pragma unroll
        for (int mt = 0; mt < kMT; mt++) {
            dv[mt] = mm32_t<HD>(dv[mt], dos, P, mt, lane);     // dV^T += dO^T P
            dk[mt] = mm32_t<HD>(dk[mt], qs, dS, mt, lane);     // dK^T += Q^T dS
        }
        wave_sync_lds();
    }
    if (dsc.w < 0) {
        const float* addk = nullptr;
        const float* addv = nullptr;
        float aw = 0.f;
        if (p.mode == 0) {
            addk = p.bwd_dkh + ((size_t)bh * nb + j) * HD;
            addv = p.bwd_dvh + ((size_t)bh * nb + j) * HD;
            aw = kvalid ? 1.0f / (float)p.cnt[(size_t)b * nb + j] : 0.f;
        }
        store_rows32<HD>(static_cast<float*>(p.dk) + coloff, dk, tau, lane, addk, aw);
        store_rows32<HD>(static_cast<float*>(p.dv) + coloff, dv, 1.0f, lane, addv, aw);
    } else {
        const size_t slot = ((size_t)bh * maxch + min(dsc.w, maxch - 1)) * kBlock * HD;
        store_part<HD>(p.bwd_part_dk + slot, dk, lane);
        store_part<HD>(p.bwd_part_dv + slot, dv, lane);
    }
}

// ---------------------------------------------------------------- reduce
// Workgroup (bh, x, side): the x-th row (side 0) or column (side 1) of head
// bh that has several chunks.  Thread t sums token t / 8, channels
// HD / 8 (t % 8) .. + HD / 8 - 1 over the chunks in order and writes them.
constexpr int kRedThreads = 256;

template <int DT, int HD>
__device__ __forceinline__ void reduce_one(const float* part, int first, int nch, float scale, void* dst_v,
                                           size_t slot0, int tid, const float* add, float aw) {
    constexpr int kCh = HD / 8, kF4 = kCh / 4;
    const int tok = tid >> 3, cg = (tid & 7) * kCh;
    float acc[kCh];
#pragma unroll
    for (int e = 0; e < kCh; e++) acc[e] = 0.f;
    const float* base = part + (slot0 + first) * kBlock * HD + tok * HD + cg;
    constexpr int kBatch = 8;   // chunks loaded together; added in chunk order
    for (int c0 = 0; c0 < nch; c0 += kBatch) {
        float4 a[kBatch][kF4];
#pragma unroll
        for (int c = 0; c < kBatch; c++) {
            if (c0 + c < nch) {
                const float4* src = reinterpret_cast<const float4*>(base + (size_t)(c0 + c) * kBlock * HD);
#pragma unroll
                for (int x = 0; x < kF4; x++) a[c][x] = src[x];
            }
        }
#pragma unroll
        for (int c = 0; c < kBatch; c++) {
            if (c0 + c < nch) {
#pragma unroll
                for (int x = 0; x < kF4; x++) {
                    acc[4 * x] += a[c][x].x;
                    acc[4 * x + 1] += a[c][x].y;
                    acc[4 * x + 2] += a[c][x].z;
                    acc[4 * x + 3] += a[c][x].w;
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < kCh; e++) acc[e] *= scale;
    if (add) {
#pragma unroll
        for (int e = 0; e < kCh; e++) acc[e] += add[cg + e] * aw;
    }
    if constexpr (DT == 1) {
#pragma unroll
        for (int x = 0; x < kCh / 8; x++) {
            const float* v = acc + 8 * x;
            uint4 pk;
            pk.x = pack_bf16x2(v[0], v[1]);
            pk.y = pack_bf16x2(v[2], v[3]);
            pk.z = pack_bf16x2(v[4], v[5]);
            pk.w = pack_bf16x2(v[6], v[7]);
            reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst_v) + tok * HD + cg)[x] = pk;
        }
    } else {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(dst_v) + tok * HD + cg);
#pragma unroll
        for (int x = 0; x < kF4; x++) dst[x] = make_float4(acc[4 * x], acc[4 * x + 1], acc[4 * x + 2], acc[4 * x + 3]);
    }
}

template <int DT, int HD>
__device__ void reduce_item(const Params& p, int bh, int x, int side) {
    const size_t es = DT == 1 ? 2 : 4;
    const int nb = p.nb, maxch = p.bwd_maxch;
    const int4 m = (side == 0 ? p.bwd_rmul : p.bwd_cmul)[(size_t)bh * nb + x];
    const int blk = min(max(m.x, 0), nb - 1);
    const int first = max(m.y, 0), nch = max(0, min(m.z, maxch - first));
    const float tau = 1.0f / __builtin_sqrtf((float)p.dscale);
    const size_t off = ((size_t)bh * p.N + (size_t)blk * kBlock) * HD, slot0 = (size_t)bh * maxch;
    // full mode: the token's share of its block mean's gradient
    const int b = bh / p.H, tok = threadIdx.x >> 3;
    const bool full = p.mode == 0;
    const float aw = (full && ((p.mbits[(size_t)b * nb + blk] >> tok) & 1u)) ? 1.0f / (float)p.cnt[(size_t)b * nb + blk]
                                                                              : 0.f;
    const size_t hb = ((size_t)bh * nb + blk) * HD;
    if (side == 0) {
        reduce_one<DT, HD>(p.bwd_part_dq, first, nch, tau, static_cast<char*>(p.dq) + off * es, slot0, threadIdx.x,
                       full ? p.bwd_dqh + hb : nullptr, aw);
    } else {
        reduce_one<DT, HD>(p.bwd_part_dk, first, nch, tau, static_cast<char*>(p.dk) + off * es, slot0, threadIdx.x,
                       full ? p.bwd_dkh + hb : nullptr, aw);
        reduce_one<DT, HD>(p.bwd_part_dv, first, nch, 1.0f, static_cast<char*>(p.dv) + off * es, slot0, threadIdx.x,
                       full ? p.bwd_dvh + hb : nullptr, aw);
    }
}

template <int DT, int HD>
__global__ __launch_bounds__(kRedThreads) void reduce_kernel(Params p) {
    const int nb = p.nb;
    // items (x, bh, side), x slowest: the few rows and columns of several
    // chunks are the first x of each head, so they spread over the workgroups
    const int64_t items = 2 * (int64_t)p.BH * nb;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        const int side = (int)(it & 1);
        const int64_t w = it >> 1;
        const int x = (int)(w / p.BH), bh = (int)(w - (int64_t)x * p.BH);
        const int4 cnt = p.bwd_count[bh];
        if (x >= (side == 0 ? cnt.z : cnt.w)) continue;
        reduce_item<DT, HD>(p, bh, x, side);
    }
}

}  // namespace

int bwd_max_chunks(int nb, int64_t K) { return nb + (int)((K + kChunkB - 1) / kChunkB); }

template <int HD>
static hipError_t launch_bwd_t(const Params& p, hipStream_t s) {
    const bool bf = p.dtype == 1;
    const size_t plan_lds = (size_t)p.nb * (p.words + 1) * 4;
    hipLaunchKernelGGL(plan_kernel, dim3(p.BH), dim3(kTrThreads), plan_lds, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.mode == 0) {
        const unsigned lr_grid = head_grid(p.BH, (p.nb + kLrWaves - 1) / kLrWaves);
        constexpr size_t kRowsLds = lr_rows_lds(HD), kColsLds = lr_cols_lds(HD);
        static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&lr_rows_kernel<1, HD>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRowsLds);
        static const hipError_t a2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&lr_rows_kernel<0, HD>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kRowsLds);
        static const hipError_t a3 = hipFuncSetAttribute(reinterpret_cast<const void*>(&lr_cols_kernel<HD>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kColsLds);
        if (a1 != hipSuccess) return a1;
        if (a2 != hipSuccess) return a2;
        if (a3 != hipSuccess) return a3;
        if (bf) hipLaunchKernelGGL((lr_rows_kernel<1, HD>), dim3(lr_grid), dim3(kLrThreads), kRowsLds, s, p);
        else hipLaunchKernelGGL((lr_rows_kernel<0, HD>), dim3(lr_grid), dim3(kLrThreads), kRowsLds, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(lr_cols_kernel<HD>, dim3(lr_grid), dim3(kLrThreads), kColsLds, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (bf) {
        constexpr int kW = chunk_waves(HD);
        const unsigned grid = head_grid(p.BH, (p.bwd_maxch + kW - 1) / kW);
        hipLaunchKernelGGL(dq_kernel<HD>, dim3(grid), dim3(64 * kW), 0, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dkv_kernel<HD>, dim3(grid), dim3(64 * kW), 0, s, p);
    } else {
        constexpr size_t kLds = lds32_bytes(HD);
        static const hipError_t a1 = hipFuncSetAttribute(reinterpret_cast<const void*>(&dq32_kernel<HD>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        static const hipError_t a2 = hipFuncSetAttribute(reinterpret_cast<const void*>(&dkv32_kernel<HD>),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
        if (a1 != hipSuccess) return a1;
        if (a2 != hipSuccess) return a2;
        const unsigned grid = head_grid(p.BH, p.bwd_maxch);   // one wave per workgroup
        hipLaunchKernelGGL(dq32_kernel<HD>, dim3(grid), dim3(64), kLds, s, p);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(dkv32_kernel<HD>, dim3(grid), dim3(64), kLds, s, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t red_items = 2 * (int64_t)p.BH * p.nb;
    const dim3 rg((unsigned)(red_items < 1024 ? red_items : 1024));
    if (bf) hipLaunchKernelGGL((reduce_kernel<1, HD>), rg, dim3(kRedThreads), 0, s, p);
    else hipLaunchKernelGGL((reduce_kernel<0, HD>), rg, dim3(kRedThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_bwd(const Params& p, hipStream_t s) {
    if ((p.dtype != 0 && p.dtype != 1) || p.nb > kTrThreads) return hipErrorInvalidValue;
    if (p.mode == 0 && (!p.bwd_g || !p.bwd_c || !p.bwd_et || !p.bwd_wt || !p.bwd_dqh || !p.bwd_dkh || !p.bwd_dvh ||
                        !p.vhat))
        return hipErrorInvalidValue;
    if (p.d == 64) return launch_bwd_t<64>(p, s);
    if (p.d == 128) return launch_bwd_t<128>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace mra
