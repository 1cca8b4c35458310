// mra_attn.hip — step 3 ([MRA] "第三步"): exact softmax attention on the
// selected 32x32 blocks, i.e. what the pages' sampled dense matmul, row max,
// sparse-dense matmul and reduce-sum do, in one pass with an online row max.
//
// Work decomposition: the selector lists every selected block of a head in
// CSR order (block row, then key block), each row cut into segments of at
// most kChunk blocks.  W waves share a head: wave k takes the blocks
// [k*K/W, (k+1)*K/W) of that list, moved to the next segment boundaries, so
// every wave gets about the same number of blocks whatever the row lengths.
// A wave streams through its blocks in batches: it issues the K, V and Q
// loads of two blocks at once, then computes them, while the other wave on
// its SIMD does the same half a batch out of step.
//
// Per key block j of a segment of query block row i:
//   S^T = K_j Q_i^T           4 x MFMA 32x32x16 bf16 (fp32: 32 x 32x32x2 f32);
//                             bf16 K_j is loaded straight into LDS as whole
//                             rows and read back in the operand layout
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
// At the end of a segment that is a whole row the wave writes the row's
// output.  In sparse mode that is O/l (0 for padded query tokens).  In full
// mode the wave also merges the low-resolution part ([MRA] "第四步"): the
// low-res sums summed the low-res attention of the row over every key block
// (lo_all, ll_all); the wave forms the low-res weight w of each of its cells
// with the same expression from the same logit, row max and count, and takes
// the selected blocks back out,
//   lo = lo_all - sum_sel w vhat_j,   ll = ll_all - sum_sel w,
// and writes (O 2^(m - M) + lo 2^(m_i - M)) / (l 2^(m - M) + ll 2^(m_i - M))
// with M the larger of the high-res max m and the low-res row max m_i (both
// in log2 units).  Other segments write un-normalised partials (O, running
// max, sum, and in full mode the segment's sums of w vhat_j and of w) that
// the finish kernel joins.
//
// Workgroups are placed XCD-aware: workgroup g runs on XCD g % 8, and all
// waves of head bh are on XCD bh % 8, so a head's K/V re-reads stay in one L2.
// When a head has enough blocks for every wave of an XCD (long sequences),
// the XCD's waves take its heads in turn rather than side by side, so that
// L2 holds one head's K and V at a time.
#include "mra_common.h"

namespace mra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16 bytes of a K, V or Q row.  A native vector, so copies are plain loads and
// stores (HIP's uint4 struct is copied with memcpy, which can keep a batch's
// register slots in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// staged row strides for a head of hd channels (elements)
__host__ __device__ constexpr int v_stride_b(int hd) { return hd + 16; }   // bf16 V: 16 pad, no bank conflicts
__host__ __device__ constexpr int q_stride_b(int hd) { return hd + 8; }    // bf16 Q: row r's 16-byte reads start at bank group r
__host__ __device__ constexpr int v_stride_f(int hd) { return hd + 4; }    // fp32 V
constexpr int kWindow = 64;     // block records a wave holds (one per lane)
constexpr float kLazyMax = 8.0f;   // log2 headroom of the running max (probabilities <= 256)
// blocks per wave before segment alignment: an end moves up to kChunk - 1
// blocks forward, a start up to kChunk / 2 back
constexpr int kMaxRun = kWindow - kChunk - kChunk / 2;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ int rl(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// key index held by accumulator register r of a 32x32 MFMA tile in lane l
__device__ __forceinline__ int acc_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

__device__ __forceinline__ int info_pos(uint32_t x) { return (int)((x >> 18) & 63u); }
__device__ __forceinline__ int info_len(uint32_t x) { return (int)((x >> 24) & 63u); }
__device__ __forceinline__ bool info_whole(uint32_t x) { return (x >> 30) & 1u; }
__device__ __forceinline__ int info_item(uint32_t x) { return (int)(x & 0x3FFFFu); }

// The segment start nearest to stream block x (whose record info is given):
// back to its segment's start when x is in the segment's first half, else
// on to the next segment's start.  x >= K maps to K.
__device__ __forceinline__ int nearest_segment_start(int x, uint32_t info, int64_t K) {
    if (x >= K) return (int)K;
    const int pos = info_pos(info), len = info_len(info);
    return 2 * pos <= len ? x - pos : x - pos + len;
}

// DT: 1 bf16, 0 fp32; HD: channels per head (64 or 128)
template <int DT, int HD> struct Cfg;
template <int HD> struct Cfg<1, HD> {       // bf16: 16 bytes per lane per 8 elements
    static constexpr int kBatch = 2;        // blocks whose loads are in flight together
    static constexpr int kKV = HD / 16;     // 16-byte pieces per lane for one V (or Q) block
    static constexpr bool kKDirect = true;  // K goes straight from memory to LDS
    using Elem = uint16_t;
};
template <int HD> struct Cfg<0, HD> {       // fp32: twice the registers per block
    static constexpr int kBatch = 1;
    static constexpr int kKV = HD / 8;
    static constexpr bool kKDirect = false;
    using Elem = float;
};

// bf16 K block in LDS: 32 token rows of 2 HD bytes, the 16-byte chunk c of
// row r at a swizzled position of the row: c ^ ((r / 2) mod 8) for 128-byte
// rows, c ^ (r mod 16) for 256-byte ones.  The direct loads place the chunks
// so (whole rows per HD / 8 lanes, i.e. full cache lines), and the MFMA
// operand reads (lane: one row, one chunk) then hit distinct banks in each
// 16-lane phase.
template <int HD>
__device__ __forceinline__ int swz_key(int row) { return HD == 64 ? row >> 1 : row; }
template <int HD>
__device__ __forceinline__ int k_swz(int row, int chunk) {
    return row * HD + ((chunk ^ swz_key<HD>(row)) & (HD / 8 - 1)) * 8;
}

// Per-wave LDS.  bf16: the K blocks of a batch (k_swz), V_j (read back
// transposed) and Q_i; fp32: V_j.
template <int DT, int HD> struct StageBuf;
template <int HD> struct StageBuf<1, HD> {
    uint16_t kring[Cfg<1, HD>::kBatch][kBlock * HD];
    uint16_t v[kBlock * v_stride_b(HD)];
    uint16_t qs[kBlock * q_stride_b(HD)];
};
template <int HD> struct StageBuf<0, HD> {
    float v[kBlock * v_stride_f(HD)];
};

// The attention kernel's dynamic LDS: kWaves StageBufs.  The direct loads
// address it through this symbol, so that the compiler sees they write LDS
// only (and can keep a batch's register slots in registers).
extern __shared__ __align__(16) unsigned char attn_smem[];

// Full mode keeps one low-res value per channel in lanes: channel lane + 64 x,
// x < HD / 64.
template <int DT, int HD>
struct Slot {
    u32x4 k[Cfg<DT, HD>::kKDirect ? 1 : Cfg<DT, HD>::kKV];   // (unused when K goes straight to LDS)
    u32x4 v[Cfg<DT, HD>::kKV];
    u32x4 q[Cfg<DT, HD>::kKV];   // Q of the block's row
    uint32_t qm;                 // and its mask word (segment's first block)
    float vh[HD / 64];           // full mode: vhat_j at this lane's channels
    float lo[HD / 64];           // full mode: lo_all_i at this lane's channels (segment's first block)
};

template <int DT, int HD>
struct Wave {
    // record window: lane t holds the record of block a + t, and in full mode
    // the low-res row max and weight sum of that block's row
    uint32_t wij, wk, winfo;
    float ww, wm, wll;
    int a;
    int bh, b, nb, lane, n, h;
    int wave;                // the wave's index in its workgroup (its StageBuf)
    const typename Cfg<DT, HD>::Elem* Qg;
    const typename Cfg<DT, HD>::Elem* Kg;
    const typename Cfg<DT, HD>::Elem* Vg;
};

// Issue the loads of stream block e into a batch slot: K_j, V_j, vhat_j at
// this lane's channel (full mode), and when the block starts a segment Q_i,
// the mask word of row i and lo_all_i at this lane's channel (full mode).
__device__ __forceinline__ int rec_i(uint32_t ij) { return (int)(ij & 0xFFFFu); }
__device__ __forceinline__ int rec_j(uint32_t ij) { return (int)(ij >> 16); }

template <int DT, int HD, bool FULL>
__device__ __forceinline__ void issue(const Params& p, const Wave<DT, HD>& W, int e, Slot<DT, HD>& s,
                                      StageBuf<DT, HD>& sb, int u) {
    constexpr int kKV = Cfg<DT, HD>::kKV;
    const int we = e - W.a;
    const uint32_t ij = (uint32_t)rl((int)W.wij, we);
    const int i = min(rec_i(ij), W.nb - 1);
    const int j = min(rec_j(ij), W.nb - 1);
    const int lane = W.lane, n = W.n, h = W.h;
    if constexpr (DT == 1) {
        constexpr int kRowLanes = HD / 8;           // lanes per 2 HD-byte token row
        constexpr int kRowsPerLoad = 64 / kRowLanes;
        const uint16_t* Kb = W.Kg + (size_t)j * kBlock * HD;
        const uint16_t* Vb = W.Vg + (size_t)j * kBlock * HD;
        const uint16_t* Qb = W.Qg + (size_t)i * kBlock * HD;
        const int off = (lane / kRowLanes) * HD + (lane % kRowLanes) * 8;
        // K_j straight into LDS slot u, 1 KiB (whole token rows) per load:
        // lane l fetches the chunk that belongs at its LDS position (a load
        // of every row's 32-byte operand piece instead would cost the
        // address unit several times more)
        typedef __attribute__((address_space(3))) void lds_void;
        using SB = StageBuf<1, HD>;
        const size_t kbase = (size_t)W.wave * sizeof(SB) + offsetof(SB, kring) + (size_t)u * sizeof(sb.kring[0]);
#pragma unroll
        for (int x = 0; x < kKV; x++) {
            const int r = kRowsPerLoad * x + lane / kRowLanes, pos = lane % kRowLanes;
            const int c = (pos ^ swz_key<HD>(r)) & (kRowLanes - 1);   // the chunk k_swz puts at pos
            __builtin_amdgcn_global_load_lds(Kb + r * HD + 8 * c, (lds_void*)(attn_smem + kbase + x * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < kKV; x++) s.v[x] = *reinterpret_cast<const u32x4*>(Vb + off + kRowsPerLoad * x * HD);
        // V_j and Q_i: whole token rows per HD / 8 lanes, so every load is
        // full cache lines; Q_i once per segment, by its first block (the
        // other blocks leave s.q unset: only a segment's first block reads it)
        if (info_pos((uint32_t)rl((int)W.winfo, we)) == 0) {
#pragma unroll
            for (int x = 0; x < kKV; x++) s.q[x] = *reinterpret_cast<const u32x4*>(Qb + off + kRowsPerLoad * x * HD);
        }
    } else {
        // lane l: token l % 32, channels HD / 2 * (l / 32) .. + HD / 2 - 1 of K and Q
        const float* Kb = W.Kg + (size_t)j * kBlock * HD;
        const float* Vb = W.Vg + (size_t)j * kBlock * HD;
        const float* Qb = W.Qg + (size_t)i * kBlock * HD;
#pragma unroll
        for (int c4 = 0; c4 < kKV; c4++)
            s.k[c4] = *reinterpret_cast<const u32x4*>(Kb + n * HD + (HD / 2) * h + 4 * c4);
        constexpr int kRowLanes = HD / 4;           // lanes per fp32 token row
        constexpr int kRowsPerLoad = 64 / kRowLanes;
#pragma unroll
        for (int x = 0; x < kKV; x++)
            s.v[x] = *reinterpret_cast<const u32x4*>(Vb + (lane / kRowLanes + kRowsPerLoad * x) * HD +
                                                      (lane % kRowLanes) * 4);
#pragma unroll
        for (int c4 = 0; c4 < kKV; c4++)
            s.q[c4] = *reinterpret_cast<const u32x4*>(Qb + n * HD + (HD / 2) * h + 4 * c4);
    }
    // once per segment, by its first block: the row's mask word (uniform, so
    // through the scalar cache) and in full mode lo_all_i; every block: vhat_j
    typedef __attribute__((address_space(4))) const uint32_t const_u32;
    if (info_pos((uint32_t)rl((int)W.winfo, we)) == 0) {
        s.qm = *reinterpret_cast<const_u32*>((uintptr_t)(p.mbits + (size_t)W.b * W.nb + i));
        if constexpr (FULL) {
#pragma unroll
            for (int x = 0; x < HD / 64; x++) s.lo[x] = p.lo_all[((size_t)W.bh * W.nb + i) * HD + lane + 64 * x];
        }
    } else {
        s.qm = 0u;
#pragma unroll
        for (int x = 0; x < HD / 64; x++) s.lo[x] = 0.f;
    }
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < HD / 64; x++) s.vh[x] = p.vhat[((size_t)W.bh * W.nb + j) * HD + lane + 64 * x];
    }
}

template <int DT, int HD>
struct Acc {
    f32x16 o[HD / 32];    // O^T, 32 channels per tile
    float mrun, lsum;
    float corr[HD / 64];  // full mode: sum over the segment's blocks of w vhat_j at this lane's channels
    float sw;             // full mode: sum of their weights w
    float lo[HD / 64];    // full mode: lo_all_i at this lane's channels
    uint32_t qm;          // valid-token mask word of the segment's row
};

// Finish a segment: a whole row writes its output, otherwise a partial.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void finish_segment(const Params& p, const Wave<DT, HD>& W, const Acc<DT, HD>& A, int we,
                                               int i, uint32_t info, float* lo_lds) {
    const int n = W.n, h = W.h;
    const float ltot = A.lsum + __shfl_xor(A.lsum, 32, 64);
    const int tok = i * kBlock + n;
    if (info_whole(info)) {
        const bool valid = (A.qm >> n) & 1u;
        float a = 1.f, bw = 0.f, den = ltot;
        float Mu = A.mrun;   // the max that den and the probabilities are relative to
        if constexpr (FULL) {
            // low-res part of the row without the selected blocks, one channel per lane
#pragma unroll
            for (int x = 0; x < HD / 64; x++) lo_lds[W.lane + 64 * x] = A.lo[x] - A.corr[x];
            const float mi2 = __int_as_float(rl(__float_as_int(W.wm), we)) * kLog2e;
            const float ll = fmaxf(__int_as_float(rl(__float_as_int(W.wll), we)) - A.sw, 0.f);
            const float M = fmaxf(A.mrun, mi2);
            a = M == -__builtin_inff() ? 0.f : fast_exp2(A.mrun - M);
            bw = M == -__builtin_inff() ? 0.f : fast_exp2(mi2 - M);
            den = ltot * a + ll * bw;
            Mu = M;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
        const float sa = a * inv, sb = bw * inv;
        if (h == 0 && p.save_stats) {   // the token's softmax statistics, for the backward pass
            const size_t st = (size_t)W.bh * p.N + tok;
            p.st_m[st] = Mu == -__builtin_inff() ? 0.f : Mu;
            p.st_linv[st] = inv;
        }
        const size_t orow = ((size_t)W.bh * p.N + tok) * HD;
#pragma unroll
        for (int mt = 0; mt < HD / 32; mt++) {
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int d0 = 32 * mt + 8 * gq + 4 * h;
                const f32x16& oo = A.o[mt];
                float v0 = oo[4 * gq] * sa, v1 = oo[4 * gq + 1] * sa;
                float v2 = oo[4 * gq + 2] * sa, v3 = oo[4 * gq + 3] * sa;
                if constexpr (FULL) {
                    const float4 lo = *reinterpret_cast<const float4*>(lo_lds + d0);
                    v0 = __builtin_fmaf(lo.x, sb, v0);
                    v1 = __builtin_fmaf(lo.y, sb, v1);
                    v2 = __builtin_fmaf(lo.z, sb, v2);
                    v3 = __builtin_fmaf(lo.w, sb, v3);
                }
                if constexpr (DT == 1) {
                    uint2 pk;
                    pk.x = (uint32_t)float_to_bf16(v0) | ((uint32_t)float_to_bf16(v1) << 16);
                    pk.y = (uint32_t)float_to_bf16(v2) | ((uint32_t)float_to_bf16(v3) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + d0) = pk;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + d0) = make_float4(v0, v1, v2, v3);
                }
            }
        }
    } else {
        const size_t pidx = (size_t)W.bh * p.max_items + min(info_item(info), p.max_items - 1);
        float* po = p.part_o + (pidx * kBlock + n) * HD;
#pragma unroll
        for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
            for (int gq = 0; gq < 4; gq++) {
                const int d0 = 32 * mt + 8 * gq + 4 * h;
                const f32x16& oo = A.o[mt];
                *reinterpret_cast<float4*>(po + d0) = make_float4(oo[4 * gq], oo[4 * gq + 1], oo[4 * gq + 2], oo[4 * gq + 3]);
            }
        if (h == 0) {
            p.part_ml[pidx * 64 + n] = A.mrun;
            p.part_ml[pidx * 64 + 32 + n] = ltot;
        }
        if constexpr (FULL) {   // the segment's share of the low-res correction
            float* pc = p.part_corr + pidx * corr_stride(HD);
#pragma unroll
            for (int x = 0; x < HD / 64; x++) pc[W.lane + 64 * x] = A.corr[x];
            if (W.lane == 0) pc[HD] = A.sw;
        }
    }
}

// One block of the stream: S^T, online softmax, O^T += V^T P^T.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void process(const Params& p, const Wave<DT, HD>& W, int e, Slot<DT, HD>& s,
                                        Acc<DT, HD>& A, StageBuf<DT, HD>& sb, int u, float scale2) {
    constexpr int kKV = Cfg<DT, HD>::kKV;
    auto* vs = sb.v;
    const int we = e - W.a;
    const int i = min(rec_i((uint32_t)rl((int)W.wij, we)), W.nb - 1);
    const uint32_t kb = (uint32_t)rl((int)W.wk, we);
    const uint32_t info = (uint32_t)rl((int)W.winfo, we);
    const int lane = W.lane, n = W.n, h = W.h;
    if (info_pos(info) == 0) {   // a segment starts: alpha = 0 below clears O and l
        A.mrun = -__builtin_inff();
        A.qm = s.qm;
        if constexpr (FULL) {
#pragma unroll
            for (int x = 0; x < HD / 64; x++) {
                A.corr[x] = 0.f;
                A.lo[x] = s.lo[x];
            }
            A.sw = 0.f;
        }
    }
    if constexpr (FULL) {
        const float w = __int_as_float(rl(__float_as_int(W.ww), we));
#pragma unroll
        for (int x = 0; x < HD / 64; x++) A.corr[x] = __builtin_fmaf(w, s.vh[x], A.corr[x]);
        A.sw += w;
    }
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; r++) S[r] = 0.f;
    if constexpr (DT == 1) {
        // stage V_j (and Q_i when the segment starts) in this wave's LDS
        // region; K_j (already in slot u) and Q are read back one token row
        // per lane (the MFMA operand layout: lane l holds token l % 32,
        // channels 16 kc + 8 (l / 32))
        constexpr int kRowLanes = HD / 8, kRowsPerLoad = 64 / kRowLanes;
        constexpr int VS = v_stride_b(HD), QS = q_stride_b(HD);
        uint16_t* qs = sb.qs;
        const int r0 = lane / kRowLanes, c0 = (lane % kRowLanes) * 8;
#pragma unroll
        for (int x = 0; x < kKV; x++)
            *reinterpret_cast<u32x4*>(vs + (r0 + kRowsPerLoad * x) * VS + c0) = s.v[x];
        if (info_pos(info) == 0) {
#pragma unroll
            for (int x = 0; x < kKV; x++)
                *reinterpret_cast<u32x4*>(qs + (r0 + kRowsPerLoad * x) * QS + c0) = s.q[x];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int kc = 0; kc < HD / 16; kc++) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(sb.kring[u] + k_swz<HD>(n, 2 * kc + h));
            const u32x4 qa = *reinterpret_cast<const u32x4*>(qs + n * QS + 16 * kc + 8 * h);
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka), as_bf16x8(qa), S, 0, 0, 0);
        }
    } else {
        constexpr int kRowLanes = HD / 4, kRowsPerLoad = 64 / kRowLanes;
        constexpr int VS = v_stride_f(HD);
#pragma unroll
        for (int x = 0; x < kKV; x++)
            *reinterpret_cast<u32x4*>(vs + (lane / kRowLanes + kRowsPerLoad * x) * VS + (lane % kRowLanes) * 4) =
                s.v[x];
#pragma unroll
        for (int c4 = 0; c4 < kKV; c4++) {
            const float4 kf = __builtin_bit_cast(float4, s.k[c4]);
            const float4 qf = __builtin_bit_cast(float4, s.q[c4]);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qf.x, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qf.y, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qf.z, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qf.w, S, 0, 0, 0);
        }
    }
    // online softmax in log2 units: max over the 32 keys of each query row
    float bm = -__builtin_inff();
    if (kb == 0xFFFFFFFFu) {
#pragma unroll
        for (int r = 0; r < 16; r++) bm = fmaxf(bm, S[r]);
    } else {
#pragma unroll
        for (int r = 0; r < 16; r++) {
            S[r] = ((kb >> acc_row(r, lane)) & 1u) ? S[r] : -__builtin_inff();
            bm = fmaxf(bm, S[r]);
        }
    }
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64)) * scale2;
    // The running max moves only when a block's max exceeds it by more than
    // kLazyMax (log2 units), so most blocks keep alpha = 1 and skip the
    // rescale of O; the probabilities then stay below 2^kLazyMax.  O and l are
    // both relative to the max in use, so the result does not change.
    const float mnew = bm > A.mrun + kLazyMax ? bm : A.mrun;
    const float muse = mnew == -__builtin_inff() ? 0.f : mnew;
    const float alpha = fast_exp2(A.mrun - muse);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        S[r] = fast_exp2(__builtin_fmaf(S[r], scale2, -muse));
        ps += S[r];
    }
    A.lsum = A.lsum * alpha + ps;
    A.mrun = mnew;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
            for (int r = 0; r < 16; r++) A.o[mt][r] *= alpha;
    }
    // the LDS writes above precede these reads in the wave's in-order LDS queue
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (DT == 1) {
        bf16x8 pb[2];
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++)
#pragma unroll
            for (int x = 0; x < 8; x++) pb[kc2][x] = static_cast<__bf16>(S[8 * kc2 + x]);
        // O^T += V_j^T P^T ; A operand read transposed from LDS
        const int g16 = lane >> 4, s16 = lane & 15;
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++) {
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++) {
                constexpr int VS = v_stride_b(HD);
                const int col = 32 * mt + 16 * (g16 & 1) + 4 * (s16 & 3);
                const int row = 16 * kc2 + 4 * h + (s16 >> 2);
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + row * VS + col));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vs + (row + 8) * VS + col));
                const short __attribute__((ext_vector_type(8))) a8 = {lo[0], lo[1], lo[2], lo[3],
                                                                      hi[0], hi[1], hi[2], hi[3]};
                const bf16x8 av = __builtin_bit_cast(bf16x8, a8);
                A.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[kc2], A.o[mt], 0, 0, 0);
            }
        }
    } else {
        constexpr int VS = v_stride_f(HD);
#pragma unroll
        for (int kc = 0; kc < 16; kc++) {
            const int key = (kc >> 2) * 8 + 4 * h + (kc & 3);
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++)
                A.o[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * VS + 32 * mt + n], S[kc], A.o[mt], 0, 0, 0);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (info_pos(info) == info_len(info) - 1)
        finish_segment<DT, HD, FULL>(p, W, A, we, i, info, reinterpret_cast<float*>(vs));
}


// Range k of the WPH ranges of head bh's record stream, by one wave.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void run_range(const Params& p, int bh, int k, int WPH, int lane, int wave,
                                          StageBuf<DT, HD>& sb) {
    // the head's stream: K records (a static layout fills row_ptr[nb] of its
    // capacity K)
    const int64_t K = p.attn_dyn ? min((int64_t)p.row_ptr[(size_t)bh * (p.nb + 1) + p.nb], p.K) : p.K;
    const int a = (int)((int64_t)k * K / WPH);
    const int bnd = (int)((int64_t)(k + 1) * K / WPH);
    // the record window starts half a segment before a: the range's first
    // block may move back that far
    const int a0 = max(a - kChunk / 2, 0);
    const BlkRec* R = p.recs + (size_t)bh * p.K;
    Wave<DT, HD> W;
    W.a = a0;
    W.bh = bh;
    W.b = bh / p.H;
    W.nb = p.nb;
    W.lane = lane;
    W.wave = wave;
    W.n = lane & 31;
    W.h = lane >> 5;
    {
        int4 r = make_int4(0, 0, 0, 0);
        if (a0 + lane < K) r = *reinterpret_cast<const int4*>(R + a0 + lane);
        W.wij = (uint32_t)r.x;
        W.wk = (uint32_t)r.y;
        W.winfo = (uint32_t)r.w;
        W.ww = 0.f;
        W.wm = 0.f;
        W.wll = 0.f;
        if (FULL && a0 + lane < K) {
            // the cell's low-res weight, formed as the low-res sums formed it
            const size_t row = (size_t)bh * p.nb + min(rec_i(W.wij), p.nb - 1);
            const float sij = p.logits[row * p.nb + min(rec_j(W.wij), p.nb - 1)];
            W.wm = p.rowmax[row];
            W.wll = p.ll_all[row];
            W.ww = lowres_weight(sij, W.wm, __popc(W.wk));
        }
    }
    const uint32_t info_b = bnd < K ? R[bnd].info : 0u;
    // Move both ends of [a, bnd) to the nearest segment start; the next
    // wave's range starts where this one ends, since both round the same
    // block index the same way.
    const int start = nearest_segment_start(a, (uint32_t)rl((int)W.winfo, a - a0), K);
    const int end = nearest_segment_start(bnd, info_b, K);
    if (start >= end) return;
    if (start < a0 || end - a0 > kWindow) {   // the window must hold every block of the range
        if (lane == 0) atomicOr(reinterpret_cast<unsigned int*>(p.error), 4u);
        return;
    }

    const size_t head_off = (size_t)bh * p.N * HD;
    using E = typename Cfg<DT, HD>::Elem;
    W.Qg = static_cast<const E*>(p.q) + head_off;
    W.Kg = static_cast<const E*>(p.k) + head_off;
    W.Vg = static_cast<const E*>(p.v) + head_off;
    const float scale2 = (1.0f / __builtin_sqrtf((float)p.dscale)) * kLog2e;

    // Blocks go in batches: the loads of a whole batch are issued, then the
    // batch is computed.  Past the end the last block is fetched again, so
    // every batch issues the same loads and the wait counts stay exact; the
    // second wave on the SIMD computes while this one waits.
    constexpr int BATCH = Cfg<DT, HD>::kBatch;
    Acc<DT, HD> A;
    A.mrun = -__builtin_inff();
    A.lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) A.o[mt][r] = 0.f;   // finite, so alpha = 0 clears them
    for (int e0 = start; e0 < end; e0 += BATCH) {
        Slot<DT, HD> sl[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; u++) issue<DT, HD, FULL>(p, W, min(e0 + u, end - 1), sl[u], sb, u);
        // keep the loads together: the scheduler must not sink them into the
        // compute of the batch
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < BATCH; u++)
            if (e0 + u < end) process<DT, HD, FULL>(p, W, e0 + u, sl[u], A, sb, u, scale2);
    }
}

// Two workgroups per CU for 64-channel heads; one for 128-channel heads,
// whose staged blocks fill the CU's LDS and whose accumulators need the
// larger register budget.
template <int DT, int HD, bool FULL>
__global__ __launch_bounds__(kThreads, HD == 64 ? 2 : 1) void attn_kernel(Params p) {
    StageBuf<DT, HD>* stage = reinterpret_cast<StageBuf<DT, HD>*>(attn_smem);   // one per wave
    const int xcd = blockIdx.x & 7;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wx = (blockIdx.x >> 3) * kWaves + wave;      // wave index within its XCD
    const int WPH = p.attn_wph;
    if (p.attn_seq) {
        // every wave of the XCD takes range wx of each of the XCD's heads in
        // turn, so the XCD's L2 holds one head's K and V at a time
        if (wx >= WPH) return;
        for (int bh = xcd; bh < p.BH; bh += 8) run_range<DT, HD, FULL>(p, bh, wx, WPH, lane, wave, stage[wave]);
    } else {
        const int hm = wx / WPH;
        const int bh = xcd + 8 * hm;
        if (bh < p.BH) run_range<DT, HD, FULL>(p, bh, wx - hm * WPH, WPH, lane, wave, stage[wave]);
    }
}

}  // namespace

// Heads whose ranges would still hold at least this many blocks each when
// every wave of an XCD shares one head are taken in turn.
constexpr int64_t kTurnMinBlocks = 12;
constexpr int kWavesPerXcd = 256;                     // about 2048 waves on the chip

bool attn_heads_in_turn(int BH, int64_t K) {
    return (BH + 7) / 8 >= 2 && K >= kTurnMinBlocks * kWavesPerXcd;
}

int attn_grid_waves_per_head(int BH, int64_t K) {
    const int heads_per_xcd = (BH + 7) / 8;
    int64_t w = attn_heads_in_turn(BH, K) ? kWavesPerXcd : kWavesPerXcd / heads_per_xcd;
    if (w < 1) w = 1;
    const int64_t hi = (K + 1) / 2;                   // at least about two blocks a wave
    if (w > hi) w = hi;
    const int64_t lo = (K + kMaxRun - 1) / kMaxRun;    // keep each range inside one record window
    if (w < lo) w = lo;
    return (int)w;
}

// Launch one instantiation with kWaves stage buffers of dynamic LDS (bf16
// needs more than the 64 KiB of static LDS); the size attribute is set once.
template <int DT, int HD, bool FULL>
static hipError_t launch_attn_t(const Params& p, unsigned grid, hipStream_t s) {
    constexpr size_t kLds = kWaves * sizeof(StageBuf<DT, HD>);
    static const hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_kernel<DT, HD, FULL>),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
    if (a != hipSuccess) return a;
    hipLaunchKernelGGL((attn_kernel<DT, HD, FULL>), dim3(grid), dim3(kThreads), kLds, s, p);
    return hipGetLastError();
}

template <int HD>
static hipError_t launch_attn_hd(const Params& p, unsigned grid, hipStream_t s) {
    const bool full = p.mode == 0;
    if (p.dtype == 1) return full ? launch_attn_t<1, HD, true>(p, grid, s) : launch_attn_t<1, HD, false>(p, grid, s);
    return full ? launch_attn_t<0, HD, true>(p, grid, s) : launch_attn_t<0, HD, false>(p, grid, s);
}

hipError_t launch_attn(const Params& p, hipStream_t s) {
    const int heads_per_xcd = (p.BH + 7) / 8;
    const int64_t waves_per_xcd = p.attn_seq ? p.attn_wph : (int64_t)heads_per_xcd * p.attn_wph;
    const unsigned grid = (unsigned)(8 * ((waves_per_xcd + kWaves - 1) / kWaves));
    if (p.d == 64) return launch_attn_hd<64>(p, grid, s);
    if (p.d == 128) return launch_attn_hd<128>(p, grid, s);
    return hipErrorInvalidValue;
}

}  // namespace mra
