// mra_attn.hip — step 3 ([MRA] "第三步"): exact softmax attention on the
// selected 32x32 blocks, i.e. what the pages' sampled dense matmul, row max,
// sparse-dense matmul and reduce-sum do, in one pass with an online row max.
//
// Work decomposition: the selector lists every selected block of a head in
// CSR order (block row, then key block); a row longer than p.seg_whole
// blocks is cut into segments of p.chunk blocks (both chosen at launch from
// the workgroups' share of the head).  The G workgroups of a head split that list into G
// ranges of about K/G blocks, each moved to the nearest segment start, and
// the kWaves waves of a workgroup split its range exactly into kWaves equal
// parts, wherever those cuts fall: every wave gets the same number of blocks
// whatever the row lengths.  A segment cut between two waves is finished by
// the wave holding its first block, after the workgroup's one barrier, from
// its own accumulators and the pieces the next waves parked (see below).
// A wave streams through its blocks one at a time: each block stages its K,
// V (and Q) in LDS and then issues the next block's loads, which arrive
// while it is computed; the other wave on the SIMD computes meanwhile.
//
// Per key block j of a segment of query block row i:
//   S^T = K_j Q_i^T           4 x MFMA 32x32x16 bf16 (fp32: 32 x 32x32x2 f32);
//                             bf16 K_j is loaded as whole rows, stored in LDS
//                             and read back in the operand layout
//   online max / exp2 / sum   in registers: lane l holds query l%32 and 16 of
//                             its 32 keys, so row reductions need one swap
//                             between the two halves of the wave
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
// the last of them joins.
//
// Joins without a separate kernel, at two levels:
//   * within a workgroup: a wave whose part starts inside a segment parks
//     its piece of it (O, running max, sum, and in full mode its sums of
//     w vhat_j and of w) in its slot with plain stores; after the barrier
//     the wave holding the segment's first block adds the parked pieces of
//     the next waves to its own and finishes the segment as if it had done
//     it alone;
//   * across workgroups: a row cut into several segments (only rows longer
//     than p.seg_whole blocks) is joined by the wave that ends its last segment
//     to arrive.  Every segment of a cut row stores its partials with
//     agent-scope (write-through) stores; after its part, the wave waits for
//     them to complete and adds one to each such row's counter; the wave
//     that completes a count reads the partials back with agent-scope loads,
//     writes the row and sets the counter back to zero.  Only these partials
//     take the coherent path, so no cache-wide writeback is needed.
// Rows with no selected block are written last, listed rows k, k + W, ... by
// wave k of the head.
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
// stores (HIP's uint4 struct is copied with memcpy, which can keep a load
// slot's registers in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// staged row strides for a head of hd channels (elements)
__host__ __device__ constexpr int v_stride_b(int hd) { return hd + 16; }   // bf16 V: 16 pad, no bank conflicts
__host__ __device__ constexpr int q_stride_b(int hd) { return hd + 8; }    // bf16 Q: row r's 16-byte reads start at bank group r
__host__ __device__ constexpr int v_stride_f(int hd) { return hd + 4; }    // fp32 V
constexpr int kWindow = 64;     // block records a wave holds (one per lane)
// blocks whose loads a wave keeps in flight
template <int HD> __host__ __device__ constexpr int kSlots() { return 1; }
constexpr float kLazyMax = 8.0f;   // log2 headroom of the running max (probabilities <= 256)
// Blocks per wave, on average over a workgroup's range, at most: a
// workgroup's range grows by up to half a segment at each end when they
// move to segment starts, and each of its kWaves parts must fit the window
// (the launch keeps the segment lengths within what this leaves).
constexpr int kMaxRun = (kWaves * kWindow - 2 * kChunkMin - 2 * kWaves) / kWaves;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ int rl(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
// x combined with its value in lane l ^ 32, by one lane swap between the two
// halves of the wave (lanes l < 32 hold the lower operand of the pair in the
// swap's first result, so both halves combine the pair in the same order)
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
    static constexpr int kKV = HD / 16;     // 16-byte pieces per lane for one K, V or Q block
    using Elem = uint16_t;
};
template <int HD> struct Cfg<0, HD> {       // fp32: twice the registers per block
    static constexpr int kKV = HD / 8;
    using Elem = float;
};

// bf16 K block in LDS: 32 token rows of 2 HD bytes, the 16-byte chunk c of
// row r at a swizzled position of the row: c ^ ((r / 2) mod 8) for 128-byte
// rows, c ^ (r mod 16) for 256-byte ones.  K is loaded as whole rows (full
// cache lines) and stored so, and the MFMA operand reads (lane: one row, one
// chunk) then hit distinct banks in each 16-lane phase.  (Loads straight
// into LDS would save the registers, but the compiler then drains every
// load in flight before each LDS access, which serialises the blocks.)
template <int HD>
__device__ __forceinline__ int swz_key(int row) { return HD == 64 ? row >> 1 : row; }
template <int HD>
__device__ __forceinline__ int k_swz(int row, int chunk) {
    return row * HD + ((chunk ^ swz_key<HD>(row)) & (HD / 8 - 1)) * 8;
}

// Per-wave LDS.  bf16: K_j (k_swz), V_j (read back transposed) and Q_i;
// fp32: V_j.
template <int DT, int HD> struct StageBuf;
template <int HD> struct StageBuf<1, HD> {
    uint16_t k[kBlock * HD];
    uint16_t v[kBlock * v_stride_b(HD)];
    uint16_t qs[kBlock * q_stride_b(HD)];
    int pend[kWindow];   // rows of the cut segments this wave ended, counted after its range
};
template <int HD> struct StageBuf<0, HD> {
    float v[kBlock * v_stride_f(HD)];
    int pend[kWindow];
};

// The attention kernel's dynamic LDS: kWaves StageBufs.
extern __shared__ __align__(16) unsigned char attn_smem[];

// Full mode keeps one low-res value per channel in lanes: channel lane + 64 x,
// x < HD / 64.
template <int DT, int HD>
struct Slot {
    u32x4 k[Cfg<DT, HD>::kKV];
    u32x4 v[Cfg<DT, HD>::kKV];
    u32x4 q[Cfg<DT, HD>::kKV];   // Q of the block's row
    uint32_t qm;                 // and its mask word
    float vh[HD / 64];           // full mode: vhat_j at this lane's channels
    float lo[HD / 64];           // full mode: lo_all_i at this lane's channels (segment's first block)
};

template <int DT, int HD>
struct Wave {
    // record window: lane t holds the record of block a + t, and in full mode
    // the low-res row max and weight sum of that block's row
    uint32_t wij, wk, winfo;
    float ww, wm, wll;       // full mode: the cell's low-res weight, its row's max and weight sum
    int a;                   // first block of the window (= start)
    int start, end;          // the wave's blocks [start, end)
    float* park;             // the wave's slot for a piece of a segment that another wave finishes
    int bh, b, nb, lane, n, h;
    int wave;                // the wave's index in its workgroup (its StageBuf)
    const typename Cfg<DT, HD>::Elem* Qg;
    const typename Cfg<DT, HD>::Elem* Kg;
    const typename Cfg<DT, HD>::Elem* Vg;
};

// Issue the loads of stream block e into the load slot: K_j, V_j, Q_i, the
// mask word of row i, and in full mode vhat_j and lo_all_i at this lane's
// channel.
__device__ __forceinline__ int rec_i(uint32_t ij) { return (int)(ij & 0xFFFFu); }
__device__ __forceinline__ int rec_j(uint32_t ij) { return (int)(ij >> 16); }

template <int DT, int HD, bool FULL>
__device__ __forceinline__ void issue(const Params& p, const Wave<DT, HD>& W, int e, Slot<DT, HD>& s,
                                      StageBuf<DT, HD>& sb) {
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
        // K_j and V_j: whole token rows per HD / 8 lanes, 1 KiB per load (a
        // load of every row's 32-byte operand piece instead would cost the
        // address unit several times more)
#pragma unroll
        for (int x = 0; x < kKV; x++) s.k[x] = *reinterpret_cast<const u32x4*>(Kb + off + kRowsPerLoad * x * HD);
#pragma unroll
        for (int x = 0; x < kKV; x++) s.v[x] = *reinterpret_cast<const u32x4*>(Vb + off + kRowsPerLoad * x * HD);
        // Q_i likewise.  Every block loads Q_i (only a piece's first
        // block stages it; the others hit the cache): with the same loads for
        // every block the waits for a slot's data count exactly, rather than
        // draining every load in flight at each piece start.
#pragma unroll
        for (int x = 0; x < kKV; x++) s.q[x] = *reinterpret_cast<const u32x4*>(Qb + off + kRowsPerLoad * x * HD);
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
    // every block, for the same reason: the row's mask word (a vector load,
    // so that it joins the same count), in full mode lo_all_i and vhat_j
    s.qm = p.mbits[(size_t)W.b * W.nb + i];
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < HD / 64; x++) s.lo[x] = p.lo_all[((size_t)W.bh * W.nb + i) * HD + lane + 64 * x];
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
    int npend;            // entries of the wave's pending-join list
    int jend;             // >= 0: the piece held at the end of the range belongs to a segment that
                          //   goes on into the next waves and ends at stream block jend
};

// Partials of cut rows go through agent-scope (coherent, write-through)
// stores and loads, so that whichever wave joins the row sees them.
__device__ __forceinline__ void store4_coherent(float* dst, float a, float b, float c, float d) {
    uint64_t* q = reinterpret_cast<uint64_t*>(dst);
    const uint64_t lo = (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(c) | ((uint64_t)__float_as_uint(d) << 32);
    __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(float* dst, float v) {
    __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* src) {
    return __hip_atomic_load(const_cast<float*>(src), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4 load4_coherent(const float* src) {
    uint64_t* q = reinterpret_cast<uint64_t*>(const_cast<float*>(src));
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float4(__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                       __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32)));
}

// Write block row i of head W.bh from nseg segment partials (items first ..
// first + nseg - 1), and in full mode the row's low-resolution part
// ([MRA] "第四步"), per query token t with M the largest of the maxima:
//   out_t = (sum_c O_c 2^(m_c - M) + lo 2^(m_i log2e - M))
//         / (sum_c l_c 2^(m_c - M) + ll 2^(m_i log2e - M)),
//   lo = lo_all_i - sum_c corr_c,  ll = ll_all_i - sum_c sw_c;
// 0 when the denominator is 0 or the token is padding.  nseg = 0 is a row
// with no selected block.  Lane l holds token l % 32 and the channels of the
// attention accumulators' layout; lo_lds: HD floats of the wave's LDS.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void join_row(const Params& p, int bh, int b, int nb, int lane, int i, int first, int nseg,
                                      float* lo_lds) {
    constexpr int kSeg = HD == 64 ? 2 : 1;   // segments whose loads are in flight together
    const int n = lane & 31, h = lane >> 5;
    const size_t pbase = (size_t)bh * p.max_items;
    const size_t row = (size_t)bh * nb + i;
    // the row's own inputs, loaded with the first segments' partials
    const uint32_t qm = p.mbits[(size_t)b * nb + i];
    float lo_in[HD / 64], ll_in = 0.f, mrow = 0.f;
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < HD / 64; x++) lo_in[x] = p.lo_all[row * HD + lane + 64 * x];
        ll_in = p.ll_all[row];
        mrow = p.rowmax[row];
    }
    float M = -__builtin_inff(), den = 0.f, sw = 0.f;
    float acc[HD / 2], corr[HD / 64];
#pragma unroll
    for (int e = 0; e < HD / 2; e++) acc[e] = 0.f;
#pragma unroll
    for (int x = 0; x < HD / 64; x++) corr[x] = 0.f;
    for (int c0 = 0; c0 < nseg; c0 += kSeg) {
        float mc[kSeg], lc[kSeg];
        float4 oc[kSeg][HD / 8];
#pragma unroll
        for (int c = 0; c < kSeg; c++) {
            const bool ok = c0 + c < nseg;
            const size_t pidx = pbase + (size_t)min(first + (ok ? c0 + c : 0), p.max_items - 1);
            mc[c] = ok ? load_coherent(p.part_ml + pidx * 64 + n) : -__builtin_inff();
            lc[c] = ok ? load_coherent(p.part_ml + pidx * 64 + 32 + n) : 0.f;
            const float* po = p.part_o + (pidx * kBlock + n) * HD;
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++)
                    oc[c][mt * 4 + gq] = ok ? load4_coherent(po + 32 * mt + 8 * gq + 4 * h)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (FULL) {
                if (ok) {
                    const float* pc = p.part_corr + pidx * corr_stride(HD);
#pragma unroll
                    for (int x = 0; x < HD / 64; x++) corr[x] += load_coherent(pc + lane + 64 * x);
                    sw += load_coherent(pc + HD);
                }
            }
        }
        float Mb = M;
#pragma unroll
        for (int c = 0; c < kSeg; c++) Mb = fmaxf(Mb, mc[c]);
        if (Mb != -__builtin_inff()) {
            const float sM = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
            den *= sM;
#pragma unroll
            for (int e = 0; e < HD / 2; e++) acc[e] *= sM;
#pragma unroll
            for (int c = 0; c < kSeg; c++) {
                const float f = mc[c] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(mc[c] - Mb);
                den += lc[c] * f;
#pragma unroll
                for (int x = 0; x < HD / 8; x++) {
                    acc[4 * x] += oc[c][x].x * f;
                    acc[4 * x + 1] += oc[c][x].y * f;
                    acc[4 * x + 2] += oc[c][x].z * f;
                    acc[4 * x + 3] += oc[c][x].w * f;
                }
            }
            M = Mb;
        }
    }
    float Mu = M;   // the max that den and the probabilities are relative to
    if constexpr (FULL) {
        // the row's low-res part: lo_all minus the segments' corrections, one channel per lane
#pragma unroll
        for (int x = 0; x < HD / 64; x++) lo_lds[lane + 64 * x] = lo_in[x] - corr[x];
        const float ll = fmaxf(ll_in - sw, 0.f), mi2 = mrow * kLog2e;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float Mf = fmaxf(M, mi2);
        if (Mf != -__builtin_inff()) {
            const float sM = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(M - Mf);
            const float f = __builtin_amdgcn_exp2f(mi2 - Mf);
            den = den * sM + ll * f;
            Mu = Mf;
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    const float4 lo = *reinterpret_cast<const float4*>(lo_lds + 32 * mt + 8 * gq + 4 * h);
                    float* a = acc + 4 * (mt * 4 + gq);
                    a[0] = a[0] * sM + lo.x * f;
                    a[1] = a[1] * sM + lo.y * f;
                    a[2] = a[2] * sM + lo.z * f;
                    a[3] = a[3] * sM + lo.w * f;
                }
        }
    }
    const bool valid = (qm >> n) & 1u;
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    const int tok = i * kBlock + n;
    if (h == 0 && p.save_stats) {   // the token's softmax statistics, for the backward pass
        const size_t st = (size_t)bh * p.N + tok;
        p.st_m[st] = Mu == -__builtin_inff() ? 0.f : Mu;
        p.st_linv[st] = inv;
    }
    const size_t orow = ((size_t)bh * p.N + tok) * HD;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const int d0 = 32 * mt + 8 * gq + 4 * h;
            const float* a = acc + 4 * (mt * 4 + gq);
            if constexpr (DT == 1) {
                uint2 pk;
                pk.x = pack_bf16x2(a[0] * inv, a[1] * inv);
                pk.y = pack_bf16x2(a[2] * inv, a[3] * inv);
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + d0) = pk;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow + d0) =
                    make_float4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
            }
        }
}

// Tokens 8 part .. 8 part + 7 of block row i, cut into nseg segments (items
// first .. first + nseg - 1), joined from the segments' partials as
// join_row does, by one wave of the workgroup that joins the row (the
// workgroup's four waves take a quarter of the tokens each).  Lane l takes
// token 8 part + l / 8 and the HD / 8 channels from (l % 8) HD / 8, so a
// lane holds only HD / 8 values of a segment and kSeg segments' loads are in
// flight together.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void join_part(const Params& p, int bh, int b, int nb, int lane, int part, int i, int first,
                                          int nseg) {
    constexpr int kCh = HD / 8, kF4 = kCh / 4;
    constexpr int kSeg = (HD == 64 ? 8 : 4) / (DT == 1 ? 1 : 2);   // fp32: the registers are scarcer
    const int t = part * 8 + (lane >> 3), c0 = (lane & 7) * kCh;
    const size_t pbase = (size_t)bh * p.max_items;
    const size_t row = (size_t)bh * nb + i;
    const uint32_t qm = p.mbits[(size_t)b * nb + i];
    float lo_in[kCh], ll_in = 0.f, mrow = 0.f;
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < kF4; x++) {
            const float4 v = *reinterpret_cast<const float4*>(p.lo_all + row * HD + c0 + 4 * x);
            lo_in[4 * x] = v.x; lo_in[4 * x + 1] = v.y; lo_in[4 * x + 2] = v.z; lo_in[4 * x + 3] = v.w;
        }
        ll_in = p.ll_all[row];
        mrow = p.rowmax[row];
    }
    float M = -__builtin_inff(), den = 0.f, sw = 0.f, acc[kCh], corr[kCh];
#pragma unroll
    for (int e = 0; e < kCh; e++) acc[e] = corr[e] = 0.f;
    for (int c0s = 0; c0s < nseg; c0s += kSeg) {
        float mc[kSeg], lc[kSeg];
        float4 oc[kSeg][kF4];
#pragma unroll
        for (int c = 0; c < kSeg; c++) {
            const bool ok = c0s + c < nseg;
            const size_t pidx = pbase + (size_t)min(first + (ok ? c0s + c : 0), p.max_items - 1);
            mc[c] = ok ? load_coherent(p.part_ml + pidx * 64 + t) : -__builtin_inff();
            lc[c] = ok ? load_coherent(p.part_ml + pidx * 64 + 32 + t) : 0.f;
#pragma unroll
            for (int x = 0; x < kF4; x++)
                oc[c][x] = ok ? load4_coherent(p.part_o + (pidx * kBlock + t) * HD + c0 + 4 * x)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            if constexpr (FULL) {
                if (ok) {
                    const float* pc = p.part_corr + pidx * corr_stride(HD);
#pragma unroll
                    for (int x = 0; x < kF4; x++) {
                        const float4 v = load4_coherent(pc + c0 + 4 * x);
                        corr[4 * x] += v.x; corr[4 * x + 1] += v.y; corr[4 * x + 2] += v.z; corr[4 * x + 3] += v.w;
                    }
                    sw += load_coherent(pc + HD);
                }
            }
        }
        float Mb = M;
#pragma unroll
        for (int c = 0; c < kSeg; c++) Mb = fmaxf(Mb, mc[c]);
        if (Mb != -__builtin_inff()) {
            const float sM = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mb);
            den *= sM;
#pragma unroll
            for (int e = 0; e < kCh; e++) acc[e] *= sM;
#pragma unroll
            for (int c = 0; c < kSeg; c++) {
                const float f = mc[c] == -__builtin_inff() ? 0.f : fast_exp2(mc[c] - Mb);
                den += lc[c] * f;
#pragma unroll
                for (int x = 0; x < kF4; x++) {
                    acc[4 * x] += oc[c][x].x * f;
                    acc[4 * x + 1] += oc[c][x].y * f;
                    acc[4 * x + 2] += oc[c][x].z * f;
                    acc[4 * x + 3] += oc[c][x].w * f;
                }
            }
            M = Mb;
        }
    }
    float Mu = M;   // the max that den and the probabilities are relative to
    if constexpr (FULL) {
        // the row's low-res part: lo_all minus the segments' corrections
        const float ll = fmaxf(ll_in - sw, 0.f), mi2 = mrow * kLog2e;
        const float Mf = fmaxf(M, mi2);
        if (Mf != -__builtin_inff()) {
            const float sM = M == -__builtin_inff() ? 0.f : fast_exp2(M - Mf);
            const float f = fast_exp2(mi2 - Mf);
            den = den * sM + ll * f;
            Mu = Mf;
#pragma unroll
            for (int e = 0; e < kCh; e++) acc[e] = acc[e] * sM + (lo_in[e] - corr[e]) * f;
        }
    }
    const bool valid = (qm >> t) & 1u;
    const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
    const int tok = i * kBlock + t;
    if ((lane & 7) == 0 && p.save_stats) {   // the token's softmax statistics, for the backward pass
        const size_t st = (size_t)bh * p.N + tok;
        p.st_m[st] = Mu == -__builtin_inff() ? 0.f : Mu;
        p.st_linv[st] = inv;
    }
    const size_t orow = ((size_t)bh * p.N + tok) * HD + c0;
    if constexpr (DT == 1) {
#pragma unroll
        for (int x = 0; x < kCh / 8; x++) {
            uint4 pk;
            pk.x = pack_bf16x2(acc[8 * x] * inv, acc[8 * x + 1] * inv);
            pk.y = pack_bf16x2(acc[8 * x + 2] * inv, acc[8 * x + 3] * inv);
            pk.z = pack_bf16x2(acc[8 * x + 4] * inv, acc[8 * x + 5] * inv);
            pk.w = pack_bf16x2(acc[8 * x + 6] * inv, acc[8 * x + 7] * inv);
            reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + orow)[x] = pk;
        }
    } else {
#pragma unroll
        for (int x = 0; x < kF4; x++)
            reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow)[x] =
                make_float4(acc[4 * x] * inv, acc[4 * x + 1] * inv, acc[4 * x + 2] * inv, acc[4 * x + 3] * inv);
    }
}

// Finish a segment: a whole row writes its output, otherwise a partial.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void finish_segment(const Params& p, const Wave<DT, HD>& W, Acc<DT, HD>& A, int we,
                                               int i, uint32_t info, float* lo_lds, int* pend) {
    const int n = W.n, h = W.h;
    const float ltot = xhalf_sum(A.lsum);
    const int tok = i * kBlock + n;
    if (info_whole(info)) {
        const bool valid = (A.qm >> n) & 1u;
        float a = 1.f, bw = 0.f, den = ltot;
        float Mu = A.mrun;   // the max that den and the probabilities are relative to
        if constexpr (FULL) {
            const float mi2 = __int_as_float(rl(__float_as_int(W.wm), we)) * kLog2e;
            const float ll = fmaxf(__int_as_float(rl(__float_as_int(W.wll), we)) - A.sw, 0.f);
            const float M = fmaxf(A.mrun, mi2);
            a = M == -__builtin_inff() ? 0.f : fast_exp2(A.mrun - M);
            bw = M == -__builtin_inff() ? 0.f : fast_exp2(mi2 - M);
            den = ltot * a + ll * bw;
            Mu = M;
        }
        const float inv = (valid && den > 0.f) ? 1.0f / den : 0.f;
        const float sa = a * inv, sb = bw * inv;
        if (h == 0 && p.save_stats) {   // the token's softmax statistics, for the backward pass
            const size_t st = (size_t)W.bh * p.N + tok;
            p.st_m[st] = Mu == -__builtin_inff() ? 0.f : Mu;
            p.st_linv[st] = inv;
        }
        const size_t orow = ((size_t)W.bh * p.N + tok) * HD;
        if constexpr (DT == 1) {
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++) {
                f32x16 o = A.o[mt];
#pragma unroll
                for (int r = 0; r < 16; r++) o[r] *= sa;
                if constexpr (FULL) {
                    // The row's low-res part lo = lo_all - sum_sel w vhat_j
                    // (lane l holds channel l + 64 x) enters as the rank-1
                    // update lo sb^T on the matrix core: A is the tile's 32
                    // channels in lanes 0..31 (k = 0; lanes 32..63, k = 1,
                    // give 0), B is sb of the 32 tokens likewise, C the
                    // scaled O^T tile.
                    float lc = A.lo[mt / 2] - A.corr[mt / 2];
                    if (mt & 1) {   // channels 32 .. 63 of the pair: from the upper half
                        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lc), __float_as_uint(lc),
                                                                        false, false);
                        lc = __uint_as_float(r[1]);
                    }
                    o = __builtin_amdgcn_mfma_f32_32x32x2f32(W.lane < 32 ? lc : 0.f, W.lane < 32 ? sb : 0.f, o, 0, 0,
                                                             0);
                }
#pragma unroll
                for (int gq = 0; gq < 4; gq++) {
                    uint2 pk;
                    pk.x = pack_bf16x2(o[4 * gq], o[4 * gq + 1]);
                    pk.y = pack_bf16x2(o[4 * gq + 2], o[4 * gq + 3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + orow + 32 * mt + 8 * gq + 4 * h) = pk;
                }
            }
        } else {
            // fp32 (registers are scarcer here): lo goes through LDS, one
            // channel per lane in, four channels per lane out
            if constexpr (FULL) {
#pragma unroll
                for (int x = 0; x < HD / 64; x++) lo_lds[W.lane + 64 * x] = A.lo[x] - A.corr[x];
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            }
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
                store4_coherent(po + d0, oo[4 * gq], oo[4 * gq + 1], oo[4 * gq + 2], oo[4 * gq + 3]);
            }
        if (h == 0) {
            store_coherent(p.part_ml + pidx * 64 + n, A.mrun);
            store_coherent(p.part_ml + pidx * 64 + 32 + n, ltot);
        }
        if constexpr (FULL) {   // the segment's share of the low-res correction
            float* pc = p.part_corr + pidx * corr_stride(HD);
#pragma unroll
            for (int x = 0; x < HD / 64; x++) store_coherent(pc + W.lane + 64 * x, A.corr[x]);
            if (W.lane == 0) store_coherent(pc + HD, A.sw);
        }
        // counted after the range (the count's atomics and the wait for
        // these stores to complete are taken once, together)
        if (A.npend < kWindow) {   // a range of at most kWindow blocks ends at most kWindow segments
            if (W.lane == 0) pend[A.npend] = i;
            A.npend++;
        } else if (W.lane == 0) {
            atomicOr(reinterpret_cast<unsigned int*>(p.error), 4u);
        }
    }
}

// A wave's piece of a segment that another wave of the workgroup finishes,
// in its slot: O^T (float4 x of every lane together), then per lane the
// running max, the sum, and in full mode the low-res correction and weight
// sum.  Plain stores: the reader is in the same workgroup, after a barrier.
template <int HD> __host__ __device__ constexpr int park_m_off() { return 64 * (HD / 2); }
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void park_piece(const Wave<DT, HD>& W, const Acc<DT, HD>& A) {
    float4* o4 = reinterpret_cast<float4*>(W.park);
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++)
            o4[(mt * 4 + gq) * 64 + W.lane] =
                make_float4(A.o[mt][4 * gq], A.o[mt][4 * gq + 1], A.o[mt][4 * gq + 2], A.o[mt][4 * gq + 3]);
    float* t = W.park + park_m_off<HD>();
    t[W.lane] = A.mrun;
    t[64 + W.lane] = A.lsum;
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < HD / 64; x++) t[128 + 64 * x + W.lane] = A.corr[x];
        t[128 + HD + W.lane] = A.sw;
    }
}

// Add a parked piece (slot src) of the segment held in A: both are relative
// to their own running maxima, the sum to the larger of the two.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void merge_piece(const float* src, int lane, Acc<DT, HD>& A) {
    const float4* o4 = reinterpret_cast<const float4*>(src);
    float4 po[HD / 8];
#pragma unroll
    for (int x = 0; x < HD / 8; x++) po[x] = o4[x * 64 + lane];
    const float* t = src + park_m_off<HD>();
    const float mp = t[lane], lp = t[64 + lane];
    if constexpr (FULL) {
#pragma unroll
        for (int x = 0; x < HD / 64; x++) A.corr[x] += t[128 + 64 * x + lane];
        A.sw += t[128 + HD + lane];
    }
    const float M = fmaxf(A.mrun, mp);
    const float sa = A.mrun == -__builtin_inff() ? 0.f : fast_exp2(A.mrun - M);
    const float sp = mp == -__builtin_inff() ? 0.f : fast_exp2(mp - M);
    A.lsum = A.lsum * sa + lp * sp;
    A.mrun = M;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++) {
            const float4 v = po[mt * 4 + gq];
            A.o[mt][4 * gq] = A.o[mt][4 * gq] * sa + v.x * sp;
            A.o[mt][4 * gq + 1] = A.o[mt][4 * gq + 1] * sa + v.y * sp;
            A.o[mt][4 * gq + 2] = A.o[mt][4 * gq + 2] * sa + v.z * sp;
            A.o[mt][4 * gq + 3] = A.o[mt][4 * gq + 3] * sa + v.w * sp;
        }
}

// One block of the stream: S^T, online softmax, O^T += V^T P^T.  Once the
// slot's data is staged, the slot is refilled with block `next` (ISSUE).
template <int DT, int HD, bool FULL, bool ISSUE = true>
__device__ __forceinline__ void process(const Params& p, const Wave<DT, HD>& W, int e, Slot<DT, HD>& s,
                                        Acc<DT, HD>& A, StageBuf<DT, HD>& sb, float scale2, int next) {
    constexpr int kKV = Cfg<DT, HD>::kKV;
    auto* vs = sb.v;
    const int we = e - W.a;
    const int i = min(rec_i((uint32_t)rl((int)W.wij, we)), W.nb - 1);
    const uint32_t kb = (uint32_t)rl((int)W.wk, we);
    const uint32_t info = (uint32_t)rl((int)W.winfo, we);
    const int lane = W.lane, n = W.n, h = W.h;
    const bool piece_start = info_pos(info) == 0 || e == W.start;
    if (piece_start) {   // a segment (or the wave's piece of one) starts: alpha = 0 below clears O and l
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
    // The padded keys of block j enter as the accumulator's start: -inf for a
    // padded key, 0 otherwise (the MFMAs add the products to it, and -inf
    // plus a finite product stays -inf), so no masking pass follows.  Blocks
    // without padded keys, the common case, start from 0; the two cases run
    // separate MFMA chains, which keeps S in one register tuple.
    f32x16 S;
    auto key_start = [&]() {
        f32x16 c;
#pragma unroll
        for (int r = 0; r < 16; r++) c[r] = ((kb >> acc_row(r, lane)) & 1u) ? 0.f : -__builtin_inff();
        return c;
    };
    if constexpr (DT == 1) {
        // stage K_j, V_j (and Q_i when a piece starts) in this wave's LDS
        // region; K and Q are read back one token row per lane (the MFMA
        // operand layout: lane l holds token l % 32, channels 16 kc + 8 (l / 32))
        constexpr int kRowLanes = HD / 8, kRowsPerLoad = 64 / kRowLanes;
        constexpr int VS = v_stride_b(HD), QS = q_stride_b(HD);
        uint16_t* qs = sb.qs;
        const int r0 = lane / kRowLanes, c0 = (lane % kRowLanes) * 8;
#pragma unroll
        for (int x = 0; x < kKV; x++)
            *reinterpret_cast<u32x4*>(sb.k + k_swz<HD>(r0 + kRowsPerLoad * x, lane % kRowLanes)) = s.k[x];
#pragma unroll
        for (int x = 0; x < kKV; x++)
            *reinterpret_cast<u32x4*>(vs + (r0 + kRowsPerLoad * x) * VS + c0) = s.v[x];
        if (piece_start) {
#pragma unroll
            for (int x = 0; x < kKV; x++)
                *reinterpret_cast<u32x4*>(qs + (r0 + kRowsPerLoad * x) * QS + c0) = s.q[x];
        }
        // the slot is free once staged: the next block's loads go out now,
        // to arrive while this block is computed
        if constexpr (ISSUE) issue<DT, HD, FULL>(p, W, next, s, sb);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // every operand read first, then the MFMA chain (one LDS round trip)
        u32x4 ka[HD / 16], qa[HD / 16];
#pragma unroll
        for (int kc = 0; kc < HD / 16; kc++) {
            ka[kc] = *reinterpret_cast<const u32x4*>(sb.k + k_swz<HD>(n, 2 * kc + h));
            qa[kc] = *reinterpret_cast<const u32x4*>(qs + n * QS + 16 * kc + 8 * h);
        }
        if (kb == 0xFFFFFFFFu) {
            f32x16 z;
#pragma unroll
            for (int r = 0; r < 16; r++) z[r] = 0.f;
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[0]), as_bf16x8(qa[0]), z, 0, 0, 0);
#pragma unroll
            for (int kc = 1; kc < HD / 16; kc++)
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kc]), as_bf16x8(qa[kc]), S, 0, 0, 0);
            // keep the reads together ahead of the MFMAs (the scheduler would
            // otherwise interleave them and wait for each pair)
            __builtin_amdgcn_sched_group_barrier(0x100, HD / 8, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x008, HD / 16, 0);  // MFMA
        } else {
            S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[0]), as_bf16x8(qa[0]), key_start(), 0, 0, 0);
#pragma unroll
            for (int kc = 1; kc < HD / 16; kc++)
                S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[kc]), as_bf16x8(qa[kc]), S, 0, 0, 0);
        }
    } else {
        constexpr int kRowLanes = HD / 4, kRowsPerLoad = 64 / kRowLanes;
        constexpr int VS = v_stride_f(HD);
#pragma unroll
        for (int x = 0; x < kKV; x++)
            *reinterpret_cast<u32x4*>(vs + (lane / kRowLanes + kRowsPerLoad * x) * VS + (lane % kRowLanes) * 4) =
                s.v[x];
        S = key_start();
#pragma unroll
        for (int c4 = 0; c4 < kKV; c4++) {
            const float4 kf = __builtin_bit_cast(float4, s.k[c4]);
            const float4 qf = __builtin_bit_cast(float4, s.q[c4]);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.x, qf.x, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.y, qf.y, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.z, qf.z, S, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x2f32(kf.w, qf.w, S, 0, 0, 0);
        }
        // K and Q are used, V is staged: the next block's loads go out now
        if constexpr (ISSUE) issue<DT, HD, FULL>(p, W, next, s, sb);
        __builtin_amdgcn_sched_barrier(0);
    }
    // online softmax in log2 units: max over the 32 keys of each query row
    float bm = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; r++) bm = fmaxf(bm, S[r]);
    bm = xhalf_max(bm) * scale2;
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
        // O^T += V_j^T P^T ; A operand read transposed from LDS, every read
        // first, then the MFMAs
        const int g16 = lane >> 4, s16 = lane & 15;
        bf16x8 av[2][HD / 32];
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
                av[kc2][mt] = __builtin_bit_cast(bf16x8, a8);
            }
        }
#pragma unroll
        for (int kc2 = 0; kc2 < 2; kc2++)
#pragma unroll
            for (int mt = 0; mt < HD / 32; mt++)
                A.o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kc2][mt], pb[kc2], A.o[mt], 0, 0, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * (HD / 32), 0);   // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * (HD / 32), 0);   // MFMA
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
    // The end of a piece: a segment that started in this range and ends here
    // is finished; a piece of a segment that another wave started is parked
    // for it; a segment that started here and goes on past the range is
    // kept in A for the join after the workgroup barrier.
    const bool seg_end = info_pos(info) == info_len(info) - 1;
    if (seg_end || e == W.end - 1) {
        const bool started_here = e - info_pos(info) >= W.start;
        if (seg_end && started_here)
            finish_segment<DT, HD, FULL>(p, W, A, we, i, info, reinterpret_cast<float*>(vs), sb.pend);
        else if (!started_here)
            park_piece<DT, HD, FULL>(W, A);
        else
            A.jend = e - info_pos(info) + info_len(info) - 1;
    }
}


// The blocks [W.start, W.end) of the wave's record window.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void run_blocks(const Params& p, Wave<DT, HD>& W, StageBuf<DT, HD>& sb, Acc<DT, HD>& A) {
    const int bh = W.bh;
    const size_t head_off = (size_t)bh * p.N * HD;
    using E = typename Cfg<DT, HD>::Elem;
    W.Qg = static_cast<const E*>(p.q) + head_off;
    W.Kg = static_cast<const E*>(p.k) + head_off;
    W.Vg = static_cast<const E*>(p.v) + head_off;
    const float scale2 = (1.0f / __builtin_sqrtf((float)p.dscale)) * kLog2e;
    const int start = W.start, end = W.end;

    // kSlots load slots in a ring: each block stages its slot's data in LDS
    // and then refills the slot with the block kSlots ahead (past the end,
    // the last block again, so that every block of the ring issues the same
    // loads and the wait counts stay exact); they arrive while the blocks
    // in between are computed.  The last blocks, fewer than kSlots, issue
    // nothing.
    constexpr int NS = kSlots<HD>();
    Slot<DT, HD> sl[NS];
#pragma unroll
    for (int x = 0; x < NS; x++) issue<DT, HD, FULL>(p, W, min(start + x, end - 1), sl[x], sb);
    // the cell's low-res weight, formed as the low-res sums formed it (0 past
    // the stream's end, where the mask word is 0)
    if constexpr (FULL) W.ww = lowres_weight(W.ww, W.wm, __popc(W.wk));
    int e = start;
    for (; e + NS <= end; e += NS) {
#pragma unroll
        for (int x = 0; x < NS; x++)
            process<DT, HD, FULL>(p, W, e + x, sl[x], A, sb, scale2, min(e + x + NS, end - 1));
    }
#pragma unroll
    for (int x = 0; x + 1 < NS; x++)
        if (e + x < end) process<DT, HD, FULL, false>(p, W, e + x, sl[x], A, sb, scale2, 0);
}

// Relative costs of the work in a wave's part, in eighths of a block: every
// block, and on top each segment end (the output or partial it writes) and
// each segment start (Q staged, accumulators reset).  Measured on MI355X: a
// segment end costs about three quarters of a block, a start about 0.4.
constexpr int kCostBlock = 8, kCostEnd = 6, kCostStart = 3;

// The cost of the stream before block e (whose record info is given), in
// eighths of a block: the segments before e's segment have all started and
// ended, and e's own segment has started unless e is its first block.
__device__ __forceinline__ int64_t cost_before(int64_t e, int item, int pos) {
    return kCostBlock * e + (int64_t)(kCostEnd + kCostStart) * item + (pos > 0 ? kCostStart : 0);
}

// Wave k of the WPH waves of head bh; waves k with the same k / kWaves are
// one workgroup.  The workgroup takes range k / kWaves of the head's record
// stream (its ends moved to the nearest segment starts) and splits it into
// kWaves parts of equal cost, one per wave, wherever those cuts fall: each
// cut is the first block at which the cost before it reaches its share,
// searched within m blocks of the equal-block cut (so that every wave finds
// the same cuts in its own record window).  A segment cut by them is
// finished by the wave holding its first block, after the workgroup's
// barrier, from its own piece and the parked pieces of the next waves.  All
// waves of the workgroup reach that barrier once per call; wg_cut (LDS)
// passes the cuts to the joiners.
template <int DT, int HD, bool FULL>
__device__ __forceinline__ void run_range(const Params& p, int bh, int k, int WPH, int lane, int wave,
                                          StageBuf<DT, HD>& sb, int* wg_cut, int4* wg_join, int* wg_njoin) {
    // the head's stream: K records (a static layout fills row_ptr[nb] of its
    // capacity K)
    const int64_t K = p.attn_dyn ? min((int64_t)p.row_ptr[(size_t)bh * (p.nb + 1) + p.nb], p.K) : p.K;
    const int G = WPH / kWaves, g = k / kWaves;
    const int an = (int)((int64_t)g * K / G), bn = (int)((int64_t)(g + 1) * K / G);
    const BlkRec* R = p.recs + (size_t)bh * p.K;
    const uint32_t info_a = an < K ? R[an].info : 0u;
    const uint32_t info_b = bn < K ? R[bn].info : 0u;
    const uint32_t info_z = K > 0 ? R[K - 1].info : 0u;   // the stream's last block
    // for after the range: the head's listed rows and the first this wave takes
    const int nm = min(p.n_merge[bh], p.nb);
    int4 dsc = p.merge_rows[(size_t)bh * p.nb + min(k, p.nb - 1)];
    // The workgroup's range [S, E): both ends moved to the nearest segment
    // start (the next workgroup's range starts where this one ends, since
    // both round the same block index the same way).
    const int S = nearest_segment_start(an, info_a, K);
    const int E = max(nearest_segment_start(bn, info_b, K), S);
    const int T = E - S;
    // the segment index (item) of a segment start x reached from block y
    auto item_at = [&](int x, int y, uint32_t info_y) {
        if (x >= K) return info_item(info_z) + 1;
        return info_item(info_y) + (x == y - info_pos(info_y) ? 0 : 1);
    };
    const int64_t c0 = cost_before(S, item_at(S, an, info_a), 0);
    const int64_t c4 = cost_before(E, item_at(E, bn, info_b), 0);
    // equal-block cuts c_w and the search margin m around them
    const int q = T / kWaves, qc = (T + kWaves - 1) / kWaves;
    const int m = max(0, min(16, min((q - 1) / 2, (kWindow - 1 - qc) / 2)));
    const int cw = S + wave * T / kWaves, cn = S + (wave + 1) * T / kWaves;
    Wave<DT, HD> W;
    W.a = wave == 0 ? S : cw - m;   // the window: [cw - m, cn + m] is inside it
    W.park = p.park + ((size_t)bh * WPH + k) * park_floats(HD);
    W.bh = bh;
    W.b = bh / p.H;
    W.nb = p.nb;
    W.lane = lane;
    W.wave = wave;
    W.n = lane & 31;
    W.h = lane >> 5;
    {
        int4 r = make_int4(0, 0, 0, 0);
        if (W.a + lane < K) r = *reinterpret_cast<const int4*>(R + W.a + lane);
        W.wij = (uint32_t)r.x;
        W.wk = (uint32_t)r.y;
        W.winfo = (uint32_t)r.w;
        W.ww = 0.f;
        W.wm = 0.f;
        W.wll = 0.f;
        if (FULL && W.a + lane < K) {
            // the cell's logit (its low-res weight is formed once the first
            // block's loads are out), the row's max and weight sum
            const size_t row = (size_t)bh * p.nb + min(rec_i(W.wij), p.nb - 1);
            W.ww = p.logits[row * p.nb + min(rec_j(W.wij), p.nb - 1)];
            W.wm = p.rowmax[row];
            W.wll = p.ll_all[row];
        }
    }
    {
        // The cuts of this wave's part: the first block in [c - m, c + m]
        // whose cost before it reaches the cut's share (else c + m).
        const int64_t e = W.a + lane;
        const int64_t pc = cost_before(e, info_item(W.winfo), info_pos(W.winfo));
        auto cut = [&](int w, int c) {
            if (w == 0) return S;
            if (w == kWaves) return E;
            const int64_t target = c0 + (c4 - c0) * w / kWaves;
            const uint64_t hit = __builtin_amdgcn_ballot_w64(e >= c - m && e <= c + m && e < K && pc >= target);
            return hit ? W.a + (int)__builtin_ctzll(hit) : c + m;
        };
        W.start = cut(wave, cw);
        W.end = cut(wave + 1, cn);
        if (lane == 0) wg_cut[wave] = W.start;
        if (lane == 0 && wave == kWaves - 1) wg_cut[kWaves] = W.end;
    }
    Acc<DT, HD> A;
    A.mrun = -__builtin_inff();
    A.lsum = 0.f;
    A.npend = 0;
    A.jend = -1;
#pragma unroll
    for (int mt = 0; mt < HD / 32; mt++)
#pragma unroll
        for (int r = 0; r < 16; r++) A.o[mt][r] = 0.f;   // finite, so alpha = 0 clears them
    if (W.start < W.a || W.end - W.a > kWindow) {   // the window must hold every block of the part
        if (lane == 0) atomicOr(reinterpret_cast<unsigned int*>(p.error), 4u);
    } else if (W.start < W.end) {
        run_blocks<DT, HD, FULL>(p, W, sb, A);
    }
    // the parked pieces are written; the next waves' pieces of a segment
    // held in A are read after this barrier
    __syncthreads();
    if (A.jend >= 0) {
        for (int x = wave + 1; x < kWaves; x++) {
            const int ax = wg_cut[x], bx = wg_cut[x + 1];
            if (ax > A.jend) break;
            if (ax < bx) merge_piece<DT, HD, FULL>(W.park + (size_t)(x - wave) * park_floats(HD), lane, A);
        }
        const int we = W.end - 1 - W.a;
        const uint32_t info = (uint32_t)rl((int)W.winfo, we);
        const int i = min(rec_i((uint32_t)rl((int)W.wij, we)), p.nb - 1);
        finish_segment<DT, HD, FULL>(p, W, A, we, i, info, reinterpret_cast<float*>(sb.v), sb.pend);
    }
    const int npend = A.npend;
    // Then count the cut segments this wave ended, one lane per segment,
    // once their partials are stored; a segment that completes its row's
    // count puts the row on the workgroup's join list.  After a second
    // barrier the workgroup's four waves join every listed row together, a
    // quarter of its tokens each.  Then the head's rows with no selected
    // block, listed rows k, k + WPH, ... by this wave alone.
    uint64_t joins = 0;        // lanes whose segment completed its row
    int jrow = 0, jfirst = 0, jn = 0;
    if (npend > 0) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every partial store has completed
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        bool last = false;
        if (lane < npend) {
            jrow = min(max(sb.pend[lane], 0), p.nb - 1);
            const uint32_t old = __hip_atomic_fetch_add(p.join_cnt + (size_t)bh * p.nb + jrow, 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int* ip = p.item_ptr + (size_t)bh * (p.nb + 1) + jrow;
            jfirst = ip[0];
            jn = ip[1] - jfirst;
            last = (int)old + 1 == jn;
        }
        joins = __builtin_amdgcn_ballot_w64(last);
    }
    {
        // this wave's rows to join, packed into its part of the list
        const int slot = __builtin_popcountll(joins & ((1ull << lane) - 1ull));
        if ((joins >> lane) & 1ull) wg_join[wave * kWindow + slot] = make_int4(jrow, jfirst, jn, 0);
        if (lane == 0) wg_njoin[wave] = __builtin_popcountll(joins);
    }
    __syncthreads();
#pragma unroll 1
    for (int w = 0; w < kWaves; w++) {
        const int nj = wg_njoin[w];
        for (int x = 0; x < nj; x++) {
            const int4 jd = wg_join[w * kWindow + x];
            join_part<DT, HD, FULL>(p, bh, W.b, p.nb, lane, wave, jd.x, jd.y, jd.z);
            // back to zero for the next launch on this workspace (every segment has counted)
            if (wave == 0 && lane == 0)
                __hip_atomic_store(p.join_cnt + (size_t)bh * p.nb + jd.x, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    for (int s = k; s < nm; s += WPH) {
        if (s != k) dsc = p.merge_rows[(size_t)bh * p.nb + s];
        if (dsc.z == 0)
            join_row<DT, HD, FULL>(p, bh, W.b, p.nb, lane, min(max(dsc.x, 0), p.nb - 1), 0, 0,
                                   reinterpret_cast<float*>(sb.v));
    }
}

// Two workgroups per CU for 64-channel heads; one for 128-channel heads,
// whose staged blocks fill the CU's LDS and whose accumulators need the
// larger register budget.
template <int DT, int HD, bool FULL>
__global__ __launch_bounds__(kThreads, HD == 64 ? 2 : 1) void attn_kernel(Params p) {
    StageBuf<DT, HD>* stage = reinterpret_cast<StageBuf<DT, HD>*>(attn_smem);   // one per wave
    // the cuts of the workgroup's range between its waves; two sets, so that
    // a wave that starts the next head in turn does not overwrite the cuts a
    // slower wave may still be reading for the previous one
    __shared__ int wg_cut[2][kWaves + 1];
    // the rows the workgroup joins together after its second barrier: (row,
    // first segment, segments) per wave's completed rows (a wave ends at most
    // kWindow segments), and their number per wave
    __shared__ int4 wg_join[kWaves * kWindow];
    __shared__ int wg_njoin[kWaves];
    const int xcd = blockIdx.x & 7;
    // the wave index is uniform: made so for the compiler, so that ranges,
    // loop bounds and addresses derived from it stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int wx = (blockIdx.x >> 3) * kWaves + wave;      // wave index within its XCD
    const int WPH = p.attn_wph;
    if (p.attn_seq) {
        // every wave of the XCD takes range wx of each of the XCD's heads in
        // turn, so the XCD's L2 holds one head's K and V at a time
        if (wx >= WPH) return;
        for (int bh = xcd; bh < p.BH; bh += 8)
            run_range<DT, HD, FULL>(p, bh, wx, WPH, lane, wave, stage[wave], wg_cut[(bh >> 3) & 1], wg_join,
                                    wg_njoin);
    } else {
        const int hm = wx / WPH;
        const int bh = xcd + 8 * hm;
        if (bh < p.BH)
            run_range<DT, HD, FULL>(p, bh, wx - hm * WPH, WPH, lane, wave, stage[wave], wg_cut[0], wg_join,
                                    wg_njoin);
    }
}

}  // namespace

// Heads whose ranges would still hold at least this many blocks each when
// every wave of an XCD shares one head are taken in turn.
constexpr int64_t kTurnMinBlocks = 12;
// Waves resident on one XCD (32 CUs): two workgroups of kWaves per CU for
// 64-channel heads, one for 128-channel heads (see attn_kernel's bounds).
// A grid of more would run a second round of workgroups.
int waves_per_xcd(int hd) { return 32 * kWaves * (hd == 64 ? 2 : 1); }

bool attn_heads_in_turn(int BH, int64_t K, int hd) {
    return (BH + 7) / 8 >= 2 && K >= kTurnMinBlocks * waves_per_xcd(hd);
}

int attn_grid_waves_per_head(int BH, int64_t K, int hd) {
    const int heads_per_xcd = (BH + 7) / 8;
    const int wx = waves_per_xcd(hd);
    int64_t w = attn_heads_in_turn(BH, K, hd) ? wx : wx / heads_per_xcd;
    const int64_t hi = (K + 1) / 2;                   // at least about two blocks a wave
    if (w > hi) w = hi;
    // whole workgroups, rounded down so that the grid stays within one
    // round of resident workgroups
    w = w / kWaves * kWaves;
    if (w < kWaves) w = kWaves;
    // keep each range inside one record window
    const int64_t lo = ((K + kMaxRun - 1) / kMaxRun + kWaves - 1) / kWaves * kWaves;
    if (w < lo) w = lo;
    return (int)w;
}

// Segment lengths.  A row of up to one workgroup's share of the head is one
// segment: moving a range end to a segment start then unbalances the
// workgroups by at most half a row, and the row needs no join.  A longer
// row is cut into segments of about half that share, whose partials go
// through memory and a join.  Both within [kChunkMin, kChunkMax], and short
// enough that a range grown by half a segment at each end still splits into
// parts the record window holds (kWaves parts of at most kWindow - 1 blocks).
void attn_segments(int BH, int64_t K, int hd, int32_t* seg_whole, int32_t* chunk) {
    const int64_t G = attn_grid_waves_per_head(BH, K, hd) / kWaves;
    const int64_t r = (K + G - 1) / G;   // blocks per workgroup range, before the moves
    const int64_t fit = (int64_t)kWaves * (kWindow - 1) - r - 2;
    auto clamp = [&](int64_t c) {
        if (c > fit) c = fit;
        if (c > kChunkMax) c = kChunkMax;
        return (int32_t)(c < kChunkMin ? kChunkMin : c);
    };
    *seg_whole = clamp(r);
    *chunk = clamp(r / 2);
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
