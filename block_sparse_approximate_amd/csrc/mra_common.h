// mra_common.h — types, constants and device helpers shared by the HIP
// kernels of the MRA-2 forward pass (gfx950, wave64).
//
// Method: "A deep dive into the MRA model in Transformers" (cited [MRA]),
// steps 1-4.  Everything here is device code or launch plumbing for this
// library only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mra {

constexpr int kBlock = 32;              // [MRA] engineering notes: block size 32
constexpr int kHeadDim = 64;            // head dims this build accepts
constexpr int kHistBits = 12;           // first radix digit of the selection key
constexpr int kHistBins = 1 << kHistBits;
constexpr float kPriorBias = 5000.0f;   // [MRA] step 2: 5e3 bias for forced blocks
// Segments of a row (selected key blocks): the attention's launch chooses
// their lengths between these two (the record's length field holds 6 bits)
constexpr int kChunkMin = 16;
constexpr int kChunkMax = 63;
constexpr int kMaxHeadDim = 128;        // widest head the forward kernels take
// floats per segment's low-res correction: hd channels, weight sum, pad
__host__ __device__ constexpr int corr_stride(int hd) { return hd + 4; }
// floats per parked piece of a segment (attention): O^T, per lane the
// running max and sum, the low-res correction and weight sum
__host__ __device__ constexpr int park_floats(int hd) { return 32 * hd + 128 + hd + 64; }
constexpr int kSelCap = 4096;           // selection candidates one head's boundary bin may hold
constexpr int kCandStride = 32;         // u32 per head's candidate counter: one 128-byte line each
constexpr float kLog2e = 1.4426950408889634f;

// One selected block, in the head's CSR order (block row ascending, then key
// block ascending).  A block row of at most Params::seg_whole selected blocks
// is one segment; a longer one is cut into segments of Params::chunk blocks
// (the last one shorter).  A segment is the unit whose partial softmax the
// attention kernel produces.
//   ij    query block row i (bits 0..15) and key block j (bits 16..31)
//   kmask valid-token mask word of key block j
//   rsv   0 (keeps a record 16 bytes, one load per lane)
//   info  bits  0..17  segment (item) index within the head
//               18..23 position of the block within its segment
//               24..29 segment length (1..63)
//               30     the segment is the whole row
struct BlkRec {
    uint32_t ij;
    uint32_t kmask;
    uint32_t rsv;
    uint32_t info;
};

__host__ __device__ constexpr uint32_t rec_ij(int i, int j) { return (uint32_t)i | ((uint32_t)j << 16); }
__host__ __device__ constexpr uint32_t rec_info(int item, int pos, int len, bool whole) {
    return (uint32_t)item | ((uint32_t)pos << 18) | ((uint32_t)len << 24) | (whole ? (1u << 30) : 0u);
}

// Segment length of a block row of n selected blocks (n itself when the row
// is one segment).
__host__ __device__ constexpr int row_seg_len(int n, int seg_whole, int chunk) { return n <= seg_whole ? n : chunk; }

// Workspace carve, shared by the host dispatcher and the kernels.
struct Layout {
    int32_t B, H, N, d, nb, BH;
    int64_t K;            // selection budget per (batch, head)
    int32_t max_items;    // segments per head, upper bound
    size_t qhat, khat, vhat, cnt, mbits, logits, keys, rowmax, hist, thresh, row_ptr, col, selbits, item_ptr, recs,
        merge_rows, n_merge, join_cnt, lo_all, ll_all, part_o, part_ml, part_corr, park, cand, ncand, st_m, st_linv,
        total;
};

// Everything a kernel needs, passed by value.
struct Params {
    int32_t B, H, N, d, nb, BH, words;  // words = u32 words per selection-bitmap row
    int32_t dscale;        // the head size the logit scale 1/sqrt(dscale) is taken from (d, or the
                           //   logical size of zero-padded heads)
    int64_t K;
    int32_t mode;          // 0 full, 1 sparse
    int32_t dtype;         // 0 fp32, 1 bf16
    int32_t prior_first, prior_diag;
    int32_t rank_raw;      // 1: step 2 ranks the raw low-res logits (no row max subtracted)
    int32_t band_exact;    // 1: the diagonal prior band is exactly prior_diag blocks wide
    int32_t save_stats;    // 1: store each token's softmax statistics (st_m, st_linv) for the backward
    int32_t max_items;
    int32_t seg_whole;     // rows of at most this many selected blocks are one segment
    int32_t chunk;         // longer rows: segments of this many blocks (both kChunkMin..kChunkMax)
    int32_t v_in_logits;   // 1: full mode's V is pooled by extra workgroups of the logits launch (of the
                           //   fused logits and selection launch for N = 2048, 4096)
    int32_t logits_given;  // 1: the logits are already in `logits` (selector hook); step 1 forms only
                           //   row maxima, keys and the histogram from them
    uint32_t wait_polls;   // polls of a workgroup's bounded wait for its head's other workgroups
                           //   (0: the default limit)
    uint32_t wait_extra;   // added to the count waited for (0; 1 makes every wait run out, a test
                           //   of the error path)
    const void* q;
    const void* k;
    const void* v;
    const uint8_t* mask;   // [B, N] or null
    void* out;
    float* qhat;           // [BH, nb, d]
    float* khat;
    float* vhat;           // full mode only
    int32_t* cnt;          // [B, nb] valid tokens per block
    uint32_t* mbits;       // [B, nb] bit t = token t of the block is valid
    float* logits;         // [BH, nb, nb]  tau * qhat_i . khat_j
    uint32_t* keys;        // [BH, nb, nb]  ordered key of each cell's selection score
    float* rowmax;         // [BH, nb]      max over valid j of logits
    uint32_t* hist;        // [BH, kHistBins]
    uint64_t* thresh;      // [BH] composite key of the last selected cell
    int32_t* row_ptr;      // [BH, nb + 1]  CSR of the selection
    int32_t* col;          // [BH, K]
    uint32_t* selbits;     // [BH, nb, words]
    int32_t* item_ptr;     // [BH, nb + 1]  first segment of each block row
    BlkRec* recs;          // [BH, K] selected blocks in CSR order
    int4* merge_rows;      // [BH, nb] rows the final kernel must combine (0 or >1 segments):
                           //   (row, first segment, number of segments, 0)
    int32_t* n_merge;      // [BH]
    uint32_t* join_cnt;    // [BH, nb] segments of a cut row that have stored their partials (the
                           //   selector clears it; the last segment joins the row and clears it again)
    float* lo_all;         // [BH, nb, d] full mode: sum over every key block j of w_ij vhat_j
    float* ll_all;         // [BH, nb]    full mode: sum over every key block j of w_ij
    float* part_o;         // [BH, max_items, 32, d] un-normalised high-res numerators
    float* part_ml;        // [BH, max_items, 2, 32] running max (log2 units) and sum
    float* part_corr;      // [BH, max_items, corr_stride(d)] full mode: the segment's sum of w vhat_j, then of w
    float* park;           // [BH, attn_wph, park_floats(d)] attention: per wave, a piece of a segment
                           //   that another wave of its workgroup finishes
    uint64_t* cand;        // [BH, kSelCap] boundary-bin cells found by the pre-marking pass
    uint32_t* ncand;       // [BH, kCandStride] their number, in word 0; in word 1 the count of the head's
                           //   workgroups whose logits are stored (both cleared by the pooling kernel)
    // backward (mra_attention_bwd)
    const void* fout;      // [B, H, N, d] the forward's output
    const void* dout;      // [B, H, N, d] dL/d out
    void* dq;              // [B, H, N, d] gradients out
    void* dk;
    void* dv;
    float* st_m;           // [BH, N] per query token (forward): the max its softmax sum is relative
                           //   to (log2 units), 0 if none
    float* st_linv;        // [BH, N] (forward) 1 / that sum; 0 for padded or keyless tokens
    // backward workspace
    float* st_d;           // [BH, N] dO . O (0 where st_linv is 0)
    int32_t* ct_ptr;       // [BH, nb + 1] per key block: start of its list in ct_row
    int32_t* ct_row;       // [BH, K] query block rows that selected each key block, ascending
    int32_t bwd_maxch;     // chunk slots per head (one per chunk, rows and columns alike)
    int4* bwd_rch;         // [BH, maxch] row chunks: (row i, first, end in col, partial slot or -1)
    int4* bwd_cch;         // [BH, maxch] column chunks: (column j, first, end in ct_row, slot or -1)
    int4* bwd_rmul;        // [BH, nb] rows of several chunks: (row, first chunk, chunks, 0)
    int4* bwd_cmul;        // [BH, nb] columns of several chunks
    int4* bwd_count;       // [BH] row chunks, column chunks, rows and columns of several chunks
    float* bwd_part_dq;    // [BH, maxch, 32, d] fp32 partials of chunks of multi-chunk rows
    float* bwd_part_dk;    // [BH, maxch, 32, d] and columns
    float* bwd_part_dv;
    // backward, full mode: the low-resolution branch through the block means
    float* bwd_g;          // [BH, nb, d]  g_i = sum over block i's tokens of a_t dO_t
    float* bwd_c;          // [BH, nb]     c_i = sum over block i's tokens of a_t D_t
    float* bwd_et;         // [BH, nb, nb] E^T: e_ij = w_ij (g_i . vhat_j - c_i) at [j][i]
    float* bwd_wt;         // [BH, nb, nb] W^T: w_ij of unselected cells (0 for selected) at [j][i]
    float* bwd_dqh;        // [BH, nb, d]  gradients of the block means qhat, khat, vhat
    float* bwd_dkh;
    float* bwd_dvh;
    int32_t* error;        // device error word (0 = fine; bits MRA_DEVERR_*), then at error[1] the
                           //   forward's save_stats (the backward checks it)
    int32_t attn_dyn;      // 1: a head's stream holds row_ptr[nb] records (a static layout), not K
    int32_t bb_f;          // BigBird layout: pattern block = bb_f blocks of 32 tokens
    int32_t bb_r;          //   random picks per pattern row
    const int32_t* bb_rand;  // [BH, N / (32 bb_f), bb_r]
    int32_t attn_wph;      // attention stream: waves sharing one head's blocks
    int32_t attn_seq;      // 1: those are all the waves of an XCD, which take the XCD's heads in turn
};

// Ordered key of an fp32 score: larger score -> larger unsigned key.
__device__ __forceinline__ uint32_t float_key(float s) {
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Step 2 score of cell (i, j) ([MRA] "第二步"): row-max-normalised low-res
// logit (raw: the logit itself) plus 5000 per prior that covers the cell;
// -inf for empty blocks;
// -0 folded to +0.  The diagonal band of pd blocks is |i - j| <= pd / 2, or
// with `exact` exactly pd blocks wide: -(pd - 1) / 2 <= j - i <= pd / 2.
// The fp32 operations and their order are fixed (this translation unit is
// built with -ffp-contract=off).
__device__ __forceinline__ float cell_score(float logit, float m, int i, int j, bool vi, bool vj,
                                            int pf, int pd, bool raw, bool exact) {
    if (!vi || !vj) return -__builtin_inff();
    float s = raw ? logit : logit - m;
    const int dist = i > j ? i - j : j - i;
    const bool band = exact ? (j - i >= -((pd - 1) / 2) && j - i <= pd / 2) : dist <= pd / 2;
    if (pd > 0 && band) s = s + kPriorBias;
    if (i < pf) s = s + kPriorBias;
    if (j < pf) s = s + kPriorBias;
    if (s == 0.0f) s = 0.0f;
    return s;
}

// Composite key: score first, then the smaller flat index wins a tie.
__device__ __forceinline__ uint64_t cell_key64(uint32_t key32, uint32_t flat) {
    return ((uint64_t)key32 << 32) | (uint64_t)(0xFFFFFFFFu - flat);
}

// Low-resolution weight of cell (i, j) ([MRA] "第四步"): cnt_j exp(S_ij - m_i),
// with m_i the row max of the low-res logits, 0 for an empty key block.
// Every kernel that forms a weight uses this one expression, so a weight
// added in one kernel and taken away in another cancels exactly.
__device__ __forceinline__ float lowres_weight(float s, float m, int cnt) {
#pragma clang fp contract(off)
    return cnt > 0 ? (float)cnt * __builtin_amdgcn_exp2f((s - m) * kLog2e) : 0.0f;
}

// Two fp32 values -> two bf16 (round to nearest even, the hardware
// conversion), low half first.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace mra

// Host-side launchers (one per translation unit).
namespace mra {
hipError_t launch_pool(const Params& p, hipStream_t s);
hipError_t launch_logits(const Params& p, hipStream_t s);
bool v_pooled_in_logits(int mode, int BH, int nb, int d);
hipError_t launch_logits_given(const Params& p, hipStream_t s);
hipError_t launch_premark(const Params& p, hipStream_t s);
hipError_t launch_select(const Params& p, hipStream_t s);
bool fused_select(int BH, int nb, int d, int mode);   // logits and selection in one launch
hipError_t launch_attn(const Params& p, hipStream_t s);
hipError_t launch_bigbird_layout(const Params& p, hipStream_t s);
int bwd_max_chunks(int nb, int64_t K);
hipError_t launch_bwd(const Params& p, hipStream_t s);
int attn_grid_waves_per_head(int BH, int64_t K, int hd);
bool attn_heads_in_turn(int BH, int64_t K, int hd);
void attn_segments(int BH, int64_t K, int hd, int32_t* seg_whole, int32_t* chunk);
}  // namespace mra
