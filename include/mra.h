/*
 * mra.h — C ABI of the MI355X (gfx950) MRA-2 attention library (libmra.so,
 * built from block_sparse_approximate_amd/csrc): the forward pass, its
 * backward pass, and BigBird's block-sparse pattern through the same block
 * attention kernels.
 *
 * The method is MRA-2 multi-resolution approximate self-attention as
 * described on the page "深入解析 Transformers 中的 MRA 模型" ("A deep dive
 * into the MRA model in Transformers", cited [MRA]):
 *   step 1 ("第一步")  average-pool Q and K (and V) over 32-token blocks and
 *                      form the low-resolution block logits;
 *   step 2 ("第二步")  pick the top num_block block pairs globally, with
 *                      optional first-n and diagonal priors (a 5e3 bias);
 *   step 3 ("第三步")  exact softmax attention on the selected 32x32 blocks;
 *   step 4 ("第四步")  "full" mode merges it with low-resolution attention on
 *                      the unselected blocks through a shared row maximum and
 *                      normaliser; "sparse" mode keeps the high-res part only.
 * Parameters and budget: section "MraConfig：四个专属参数" (block_per_row,
 * approx_mode, initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks,
 * num_block = (N/32)*block_per_row capped at (N/32)^2).  N must be a
 * multiple of 32 (engineering notes after step 4).  Attention is
 * bidirectional (section "使用边界与结论").
 *
 * Readings of points the pages leave open: the logit scale is 1/sqrt(d);
 * selection ranks the row-max-normalised low-res logits; ties at the k-th
 * score go to the smaller flat index i*nb + j; the first-n prior adds 5000
 * to rows i < n and again to columns j < n; the diagonal prior covers
 * |i - j| <= floor(n/2) (or, as an option, a band exactly n blocks wide);
 * a low-res cell weighs cnt_j * exp(logit); an empty
 * block scores -inf; padded query rows output 0; 0/0 gives 0.
 *
 * Conventions for every entry point:
 *   - Tensors are row-major and contiguous.  q, k, v, out: [batch, heads,
 *     seq_len, head_dim] in the dtype of `dims->dtype`; out has the same
 *     dtype.  mask: [batch, seq_len] uint8, nonzero = valid token, or NULL
 *     (every token valid).
 *   - Pointers named device pointers are device memory owned by the caller;
 *     q, k, v, out and mask must be 16-byte aligned; the library allocates
 *     nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is queued
 *     asynchronously on it; nothing synchronises.
 *   - Arguments are checked on the host before anything is queued; on an
 *     error nothing is written and the status says why.  MRA_ERR_HIP means a
 *     launch failed; the outputs are then undefined.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef MRA_H
#define MRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MRA_OK = 0,
    MRA_ERR_NULL = 1,       /* a required pointer is NULL */
    MRA_ERR_SHAPE = 2,      /* batch or heads < 1, or the sizes overflow */
    MRA_ERR_SEQ_LEN = 3,    /* seq_len not a multiple of 32, < 32 or > 16384 (BigBird: or of its block size) */
    MRA_ERR_HEAD_DIM = 4,   /* head_dim other than 64 or 128, or scale_dim outside 0 .. head_dim */
    MRA_ERR_DTYPE = 5,      /* dtype not MRA_F32 or MRA_BF16 */
    MRA_ERR_MODE = 6,       /* approx_mode not MRA_APPROX_FULL or MRA_APPROX_SPARSE */
    MRA_ERR_BUDGET = 7,     /* block_per_row < 1 (BigBird: num_random_blocks < 1) */
    MRA_ERR_PRIOR = 8,      /* a prior count < 0, or an unknown diagonal band reading */
    MRA_ERR_ALIAS = 9,      /* an output overlaps an input, another output or a workspace */
    MRA_ERR_WORKSPACE = 10, /* a workspace NULL or smaller than its size query returns */
    MRA_ERR_HIP = 11,       /* a HIP call failed */
    MRA_ERR_ALIGN = 12,     /* a tensor pointer is not 16-byte aligned */
    MRA_ERR_STAGE = 13,     /* mra_debug_replay: a stage other than 3, or count < 1;
                               mra_debug_wait_timeout: polls out of range */
    MRA_ERR_SCRATCH = 14    /* mra_attention_fwd_noalloc: the sizes need more than its 64 MiB scratch */
} mra_status;

/* Bits of a workspace's device error word (mra_workspace_error).  The
 * kernels check their own bookkeeping as they run and set a bit when it does
 * not add up; every bit means the call's outputs are undefined.
 *   MRA_DEVERR_CANDIDATES  selector: the boundary bin's candidate list does
 *                          not hold the bin's count (selection undefined)
 *   MRA_DEVERR_STREAM      selector or layout: the selection does not hold
 *                          num_block cells (BigBird: more than its capacity),
 *                          or a head needs more segments than the workspace
 *                          holds (selection and output undefined)
 *   MRA_DEVERR_WINDOW      block attention: a wave's share of a head's blocks
 *                          does not fit its record window; that wave wrote
 *                          none of its rows (output undefined)
 *   MRA_DEVERR_BWD_PLAN    backward: the transposed selection or the chunk
 *                          plan does not match the forward's selection
 *                          (gradients undefined)
 *   MRA_DEVERR_NO_STATS    backward: the forward call did not save the
 *                          softmax statistics (mra_options.save_stats = 0;
 *                          gradients undefined)
 *   MRA_DEVERR_WAIT        selector (N = 2048 or 4096): a workgroup gave up
 *                          waiting for the other workgroups of its head to
 *                          store their logits, i.e. the device did not run
 *                          them (selection and output undefined) */
enum {
    MRA_DEVERR_CANDIDATES = 1,
    MRA_DEVERR_STREAM = 2,
    MRA_DEVERR_WINDOW = 4,
    MRA_DEVERR_BWD_PLAN = 8,
    MRA_DEVERR_NO_STATS = 16,
    MRA_DEVERR_WAIT = 32
};

typedef enum { MRA_F32 = 0, MRA_BF16 = 1 } mra_dtype;
typedef enum { MRA_APPROX_FULL = 0, MRA_APPROX_SPARSE = 1 } mra_approx_mode;

/* What step 2's global top-k ranks ([MRA] "第二步": top-k on the low-res
 * logits, each row's best blocks).  The default takes each cell's logit
 * minus its row's maximum, so that every row's best block ranks first (the
 * plainest reading of "each row" within one global top-k); the alternative
 * ranks the raw logits themselves.  Priors and empty blocks apply to both. */
typedef enum { MRA_RANK_ROW_NORMALIZED = 0, MRA_RANK_RAW_LOGITS = 1 } mra_score_ranking;

/* Width of the diagonal prior band of initial_prior_diagonal_n_blocks = n
 * ([MRA] "第二步": a band of blocks centred on the main diagonal).  For odd n
 * both readings are the band |i - j| <= (n - 1) / 2.  For even n a band
 * centred on the diagonal cannot be exactly n blocks wide and symmetric:
 *   MRA_BAND_SYMMETRIC  |i - j| <= floor(n / 2), n + 1 blocks wide (default);
 *   MRA_BAND_EXACT      exactly n blocks wide, offsets j - i from
 *                       -floor((n - 1) / 2) to +floor(n / 2). */
typedef enum { MRA_BAND_SYMMETRIC = 0, MRA_BAND_EXACT = 1 } mra_diag_band;

/* The selection options of mra_attention_fwd_ex: the four MraConfig
 * parameters, the ranking, the band reading, and whether to keep what the
 * backward pass needs. */
typedef struct {
    int32_t block_per_row;
    int32_t approx_mode;     /* mra_approx_mode */
    int32_t prior_first;     /* initial_prior_first_n_blocks */
    int32_t prior_diag;      /* initial_prior_diagonal_n_blocks */
    int32_t score_ranking;   /* mra_score_ranking; MRA_ERR_MODE if neither */
    int32_t diag_band;       /* mra_diag_band; MRA_ERR_PRIOR if neither */
    int32_t save_stats;      /* 1: also store each token's softmax maximum and
                                1/normaliser in the workspace, for
                                mra_attention_bwd; 0: inference only (the
                                backward then flags MRA_DEVERR_NO_STATS) */
} mra_options;

typedef struct {
    int32_t batch;
    int32_t heads;
    int32_t seq_len;  /* N: multiple of 32, 32 <= N <= 16384 */
    int32_t head_dim; /* d: 64 or 128 */
    int32_t dtype;    /* mra_dtype */
    int32_t scale_dim; /* 0, or the logical head size (1 .. head_dim) of heads zero-padded to head_dim:
                          the logit scale is 1/sqrt(scale_dim).  Zero channels add exact zeros to
                          every pooled mean, logit and product, so a head of d < 64 channels padded
                          with zeros to 64 (or 64 < d < 128 padded to 128) gives the result of a
                          d-channel head ([MRA] engineering notes: the model pads small heads for
                          the kernels). */
} mra_dims;

/* Version of this ABI (changes when a signature or a layout changes). */
int32_t mra_abi_version(void);

/* Static text for a status code; never NULL. */
const char* mra_status_string(int32_t status);

/* Selection budget per (batch, head) ([MRA] "MraConfig" section):
 * min((seq_len/32) * block_per_row, (seq_len/32)^2).  Returns -1 when
 * seq_len is not a positive multiple of 32 or block_per_row < 1. */
int64_t mra_num_block(int32_t seq_len, int32_t block_per_row);

/* Bytes of device workspace mra_attention_fwd needs for these sizes.
 * Host-only; *bytes is written on MRA_OK. */
mra_status mra_workspace_size(const mra_dims* dims, int32_t block_per_row, int32_t approx_mode,
                              size_t* bytes);

/* The MRA-2 forward pass ([MRA] steps 1-4).
 *   q, k, v      device, [B, H, N, d], dtype dims->dtype
 *   mask         device, [B, N] uint8 (nonzero = valid), or NULL
 *   block_per_row, approx_mode, prior_first, prior_diag: the four MraConfig
 *                parameters (block_per_row >= 1, priors >= 0)
 *   out          device, [B, H, N, d], dtype dims->dtype; written in full
 *   workspace    device, at least mra_workspace_size() bytes, 256-byte
 *                aligned, overlapping no input or output (MRA_ERR_ALIAS);
 *                its contents need not be initialised
 *   stream       hipStream_t or NULL
 * The default options of mra_attention_fwd_ex: row-normalised ranking, the
 * symmetric band, and no softmax statistics kept (inference); a forward
 * call whose output is to be differentiated goes through
 * mra_attention_fwd_ex with save_stats = 1. */
mra_status mra_attention_fwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                             const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                             int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* mra_attention_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, with no workspace argument.  The workspace
 * is a fixed 64 MiB device array inside the library, one copy per GPU, held
 * until the process ends; the call allocates nothing.  Sizes whose
 * mra_workspace_size exceeds 64 MiB return MRA_ERR_SCRATCH (B=2, H=12,
 * N=4096 full mode needs 57.9 MiB).  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller; each call clears what
 * it needs cleared.  Its device error word is not exposed.  Other arguments
 * and errors as for mra_attention_fwd. */
mra_status mra_attention_fwd_noalloc(const mra_dims* dims, const void* q, const void* k, const void* v,
                                     const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                     int32_t prior_first, int32_t prior_diag, void* out, void* stream);

/* mra_attention_fwd with its options in a struct (opts: host pointer, read
 * during the call), which adds the choice of ranking and band reading and
 * the softmax statistics for the backward pass; MRA_ERR_NULL when opts is
 * NULL.  With score_ranking = MRA_RANK_ROW_NORMALIZED, diag_band =
 * MRA_BAND_SYMMETRIC and save_stats = 0 it is exactly mra_attention_fwd.
 * The backward pass reads the selection the forward made, so it needs no
 * ranking or band of its own. */
mra_status mra_attention_fwd_ex(const mra_dims* dims, const void* q, const void* k, const void* v,
                                const uint8_t* mask, const mra_options* opts, void* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Profiling variant of mra_attention_fwd: the same work, plus a
 * hipEventRecord on `stream` before and after each kernel launch.
 *   events  array of 8 hipEvent_t created by the caller (with timing);
 *           entries 2s and 2s+1 bracket stage s: 0 pooling, 1 low-res
 *           logits, 2 top-k selection, 3 block attention with the low-res
 *           merge and the join of rows cut into several segments.  NULL
 *           entries are skipped.  The events stay owned by the caller. */
mra_status mra_attention_fwd_profiled(const mra_dims* dims, const void* q, const void* k, const void* v,
                                      const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                      int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream, void* const* events);

/* Stage hook for parity tests: runs steps 1 and 2 of the same kernels and
 * copies the intermediate results out (device buffers owned by the caller,
 * any of them may be NULL to skip it):
 *   qhat, khat, vhat  [B, H, N/32, d] fp32 pooled blocks (vhat: full mode only)
 *   count             [B, N/32] int32 valid tokens per block
 *   logits            [B, H, N/32, N/32] fp32 low-res logits, tau * qhat . khat
 *   rowmax            [B, H, N/32] fp32 row max over non-empty key blocks
 *   sel               [B, H, num_block] int32 selected flat indices i*nb + j,
 *                     ascending
 *   error             [1] int32 device error word (0 = consistent)
 * score_ranking and diag_band as in mra_options; the other arguments are as
 * for mra_attention_fwd. */
mra_status mra_debug_stages(const mra_dims* dims, const void* q, const void* k, const void* v,
                            const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                            int32_t prior_first, int32_t prior_diag, int32_t score_ranking,
                            int32_t diag_band, float* qhat, float* khat,
                            float* vhat, int32_t* count, float* logits, float* rowmax, int32_t* sel,
                            int32_t* error, void* workspace, size_t workspace_bytes, void* stream);

/* Test hook for the selector's bounded wait (heads of 64 or 128 block rows,
 * seq_len 2048 or 4096, where one launch forms the logits and selects): runs
 * pooling and that launch as mra_debug_stages does (no mask, no priors), but
 * with every workgroup waiting for one workgroup more than its head has, for
 * at most `polls` polls (1 .. 65536).  Each wait runs out, sets
 * MRA_DEVERR_WAIT in the workspace's error word (read it with
 * mra_workspace_error) and the workgroup goes on, so the launch ends however
 * the device schedules it.  The selection it leaves is not meant for use.
 * Callers: tests of the error path.  Returns MRA_ERR_STAGE for polls out of
 * range, MRA_ERR_SEQ_LEN for other sequence lengths or for sizes that take
 * the separate logits and selection launches (more heads than the device
 * holds at once, or no device), otherwise as mra_debug_stages. */
mra_status mra_debug_wait_timeout(const mra_dims* dims, const void* q, const void* k, const void* v,
                                  int32_t block_per_row, int32_t approx_mode, uint32_t polls, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Stage hook: the step-2 selector alone on caller-given logits, so that its
 * result can be compared with the oracle's on identical fp32 inputs.
 *   logits  device [B, H, nb, nb] fp32, count device [B, nb] int32
 *   sel     device [B, H, num_block] int32, ascending flat indices
 * seq_len = 32 * nb comes from dims; q/k/v are not read; score_ranking and
 * diag_band as in mra_options. */
mra_status mra_debug_select(const mra_dims* dims, const float* logits, const int32_t* count,
                            int32_t block_per_row, int32_t prior_first, int32_t prior_diag,
                            int32_t score_ranking, int32_t diag_band, int32_t* sel, void* workspace,
                            size_t workspace_bytes, void* stream);

/* BigBird block-sparse attention through the same block-attention kernels
 * (page "Transformers 中的 BigBird：面向超长序列的稀疏注意力模型完全指南",
 * its description of the three attention patterns and the BigBirdConfig
 * table).  The sequence is cut into nbb = seq_len / block_size pattern
 * blocks; query block I attends key block J when I or J is the first or the
 * last block (the two global blocks), when |I - J| <= 1 (the window of three
 * blocks), or when J is one of row I's random picks; each valid query token
 * then takes exact softmax attention (scale 1/sqrt(d)) over the valid keys of
 * its attended blocks.  Padded query rows output 0.
 *   block_size        32, 64 (the page's default) or 128; seq_len a
 *                     multiple of it (MRA_ERR_SEQ_LEN otherwise)
 *   num_random_blocks r >= 1 (the page: 0 is not supported; MRA_ERR_BUDGET)
 *   rand_blocks       device int32 [B, H, nbb, r]: the random key blocks the
 *                     layer drew for each query block (the caller draws them);
 *                     values outside [0, nbb) name no block, a block named
 *                     more than once or also in the window is attended once
 *   the other arguments as for mra_attention_fwd; workspace of
 *   mra_bigbird_workspace_size bytes.  No fallback to full attention for
 *   short sequences: the pattern is applied as stated at every length. */
mra_status mra_bigbird_workspace_size(const mra_dims* dims, int32_t block_size, int32_t num_random_blocks,
                                      size_t* bytes);
mra_status mra_bigbird_fwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                           const uint8_t* mask, int32_t block_size, int32_t num_random_blocks,
                           const int32_t* rand_blocks, void* out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Gradients of a mra_bigbird_fwd call's output with respect to q, k and v:
 * the chunked backward of mra_attention_bwd (sparse mode) on the layout that
 * call made (the pattern is a constant of the backward pass).
 *   q, k, v, mask, block_size, num_random_blocks: as for that call (its
 *   rand_blocks are not read again: the layout is in its workspace);
 *   out, dout, dq, dk, dv, workspace, bwd_workspace: as for
 *   mra_attention_bwd, with bwd_workspace of
 *   mra_bigbird_backward_workspace_size bytes.  bf16 or fp32. */
mra_status mra_bigbird_backward_workspace_size(const mra_dims* dims, int32_t block_size,
                                               int32_t num_random_blocks, size_t* bytes);
mra_status mra_bigbird_bwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                           const uint8_t* mask, int32_t block_size, int32_t num_random_blocks,
                           const void* out, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                           size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                           void* stream);

/* Bytes of the backward pass's own workspace for these dimensions and
 * selection parameters (mra_attention_bwd's bwd_workspace): the dO . O row
 * terms, the transposed selection, the work chunks, fp32 partial gradients
 * and in full mode the low-resolution gradient terms (block-level vectors and
 * two [nb, nb] fp32 matrices per head).  Status as for mra_workspace_size. */
mra_status mra_backward_workspace_size(const mra_dims* dims, int32_t block_per_row, int32_t approx_mode,
                                       size_t* bytes);

/* Gradients of the forward pass with respect to q, k and v ([MRA] "第三步":
 * the block products' backward reuses the kernels on transposed block
 * indices, so the block selection is a constant of the backward pass).
 *   q, k, v, mask, block_per_row, approx_mode, priors: as for the forward
 *             call whose selection is used;
 *   out       [B, H, N, d] that call's output;
 *   dout      [B, H, N, d] dL/d out;
 *   dq, dk, dv [B, H, N, d] gradients, written (in the dtype of dims);
 *   workspace the workspace that forward call filled (its selection and
 *             each token's softmax statistics, so a forward call made with
 *             save_stats = 1), unchanged since; read only except for its
 *             device error word, where the backward's own checks add bits;
 *   bwd_workspace  device scratch of mra_backward_workspace_size bytes
 *             (16-byte aligned, caller-owned, no contents kept between
 *             calls; MRA_ERR_WORKSPACE if smaller).
 * Must be queued after that forward call (stream order).  Both modes; in
 * full mode the low-resolution branch is differentiated too ([MRA] "第四步"),
 * through the block means to every valid token of each block.  bf16 or fp32
 * (the dtype of dims; fp32 runs its products on fp32 matrix instructions).
 * dq, dk, dv and bwd_workspace must be 16-byte aligned and overlap no input
 * or each other (MRA_ERR_ALIAS).  The result does not depend on scheduling:
 * partial sums are added in a fixed order. */
mra_status mra_attention_bwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                             const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                             int32_t prior_first, int32_t prior_diag, const void* out, const void* dout,
                             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                             void* bwd_workspace, size_t bwd_workspace_bytes, void* stream);

/* The device error word of a workspace (a forward call's; the backward
 * passes that read it add their bits there too): waits for `stream` to
 * finish its queued work, then copies the word to *error (host pointer).
 * 0 means every kernel's bookkeeping added up; any MRA_DEVERR_ bit means the
 * outputs of the call that set it are undefined.  The word is cleared by
 * the next forward call on the workspace.  MRA_ERR_NULL / MRA_ERR_WORKSPACE
 * for a missing pointer or a workspace smaller than 256 bytes,
 * MRA_ERR_HIP if the wait or the copy fails. */
mra_status mra_workspace_error(const void* workspace, size_t workspace_bytes, void* stream,
                               uint32_t* error);

/* Timing hook: relaunches one stage of the forward pass `count` times in a
 * row on `stream`, on a workspace that a call of mra_attention_fwd with the
 * same arguments has filled (stream order: after that call).  Only stage 3
 * (block attention, low-res merge and join) is accepted: it leaves the
 * workspace as it found it (its per-row join counters end at zero) and each
 * relaunch rewrites the same output.  A pair of events around the call then
 * times the kernel alone,
 * with no event between its launches.  The arguments are checked as for
 * mra_attention_fwd; MRA_ERR_STAGE for another stage or count < 1. */
mra_status mra_debug_replay(const mra_dims* dims, const void* q, const void* k, const void* v,
                            const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                            int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                            size_t workspace_bytes, int32_t stage, int32_t count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MRA_H */
