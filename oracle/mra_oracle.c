/*
 * mra_oracle.c — plain, slow CPU oracle for the MRA-2 forward pass and its
 * gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path (the
 * HIP library under block_sparse_approximate_amd/) never calls it, shares no
 * code, header, table or helper with it, and must fail loudly when its own
 * extension is missing.
 *
 * Source of the method: the page "深入解析 Transformers 中的 MRA 模型"
 * ("A deep dive into the MRA model in Transformers"; cited below as [MRA]),
 * sections "MraConfig：四个专属参数" (the four MRA parameters and the
 * num_block formula), "第一步" (step 1: pooling and low-resolution logits),
 * "第二步" (step 2: block selection with priors), "第三步" (step 3: exact
 * attention on the selected blocks), "第四步" (step 4: merging the two
 * resolutions), the engineering notes after step 4 (block size 32, N a
 * multiple of 32) and "使用边界与结论" (bidirectional only).
 * The dense reference follows the textbook scaled-dot-product softmax
 * attention printed as "global MHRA" on the page "UniFormer ... MHRA"
 * (cited as [MHRA]).  The block-sparse pattern of the last section follows
 * the page "Transformers 中的 BigBird：面向超长序列的稀疏注意力模型完全指南"
 * (cited as [BigBird]).
 *
 * Precision: selection is decided in fp32 in the fixed order written out
 * below (sequential sums and fused multiply-add chains, no reassociation);
 * every output value is computed in fp64.  Build with -O2 -ffp-contract=off
 * and no fast-math so that the fp32 steps are exactly the operations
 * written here.
 *
 * Readings of points the pages leave open (each one also appears in the
 * design notes of the repository):
 *   R1  logit scale tau = 1/sqrt(d) on both resolutions.
 *   R2  the top-k ranks the row-max-normalised low-res logits
 *       S_ij - max_j S_ij, globally over the (N/32)^2 block grid.
 *   R3  num_block is a total per (batch, head), not per row.
 *   R4  the budget uses the sequence length N.
 *   R5  ties at the k-th score go to the smaller flat index i*nb + j.
 *   R6  first-n prior: +5000 for rows i < n and +5000 for columns j < n
 *       (additive).
 *   R7  diagonal prior: +5000 where |i - j| <= floor(n/2).  For even n
 *       that band is n + 1 blocks wide; the other reading (R7', variant
 *       bit 1) keeps it exactly n wide, offsets j - i from
 *       -floor((n-1)/2) to +floor(n/2).
 *   R8  the low-resolution branch covers exactly the unselected blocks.
 *   R9  a low-res cell stands for cnt_j keys, so its weight is
 *       cnt_j * exp(S_ij).
 *   R10 the shared row max cancels; the oracle uses one shift per token.
 *   R11 no epsilon in the normaliser; 0/0 gives 0.
 *   R12 empty query or key blocks score -inf; masked keys weigh 0; masked
 *       query rows output 0; an empty block pools to the zero vector.
 *   R13 selections are reported as ascending flat indices i*nb + j.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MRA_BLOCK 32          /* [MRA] engineering notes: block size 32 */
#define MRA_PRIOR_BIAS 5000.0f /* [MRA] step 2: a 5e3 bias forces priors */

/* ------------------------------------------------------------------------ */
/* Budget. [MRA] "MraConfig": num_block = (len // 32) * block_per_row,
 * capped at (len // 32)^2 (reading R4: len is the sequence length).
 * Returns -1 for an invalid argument. */
int64_t oracle_num_block(int32_t seq_len, int32_t block_per_row)
{
    if (seq_len < MRA_BLOCK || seq_len % MRA_BLOCK != 0 || block_per_row < 1)
        return -1;
    int64_t nb = seq_len / MRA_BLOCK;
    int64_t k = nb * (int64_t)block_per_row;
    int64_t cap = nb * nb;
    return k < cap ? k : cap;
}

/* ------------------------------------------------------------------------ */
/* Step 1, pooling ([MRA] "第一步"): the masked mean of each 32-token block.
 * fp32 version, in the canonical order: acc starts at +0.0f and adds the
 * valid tokens t = 0..31 of the block one after another; the mean is
 * acc / (float)cnt, correctly rounded; an empty block gives zeros.
 * x: [N, d] one head; mask: [N] (1 = valid) or NULL; xhat: [nb, d];
 * cnt: [nb] (may be NULL). */
void oracle_pool_f32(int32_t N, int32_t d, const float* x, const uint8_t* mask,
                     float* xhat, int32_t* cnt)
{
    int32_t nb = N / MRA_BLOCK;
    for (int32_t i = 0; i < nb; i++) {
        int32_t c = 0;
        for (int32_t t = 0; t < MRA_BLOCK; t++)
            c += (mask == NULL || mask[i * MRA_BLOCK + t]) ? 1 : 0;
        if (cnt)
            cnt[i] = c;
        for (int32_t ch = 0; ch < d; ch++) {
            float acc = 0.0f;
            for (int32_t t = 0; t < MRA_BLOCK; t++) {
                int32_t tok = i * MRA_BLOCK + t;
                if (mask == NULL || mask[tok])
                    acc = acc + x[(int64_t)tok * d + ch];
            }
            xhat[(int64_t)i * d + ch] = c > 0 ? acc / (float)c : 0.0f;
        }
    }
}

/* The same masked block mean in fp64, used for output values only. */
void oracle_pool_f64(int32_t N, int32_t d, const float* x, const uint8_t* mask,
                     double* xhat)
{
    int32_t nb = N / MRA_BLOCK;
    for (int32_t i = 0; i < nb; i++) {
        int32_t c = 0;
        for (int32_t t = 0; t < MRA_BLOCK; t++)
            c += (mask == NULL || mask[i * MRA_BLOCK + t]) ? 1 : 0;
        for (int32_t ch = 0; ch < d; ch++) {
            double acc = 0.0;
            for (int32_t t = 0; t < MRA_BLOCK; t++) {
                int32_t tok = i * MRA_BLOCK + t;
                if (mask == NULL || mask[tok])
                    acc += (double)x[(int64_t)tok * d + ch];
            }
            xhat[(int64_t)i * d + ch] = c > 0 ? acc / (double)c : 0.0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Step 1, low-resolution logits ([MRA] "第一步": query_hat @ key_hat^T),
 * scaled by tau (reading R1).  Canonical fp32 order: a fused multiply-add
 * chain over channels c = 0..d-1 starting from +0.0f, then one multiply by
 * tau_f32 = (float)(1/sqrt(d)).  S: [nb, nb] row-major. */
void oracle_lowres_logits_f32(int32_t nb, int32_t d, const float* qhat,
                              const float* khat, float* S)
{
    float tau = (float)(1.0 / sqrt((double)d));
    for (int32_t i = 0; i < nb; i++)
        for (int32_t j = 0; j < nb; j++) {
            float acc = 0.0f;
            for (int32_t c = 0; c < d; c++)
                acc = fmaf(qhat[(int64_t)i * d + c], khat[(int64_t)j * d + c], acc);
            S[(int64_t)i * nb + j] = acc * tau;
        }
}

/* ------------------------------------------------------------------------ */
/* Step 2, selection scores ([MRA] "第二步"; readings R2, R6, R7, R12).
 *   rowmax_i = max over key blocks j with cnt_j > 0 of S_ij (-inf if none);
 *   score_ij = S_ij - rowmax_i                                      (fp32)
 *            + 5000 if the diagonal prior is on and |i-j| <= floor(g/2)
 *                   (bit 1 of variant: -floor((g-1)/2) <= j-i <= floor(g/2))
 *            + 5000 if i < f   + 5000 if j < f                  (fp32 adds)
 *   score_ij = -inf if cnt_i == 0 or cnt_j == 0;  -0.0 becomes +0.0.
 * variant is a bit set of the readings the step leaves open:
 *   bit 0 (R2')  rank the raw logit S_ij in place of S_ij - rowmax_i ("top-k
 *                on the low-res logits" taken literally), the rest unchanged;
 *   bit 1 (R7')  the diagonal band is exactly g blocks wide, centred on the
 *                main diagonal: offsets j - i in [-floor((g-1)/2), floor(g/2)]
 *                (the same band as R7 for odd g; for even g it leans one
 *                block to the right of the diagonal).
 * rowmax: [nb] (may be NULL), score: [nb, nb]. */
void oracle_scores_f32(int32_t nb, const float* S, const int32_t* cnt,
                       int32_t prior_first, int32_t prior_diag, int32_t variant,
                       float* rowmax, float* score)
{
    for (int32_t i = 0; i < nb; i++) {
        float m = -INFINITY;
        for (int32_t j = 0; j < nb; j++)
            if (cnt[j] > 0 && S[(int64_t)i * nb + j] > m)
                m = S[(int64_t)i * nb + j];
        if (rowmax)
            rowmax[i] = m;
        for (int32_t j = 0; j < nb; j++) {
            float s;
            if (cnt[i] == 0 || cnt[j] == 0) {
                s = -INFINITY;
            } else {
                s = (variant & 1) ? S[(int64_t)i * nb + j] : S[(int64_t)i * nb + j] - m;
                int32_t dist = i > j ? i - j : j - i;
                int32_t in_band = (variant & 2) ? (j - i >= -((prior_diag - 1) / 2) && j - i <= prior_diag / 2)
                                                : dist <= prior_diag / 2;
                if (prior_diag > 0 && in_band)
                    s = s + MRA_PRIOR_BIAS;
                if (i < prior_first)
                    s = s + MRA_PRIOR_BIAS;
                if (j < prior_first)
                    s = s + MRA_PRIOR_BIAS;
                if (s == 0.0f)
                    s = 0.0f; /* canonical +0.0 */
            }
            score[(int64_t)i * nb + j] = s;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Step 2, global top-k ([MRA] "第二步"; readings R3, R5, R13): the K cells
 * that come first in the order (score descending, flat index ascending),
 * written as ascending flat indices.  A library sort is the only tool. */
typedef struct {
    float s;
    int32_t flat;
} cell_t;

static int cell_cmp(const void* a, const void* b)
{
    const cell_t* x = (const cell_t*)a;
    const cell_t* y = (const cell_t*)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return x->flat < y->flat ? -1 : (x->flat > y->flat ? 1 : 0);
}

static int int_cmp(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

int oracle_select_top(int32_t nb, const float* score, int64_t K, int32_t* sel)
{
    int64_t n = (int64_t)nb * nb;
    if (K < 0 || K > n)
        return -1;
    cell_t* cells = (cell_t*)malloc(sizeof(cell_t) * (size_t)n);
    if (!cells)
        return -2;
    for (int64_t f = 0; f < n; f++) {
        cells[f].s = score[f];
        cells[f].flat = (int32_t)f;
    }
    qsort(cells, (size_t)n, sizeof(cell_t), cell_cmp);
    for (int64_t r = 0; r < K; r++)
        sel[r] = cells[r].flat;
    qsort(sel, (size_t)K, sizeof(int32_t), int_cmp);
    free(cells);
    return 0;
}

/* Selection from given fp32 low-res logits and block counts (what the GPU
 * selector is compared against on identical logits). */
int oracle_select_from_logits(int32_t nb, const float* S, const int32_t* cnt,
                              int64_t K, int32_t prior_first, int32_t prior_diag,
                              int32_t variant, int32_t* sel)
{
    float* score = (float*)malloc(sizeof(float) * (size_t)nb * nb);
    if (!score)
        return -2;
    oracle_scores_f32(nb, S, cnt, prior_first, prior_diag, variant, NULL, score);
    int rc = oracle_select_top(nb, score, K, sel);
    free(score);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* One (batch, head) unit of the whole forward pass.
 * q,k,v: [N, d] fp32 values (bf16 inputs arrive widened exactly);
 * mask: [N] or NULL; out: [N, d] fp64; sel: [K] or NULL (ascending flat). */
typedef struct {
    int32_t N, d, block_per_row, mode, prior_first, prior_diag, variant;
} head_args_t;

static int oracle_mra_head(const head_args_t* a, const float* q, const float* k,
                           const float* v, const uint8_t* mask, double* out,
                           int32_t* sel_out)
{
    const int32_t N = a->N, d = a->d, nb = N / MRA_BLOCK;
    const int64_t K = oracle_num_block(N, a->block_per_row);
    const double tau = 1.0 / sqrt((double)d);
    int rc = 0;

    float* qh = (float*)malloc(sizeof(float) * (size_t)nb * d);
    float* kh = (float*)malloc(sizeof(float) * (size_t)nb * d);
    int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)nb);
    float* S = (float*)malloc(sizeof(float) * (size_t)nb * nb);
    float* score = (float*)malloc(sizeof(float) * (size_t)nb * nb);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    uint8_t* chosen = (uint8_t*)calloc((size_t)nb * nb, 1);
    double* qh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* kh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* vh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* s_hi = (double*)malloc(sizeof(double) * (size_t)N);
    double* s_lo = (double*)malloc(sizeof(double) * (size_t)nb);
    if (!qh || !kh || !cnt || !S || !score || !sel || !chosen || !qh64 || !kh64 ||
        !vh64 || !s_hi || !s_lo) {
        rc = -2;
        goto done;
    }

    /* Steps 1 and 2 in fp32: pooled vectors, low-res logits, scores, top-k. */
    oracle_pool_f32(N, d, q, mask, qh, cnt);
    oracle_pool_f32(N, d, k, mask, kh, NULL);
    oracle_lowres_logits_f32(nb, d, qh, kh, S);
    oracle_scores_f32(nb, S, cnt, a->prior_first, a->prior_diag, a->variant, NULL, score);
    rc = oracle_select_top(nb, score, K, sel);
    if (rc)
        goto done;
    for (int64_t r = 0; r < K; r++)
        chosen[sel[r]] = 1;
    if (sel_out)
        memcpy(sel_out, sel, sizeof(int32_t) * (size_t)K);

    /* fp64 pooled vectors for the low-resolution values (step 4). */
    oracle_pool_f64(N, d, q, mask, qh64);
    oracle_pool_f64(N, d, k, mask, kh64);
    oracle_pool_f64(N, d, v, mask, vh64);

    for (int32_t i = 0; i < nb; i++) {
        /* Low-res logits of row i in fp64 for unselected, non-empty key
         * blocks (full mode only; [MRA] step 4 and reading R8). */
        if (a->mode == 0)
            for (int32_t j = 0; j < nb; j++) {
                s_lo[j] = -INFINITY;
                if (!chosen[(int64_t)i * nb + j] && cnt[j] > 0) {
                    double dot = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dot += qh64[(int64_t)i * d + c] * kh64[(int64_t)j * d + c];
                    s_lo[j] = tau * dot;
                }
            }
        for (int32_t t = i * MRA_BLOCK; t < (i + 1) * MRA_BLOCK; t++) {
            double* o = out + (int64_t)t * d;
            for (int32_t c = 0; c < d; c++)
                o[c] = 0.0;
            if (mask && !mask[t])
                continue; /* reading R12: padded query rows output 0 */
            /* Step 3: exact logits on the selected blocks of row i. */
            double shift = -INFINITY;
            for (int32_t j = 0; j < nb; j++) {
                if (!chosen[(int64_t)i * nb + j])
                    continue;
                for (int32_t u = j * MRA_BLOCK; u < (j + 1) * MRA_BLOCK; u++) {
                    s_hi[u] = -INFINITY;
                    if (mask && !mask[u])
                        continue;
                    double dot = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dot += (double)q[(int64_t)t * d + c] * (double)k[(int64_t)u * d + c];
                    s_hi[u] = tau * dot;
                    if (s_hi[u] > shift)
                        shift = s_hi[u];
                }
            }
            if (a->mode == 0)
                for (int32_t j = 0; j < nb; j++)
                    if (s_lo[j] > shift)
                        shift = s_lo[j];
            if (shift == -INFINITY)
                continue; /* nothing to attend to: 0/0 gives 0 (R11) */
            double den = 0.0;
            for (int32_t c = 0; c < d; c++)
                o[c] = 0.0;
            for (int32_t j = 0; j < nb; j++) {
                if (!chosen[(int64_t)i * nb + j])
                    continue;
                for (int32_t u = j * MRA_BLOCK; u < (j + 1) * MRA_BLOCK; u++) {
                    if (s_hi[u] == -INFINITY)
                        continue;
                    double w = exp(s_hi[u] - shift);
                    den += w;
                    for (int32_t c = 0; c < d; c++)
                        o[c] += w * (double)v[(int64_t)u * d + c];
                }
            }
            /* Step 4, full mode: the low-resolution attention on the
             * unselected blocks, each cell weighted by its count (R9). */
            if (a->mode == 0)
                for (int32_t j = 0; j < nb; j++) {
                    if (s_lo[j] == -INFINITY)
                        continue;
                    double w = (double)cnt[j] * exp(s_lo[j] - shift);
                    den += w;
                    for (int32_t c = 0; c < d; c++)
                        o[c] += w * vh64[(int64_t)j * d + c];
                }
            if (den > 0.0)
                for (int32_t c = 0; c < d; c++)
                    o[c] /= den;
            else
                for (int32_t c = 0; c < d; c++)
                    o[c] = 0.0;
        }
    }

done:
    free(qh); free(kh); free(cnt); free(S); free(score); free(sel); free(chosen);
    free(qh64); free(kh64); free(vh64); free(s_hi); free(s_lo);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Dense reference: softmax(tau * q k^T over valid keys) v for each valid
 * query token ([MHRA] "global MHRA", reading R1 for tau); masked query
 * rows and rows with no valid key give 0. */
static int oracle_dense_head(int32_t N, int32_t d, const float* q, const float* k,
                             const float* v, const uint8_t* mask, double* out)
{
    const double tau = 1.0 / sqrt((double)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    if (!s)
        return -2;
    for (int32_t t = 0; t < N; t++) {
        double* o = out + (int64_t)t * d;
        for (int32_t c = 0; c < d; c++)
            o[c] = 0.0;
        if (mask && !mask[t])
            continue;
        double shift = -INFINITY;
        for (int32_t u = 0; u < N; u++) {
            s[u] = -INFINITY;
            if (mask && !mask[u])
                continue;
            double dot = 0.0;
            for (int32_t c = 0; c < d; c++)
                dot += (double)q[(int64_t)t * d + c] * (double)k[(int64_t)u * d + c];
            s[u] = tau * dot;
            if (s[u] > shift)
                shift = s[u];
        }
        if (shift == -INFINITY)
            continue;
        double den = 0.0;
        for (int32_t u = 0; u < N; u++) {
            if (s[u] == -INFINITY)
                continue;
            double w = exp(s[u] - shift);
            den += w;
            for (int32_t c = 0; c < d; c++)
                o[c] += w * (double)v[(int64_t)u * d + c];
        }
        for (int32_t c = 0; c < d; c++)
            o[c] /= den;
    }
    free(s);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Gradients of one (batch, head) unit of the forward pass above with respect
 * to q, k and v, given dO = dL/d out.  [MRA] "第三步": the block products are
 * autograd functions whose backward reuses the kernels on transposed block
 * indices, so the selection (a top-k, step 2) is a constant of the backward
 * pass; "第四步": in full mode the low-resolution branch is ordinary tensor
 * code, so it is differentiated too, down through the block means.
 *
 * With the selection fixed, for a valid query token t of block row i:
 *   out_t = (sum_u w_u v_u + sum_j W_j vhat_j) / (sum_u w_u + sum_j W_j),
 *   w_u = e^{s_u}, s_u = tau q_t . k_u      (u: valid keys of selected blocks)
 *   W_j = cnt_j e^{shat_ij}, shat_ij = tau qhat_i . khat_j
 *                          (j: unselected non-empty blocks; full mode only)
 * With Z the denominator, P_u = w_u / Z, Pi_j = W_j / Z, D_t = dO_t . out_t:
 *   dv_u     += P_u dO_t                  dvhat_j  += Pi_j dO_t
 *   ds_u      = P_u (dO_t . v_u - D_t)    dshat_ij  = Pi_j (dO_t . vhat_j - D_t)
 *   dq_t     += tau ds_u k_u              dk_u     += tau ds_u q_t
 *   dqhat_i  += tau dshat_ij khat_j       dkhat_j  += tau dshat_ij qhat_i
 * and a block mean passes its gradient to each valid token of the block
 * divided by the block's count.  Padded query rows (zero output) pass no
 * gradient; empty blocks have zero means and no weight.
 * dout: [N, d] fp32; dq, dk, dv: [N, d] fp64, overwritten. */
static int oracle_mra_head_bwd(const head_args_t* a, const float* q, const float* k,
                               const float* v, const uint8_t* mask, const float* dout,
                               double* dq, double* dk, double* dv)
{
    const int32_t N = a->N, d = a->d, nb = N / MRA_BLOCK;
    const int64_t K = oracle_num_block(N, a->block_per_row);
    const double tau = 1.0 / sqrt((double)d);
    const int full = a->mode == 0;
    int rc = 0;

    float* qh = (float*)malloc(sizeof(float) * (size_t)nb * d);
    float* kh = (float*)malloc(sizeof(float) * (size_t)nb * d);
    int32_t* cnt = (int32_t*)malloc(sizeof(int32_t) * (size_t)nb);
    float* S = (float*)malloc(sizeof(float) * (size_t)nb * nb);
    float* score = (float*)malloc(sizeof(float) * (size_t)nb * nb);
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)(K > 0 ? K : 1));
    uint8_t* chosen = (uint8_t*)calloc((size_t)nb * nb, 1);
    double* qh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* kh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* vh64 = (double*)malloc(sizeof(double) * (size_t)nb * d);
    double* dqh = (double*)calloc((size_t)nb * d, sizeof(double));
    double* dkh = (double*)calloc((size_t)nb * d, sizeof(double));
    double* dvh = (double*)calloc((size_t)nb * d, sizeof(double));
    double* s_hi = (double*)malloc(sizeof(double) * (size_t)N);
    double* s_lo = (double*)malloc(sizeof(double) * (size_t)nb);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!qh || !kh || !cnt || !S || !score || !sel || !chosen || !qh64 || !kh64 || !vh64 ||
        !dqh || !dkh || !dvh || !s_hi || !s_lo || !o) {
        rc = -2;
        goto done;
    }
    memset(dq, 0, sizeof(double) * (size_t)N * d);
    memset(dk, 0, sizeof(double) * (size_t)N * d);
    memset(dv, 0, sizeof(double) * (size_t)N * d);

    /* the forward's selection, made exactly as oracle_mra_head makes it */
    oracle_pool_f32(N, d, q, mask, qh, cnt);
    oracle_pool_f32(N, d, k, mask, kh, NULL);
    oracle_lowres_logits_f32(nb, d, qh, kh, S);
    oracle_scores_f32(nb, S, cnt, a->prior_first, a->prior_diag, a->variant, NULL, score);
    rc = oracle_select_top(nb, score, K, sel);
    if (rc)
        goto done;
    for (int64_t r = 0; r < K; r++)
        chosen[sel[r]] = 1;
    oracle_pool_f64(N, d, q, mask, qh64);
    oracle_pool_f64(N, d, k, mask, kh64);
    oracle_pool_f64(N, d, v, mask, vh64);

    for (int32_t i = 0; i < nb; i++) {
        if (full)
            for (int32_t j = 0; j < nb; j++) {
                s_lo[j] = -INFINITY;
                if (!chosen[(int64_t)i * nb + j] && cnt[j] > 0) {
                    double dot = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dot += qh64[(int64_t)i * d + c] * kh64[(int64_t)j * d + c];
                    s_lo[j] = tau * dot;
                }
            }
        for (int32_t t = i * MRA_BLOCK; t < (i + 1) * MRA_BLOCK; t++) {
            if (mask && !mask[t])
                continue;
            const float* g = dout + (int64_t)t * d;
            double shift = -INFINITY;
            for (int32_t j = 0; j < nb; j++) {
                if (!chosen[(int64_t)i * nb + j])
                    continue;
                for (int32_t u = j * MRA_BLOCK; u < (j + 1) * MRA_BLOCK; u++) {
                    s_hi[u] = -INFINITY;
                    if (mask && !mask[u])
                        continue;
                    double dot = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dot += (double)q[(int64_t)t * d + c] * (double)k[(int64_t)u * d + c];
                    s_hi[u] = tau * dot;
                    if (s_hi[u] > shift)
                        shift = s_hi[u];
                }
            }
            if (full)
                for (int32_t j = 0; j < nb; j++)
                    if (s_lo[j] > shift)
                        shift = s_lo[j];
            if (shift == -INFINITY)
                continue;
            /* the forward quantities of token t: Z and out_t */
            double Z = 0.0;
            for (int32_t c = 0; c < d; c++)
                o[c] = 0.0;
            for (int32_t j = 0; j < nb; j++) {
                if (!chosen[(int64_t)i * nb + j])
                    continue;
                for (int32_t u = j * MRA_BLOCK; u < (j + 1) * MRA_BLOCK; u++) {
                    if (s_hi[u] == -INFINITY)
                        continue;
                    const double w = exp(s_hi[u] - shift);
                    Z += w;
                    for (int32_t c = 0; c < d; c++)
                        o[c] += w * (double)v[(int64_t)u * d + c];
                }
            }
            if (full)
                for (int32_t j = 0; j < nb; j++) {
                    if (s_lo[j] == -INFINITY)
                        continue;
                    const double w = (double)cnt[j] * exp(s_lo[j] - shift);
                    Z += w;
                    for (int32_t c = 0; c < d; c++)
                        o[c] += w * vh64[(int64_t)j * d + c];
                }
            if (!(Z > 0.0))
                continue;
            double D = 0.0;
            for (int32_t c = 0; c < d; c++) {
                o[c] /= Z;
                D += (double)g[c] * o[c];
            }
            /* high-resolution terms */
            for (int32_t j = 0; j < nb; j++) {
                if (!chosen[(int64_t)i * nb + j])
                    continue;
                for (int32_t u = j * MRA_BLOCK; u < (j + 1) * MRA_BLOCK; u++) {
                    if (s_hi[u] == -INFINITY)
                        continue;
                    const double P = exp(s_hi[u] - shift) / Z;
                    double dP = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dP += (double)g[c] * (double)v[(int64_t)u * d + c];
                    const double ds = P * (dP - D);
                    for (int32_t c = 0; c < d; c++) {
                        dv[(int64_t)u * d + c] += P * (double)g[c];
                        dq[(int64_t)t * d + c] += tau * ds * (double)k[(int64_t)u * d + c];
                        dk[(int64_t)u * d + c] += tau * ds * (double)q[(int64_t)t * d + c];
                    }
                }
            }
            /* low-resolution terms (full mode), onto the block means */
            if (full)
                for (int32_t j = 0; j < nb; j++) {
                    if (s_lo[j] == -INFINITY)
                        continue;
                    const double Pi = (double)cnt[j] * exp(s_lo[j] - shift) / Z;
                    double dPi = 0.0;
                    for (int32_t c = 0; c < d; c++)
                        dPi += (double)g[c] * vh64[(int64_t)j * d + c];
                    const double ds = Pi * (dPi - D);
                    for (int32_t c = 0; c < d; c++) {
                        dvh[(int64_t)j * d + c] += Pi * (double)g[c];
                        dqh[(int64_t)i * d + c] += tau * ds * kh64[(int64_t)j * d + c];
                        dkh[(int64_t)j * d + c] += tau * ds * qh64[(int64_t)i * d + c];
                    }
                }
        }
    }
    /* a block mean's gradient goes to each valid token of the block / cnt */
    if (full)
        for (int32_t b = 0; b < nb; b++) {
            if (cnt[b] <= 0)
                continue;
            const double inv = 1.0 / (double)cnt[b];
            for (int32_t t = b * MRA_BLOCK; t < (b + 1) * MRA_BLOCK; t++) {
                if (mask && !mask[t])
                    continue;
                for (int32_t c = 0; c < d; c++) {
                    dq[(int64_t)t * d + c] += dqh[(int64_t)b * d + c] * inv;
                    dk[(int64_t)t * d + c] += dkh[(int64_t)b * d + c] * inv;
                    dv[(int64_t)t * d + c] += dvh[(int64_t)b * d + c] * inv;
                }
            }
        }

done:
    free(qh); free(kh); free(cnt); free(S); free(score); free(sel); free(chosen);
    free(qh64); free(kh64); free(vh64); free(dqh); free(dkh); free(dvh);
    free(s_hi); free(s_lo); free(o);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* BigBird block-sparse attention ([BigBird], the description of its three
 * attention patterns, the usage notes and the BigBirdConfig table): the
 * sequence is cut into nbb = N / bs blocks and query block I attends key
 * block J when
 *   I is a global block or J is a global block (the first and the last
 *     block: two global blocks; reading B1),
 *   |I - J| <= 1 (a window of three blocks, clipped at the ends; B2), or
 *   J is one of row I's r random picks rand[I][0 .. r-1] (drawn outside and
 *     passed in; a block is attended once however often it is named, and
 *     picks outside [0, nbb) name nothing; B3).
 * Each valid query token then takes exact softmax attention, scale
 * 1/sqrt(d), over the valid keys of its attended blocks (B4); padded query
 * rows and rows with no valid key output 0.  rand: [nbb, r]. */
/* The attended-block matrix att [nbb, nbb] of the pattern described below. */
static void bigbird_pattern(int32_t nbb, int32_t r, const int32_t* rand, uint8_t* att)
{
    for (int32_t I = 0; I < nbb; I++)
        for (int32_t J = 0; J < nbb; J++) {
            const int global = I == 0 || I == nbb - 1 || J == 0 || J == nbb - 1;
            const int window = I - J <= 1 && J - I <= 1;
            att[(int64_t)I * nbb + J] = (uint8_t)(global || window);
        }
    for (int32_t I = 0; I < nbb; I++)
        for (int32_t x = 0; x < r; x++) {
            const int32_t J = rand[(int64_t)I * r + x];
            if (J >= 0 && J < nbb)
                att[(int64_t)I * nbb + J] = 1;
        }
}

static int oracle_bigbird_head(int32_t N, int32_t d, int32_t bs, int32_t r, const int32_t* rand,
                               const float* q, const float* k, const float* v, const uint8_t* mask,
                               double* out)
{
    const int32_t nbb = N / bs;
    const double tau = 1.0 / sqrt((double)d);
    uint8_t* att = (uint8_t*)calloc((size_t)nbb * nbb, 1);
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    if (!att || !s) {
        free(att);
        free(s);
        return -2;
    }
    bigbird_pattern(nbb, r, rand, att);
    for (int32_t t = 0; t < N; t++) {
        double* o = out + (int64_t)t * d;
        for (int32_t c = 0; c < d; c++)
            o[c] = 0.0;
        if (mask && !mask[t])
            continue;
        double shift = -INFINITY;
        for (int32_t u = 0; u < N; u++) {
            s[u] = -INFINITY;
            if ((mask && !mask[u]) || !att[(int64_t)(t / bs) * nbb + u / bs])
                continue;
            double dot = 0.0;
            for (int32_t c = 0; c < d; c++)
                dot += (double)q[(int64_t)t * d + c] * (double)k[(int64_t)u * d + c];
            s[u] = tau * dot;
            if (s[u] > shift)
                shift = s[u];
        }
        if (shift == -INFINITY)
            continue;
        double den = 0.0;
        for (int32_t u = 0; u < N; u++) {
            if (s[u] == -INFINITY)
                continue;
            const double w = exp(s[u] - shift);
            den += w;
            for (int32_t c = 0; c < d; c++)
                o[c] += w * (double)v[(int64_t)u * d + c];
        }
        for (int32_t c = 0; c < d; c++)
            o[c] /= den;
    }
    free(att);
    free(s);
    return 0;
}

/* Gradients of oracle_bigbird_head's output with respect to q, k and v,
 * given dO = dL/d out.  The pattern depends on block positions and the given
 * picks only, so it is a constant; for a valid query token t and the valid
 * keys u of its attended blocks, with P_u = e^{s_u} / Z and D_t = dO_t . out_t:
 *   dS_u = P_u (dO_t . v_u - D_t),  dq_t += tau dS_u k_u,
 *   dk_u += tau dS_u q_t,           dv_u += P_u dO_t.
 * dout: [N, d] fp32; dq, dk, dv: [N, d] fp64, overwritten. */
static int oracle_bigbird_head_bwd(int32_t N, int32_t d, int32_t bs, int32_t r, const int32_t* rand,
                                   const float* q, const float* k, const float* v, const uint8_t* mask,
                                   const float* dout, double* dq, double* dk, double* dv)
{
    const int32_t nbb = N / bs;
    const double tau = 1.0 / sqrt((double)d);
    uint8_t* att = (uint8_t*)calloc((size_t)nbb * nbb, 1);
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    if (!att || !s || !o) {
        free(att); free(s); free(o);
        return -2;
    }
    bigbird_pattern(nbb, r, rand, att);
    memset(dq, 0, sizeof(double) * (size_t)N * d);
    memset(dk, 0, sizeof(double) * (size_t)N * d);
    memset(dv, 0, sizeof(double) * (size_t)N * d);
    for (int32_t t = 0; t < N; t++) {
        if (mask && !mask[t])
            continue;
        const float* g = dout + (int64_t)t * d;
        double shift = -INFINITY;
        for (int32_t u = 0; u < N; u++) {
            s[u] = -INFINITY;
            if ((mask && !mask[u]) || !att[(int64_t)(t / bs) * nbb + u / bs])
                continue;
            double dot = 0.0;
            for (int32_t c = 0; c < d; c++)
                dot += (double)q[(int64_t)t * d + c] * (double)k[(int64_t)u * d + c];
            s[u] = tau * dot;
            if (s[u] > shift)
                shift = s[u];
        }
        if (shift == -INFINITY)
            continue;
        double Z = 0.0;
        for (int32_t c = 0; c < d; c++)
            o[c] = 0.0;
        for (int32_t u = 0; u < N; u++) {
            if (s[u] == -INFINITY)
                continue;
            const double w = exp(s[u] - shift);
            Z += w;
            for (int32_t c = 0; c < d; c++)
                o[c] += w * (double)v[(int64_t)u * d + c];
        }
        double D = 0.0;
        for (int32_t c = 0; c < d; c++)
            D += (double)g[c] * (o[c] / Z);
        for (int32_t u = 0; u < N; u++) {
            if (s[u] == -INFINITY)
                continue;
            const double P = exp(s[u] - shift) / Z;
            double dP = 0.0;
            for (int32_t c = 0; c < d; c++)
                dP += (double)g[c] * (double)v[(int64_t)u * d + c];
            const double ds = P * (dP - D);
            for (int32_t c = 0; c < d; c++) {
                dv[(int64_t)u * d + c] += P * (double)g[c];
                dq[(int64_t)t * d + c] += tau * ds * (double)k[(int64_t)u * d + c];
                dk[(int64_t)u * d + c] += tau * ds * (double)q[(int64_t)t * d + c];
            }
        }
    }
    free(att); free(s); free(o);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Batched drivers: independent (batch, head) units spread over nthreads
 * POSIX threads.  Each unit is computed by exactly the code above; the
 * threads only decide which unit runs where. */
typedef struct {
    int32_t B, H, N, d;
    const float *q, *k, *v;
    const uint8_t* mask;
    head_args_t ha;
    double* out;
    int32_t* sel;
    int64_t K;
    int dense;
    int bwd;           /* gradients: dout in, dq / dk / dv out */
    int bigbird;       /* BigBird pattern: block size bs, r picks per block row */
    int32_t bs, r;
    const int32_t* rand;
    const float* dout;
    double *dq, *dk, *dv;
    int next; /* shared unit counter */
    int rc;
} job_t;

static void* worker(void* p)
{
    job_t* j = (job_t*)p;
    const int units = j->B * j->H;
    for (;;) {
        int u = __atomic_fetch_add(&j->next, 1, __ATOMIC_RELAXED);
        if (u >= units)
            break;
        int b = u / j->H;
        int64_t off = (int64_t)u * j->N * j->d;
        const uint8_t* m = j->mask ? j->mask + (int64_t)b * j->N : NULL;
        int rc;
        if (j->bigbird && j->bwd)
            rc = oracle_bigbird_head_bwd(j->N, j->d, j->bs, j->r,
                                         j->rand + (int64_t)u * (j->N / j->bs) * j->r, j->q + off,
                                         j->k + off, j->v + off, m, j->dout + off, j->dq + off,
                                         j->dk + off, j->dv + off);
        else if (j->bigbird)
            rc = oracle_bigbird_head(j->N, j->d, j->bs, j->r,
                                     j->rand + (int64_t)u * (j->N / j->bs) * j->r, j->q + off,
                                     j->k + off, j->v + off, m, j->out + off);
        else if (j->bwd)
            rc = oracle_mra_head_bwd(&j->ha, j->q + off, j->k + off, j->v + off, m, j->dout + off,
                                     j->dq + off, j->dk + off, j->dv + off);
        else if (j->dense)
            rc = oracle_dense_head(j->N, j->d, j->q + off, j->k + off, j->v + off, m,
                                   j->out + off);
        else
            rc = oracle_mra_head(&j->ha, j->q + off, j->k + off, j->v + off, m,
                                 j->out + off, j->sel ? j->sel + (int64_t)u * j->K : NULL);
        if (rc)
            __atomic_store_n(&j->rc, rc, __ATOMIC_RELAXED);
    }
    return NULL;
}

static int run_jobs(job_t* j, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    int started = 0;
    for (int t = 1; t < nthreads; t++)
        if (pthread_create(&th[started], NULL, worker, j) == 0)
            started++;
    worker(j);
    for (int t = 0; t < started; t++)
        pthread_join(th[t], NULL);
    return j->rc;
}

/* MRA-2 forward over [B, H, N, d] inputs.  mode 0 = "full", 1 = "sparse".
 * Returns 0, or -1 for invalid arguments, -2 when out of memory. */
int oracle_mra_fwd(int32_t B, int32_t H, int32_t N, int32_t d, const float* q,
                   const float* k, const float* v, const uint8_t* mask,
                   int32_t block_per_row, int32_t mode, int32_t prior_first,
                   int32_t prior_diag, int32_t variant, double* out, int32_t* sel,
                   int32_t nthreads)
{
    int64_t K = oracle_num_block(N, block_per_row);
    if (B < 1 || H < 1 || d < 1 || K < 0 || (mode != 0 && mode != 1) ||
        prior_first < 0 || prior_diag < 0 || (variant & ~3) != 0 || !q || !k || !v || !out)
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.B = B; j.H = H; j.N = N; j.d = d;
    j.q = q; j.k = k; j.v = v; j.mask = mask;
    j.ha.N = N; j.ha.d = d; j.ha.block_per_row = block_per_row; j.ha.mode = mode;
    j.ha.prior_first = prior_first; j.ha.prior_diag = prior_diag; j.ha.variant = variant;
    j.out = out; j.sel = sel; j.K = K; j.dense = 0;
    return run_jobs(&j, nthreads);
}

/* Dense softmax attention over [B, H, N, d] inputs (any N >= 1). */
int oracle_dense_fwd(int32_t B, int32_t H, int32_t N, int32_t d, const float* q,
                     const float* k, const float* v, const uint8_t* mask,
                     double* out, int32_t nthreads)
{
    if (B < 1 || H < 1 || N < 1 || d < 1 || !q || !k || !v || !out)
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.B = B; j.H = H; j.N = N; j.d = d;
    j.q = q; j.k = k; j.v = v; j.mask = mask;
    j.out = out; j.dense = 1;
    return run_jobs(&j, nthreads);
}

/* Gradients of the MRA-2 forward over [B, H, N, d] inputs with respect to
 * q, k and v (oracle_mra_head_bwd), given dout = dL/d out.  Returns 0, or -1
 * for invalid arguments, -2 when out of memory. */
int oracle_mra_bwd(int32_t B, int32_t H, int32_t N, int32_t d, const float* q,
                   const float* k, const float* v, const uint8_t* mask,
                   int32_t block_per_row, int32_t mode, int32_t prior_first,
                   int32_t prior_diag, int32_t variant, const float* dout, double* dq,
                   double* dk, double* dv, int32_t nthreads)
{
    int64_t K = oracle_num_block(N, block_per_row);
    if (B < 1 || H < 1 || d < 1 || K < 0 || (mode != 0 && mode != 1) ||
        prior_first < 0 || prior_diag < 0 || (variant & ~3) != 0 || !q || !k || !v ||
        !dout || !dq || !dk || !dv)
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.B = B; j.H = H; j.N = N; j.d = d;
    j.q = q; j.k = k; j.v = v; j.mask = mask;
    j.ha.N = N; j.ha.d = d; j.ha.block_per_row = block_per_row; j.ha.mode = mode;
    j.ha.prior_first = prior_first; j.ha.prior_diag = prior_diag; j.ha.variant = variant;
    j.K = K; j.bwd = 1; j.dout = dout; j.dq = dq; j.dk = dk; j.dv = dv;
    return run_jobs(&j, nthreads);
}

/* BigBird block-sparse attention (oracle_bigbird_head) over [B, H, N, d]
 * inputs; rand: [B, H, N / bs, r].  Returns 0, or -1 for invalid arguments
 * (N not a positive multiple of bs, r < 0), -2 when out of memory. */
int oracle_bigbird_fwd(int32_t B, int32_t H, int32_t N, int32_t d, const float* q,
                       const float* k, const float* v, const uint8_t* mask, int32_t bs,
                       int32_t r, const int32_t* rand, double* out, int32_t nthreads)
{
    if (B < 1 || H < 1 || d < 1 || bs < 1 || N < bs || N % bs != 0 || r < 0 ||
        (r > 0 && !rand) || !q || !k || !v || !out)
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.B = B; j.H = H; j.N = N; j.d = d;
    j.q = q; j.k = k; j.v = v; j.mask = mask;
    j.out = out; j.bigbird = 1; j.bs = bs; j.r = r; j.rand = rand;
    return run_jobs(&j, nthreads);
}

/* Gradients of oracle_bigbird_fwd's output (oracle_bigbird_head_bwd) given
 * dout; all [B, H, N, d], rand [B, H, N / bs, r]. */
int oracle_bigbird_bwd(int32_t B, int32_t H, int32_t N, int32_t d, const float* q,
                       const float* k, const float* v, const uint8_t* mask, int32_t bs,
                       int32_t r, const int32_t* rand, const float* dout, double* dq, double* dk,
                       double* dv, int32_t nthreads)
{
    if (B < 1 || H < 1 || d < 1 || bs < 1 || N < bs || N % bs != 0 || r < 0 ||
        (r > 0 && !rand) || !q || !k || !v || !dout || !dq || !dk || !dv)
        return -1;
    job_t j;
    memset(&j, 0, sizeof(j));
    j.B = B; j.H = H; j.N = N; j.d = d;
    j.q = q; j.k = k; j.v = v; j.mask = mask;
    j.bigbird = 1; j.bs = bs; j.r = r; j.rand = rand;
    j.bwd = 1; j.dout = dout; j.dq = dq; j.dk = dk; j.dv = dv;
    return run_jobs(&j, nthreads);
}
