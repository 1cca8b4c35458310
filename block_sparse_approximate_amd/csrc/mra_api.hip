// mra_api.hip — host side of the C ABI declared in include/mra.h:
// argument checks, workspace carve and the launch sequence on one stream.
//
//   pool      step 1 pooling, counts, mask words; clears the selection
//             histogram
//   logits    step 1 low-res logits, row maxima, selection-key histogram
//   select    step 2 top-K selection: bitmap, CSR, attention stream records
//   attn      steps 3 and 4: block attention, the low-res merge (full mode)
//             and the join of rows cut into several segments or with no
//             selected block
// Everything after the argument checks is asynchronous; nothing here waits.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "../../include/mra.h"
#include "mra_common.h"

#define MRA_API extern "C" __attribute__((visibility("default")))

namespace mra {
namespace {

constexpr int32_t kAbiVersion = 4;
constexpr int32_t kMaxSeqLen = 16384;

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

bool carve(const mra_dims& d, int32_t bpr, int32_t mode, Layout* L) {
    L->B = d.batch; L->H = d.heads; L->N = d.seq_len; L->d = d.head_dim;
    L->nb = d.seq_len / kBlock;
    L->BH = d.batch * d.heads;
    L->K = mra_num_block(d.seq_len, bpr);
    if (L->K < 0) return false;
    L->max_items = L->nb + (int32_t)((L->K + kChunkMin - 1) / kChunkMin);   // segments of kChunkMin or more
    const size_t BH = (size_t)L->BH, nb = (size_t)L->nb, dd = (size_t)d.head_dim;
    const size_t words = (nb + 31) / 32;
    size_t o = 256;  // first 256 bytes: device error word
    auto take = [&](size_t bytes) { size_t at = o; o = up256(o + bytes); return at; };
    L->qhat = take(BH * nb * dd * 4);
    L->khat = take(BH * nb * dd * 4);
    L->vhat = mode == MRA_APPROX_FULL ? take(BH * nb * dd * 4) : 0;
    L->cnt = take((size_t)d.batch * nb * 4);
    L->mbits = take((size_t)d.batch * nb * 4);
    L->logits = take(BH * nb * nb * 4);
    L->keys = take(BH * nb * nb * 4);
    L->rowmax = take(BH * nb * 4);
    L->hist = take(BH * kHistBins * 4);
    L->thresh = take(BH * 8);
    L->row_ptr = take(BH * (nb + 1) * 4);
    L->col = take(BH * (size_t)L->K * 4);
    L->selbits = take(BH * nb * words * 4);
    L->item_ptr = take(BH * (nb + 1) * 4);
    L->recs = take(BH * (size_t)L->K * sizeof(BlkRec));
    L->merge_rows = take(BH * nb * 16);
    L->n_merge = take(BH * 4);
    L->join_cnt = take(BH * nb * 4);
    L->lo_all = mode == MRA_APPROX_FULL ? take(BH * nb * dd * 4) : 0;
    L->ll_all = mode == MRA_APPROX_FULL ? take(BH * nb * 4) : 0;
    L->part_o = take(BH * (size_t)L->max_items * kBlock * dd * 4);
    L->part_ml = take(BH * (size_t)L->max_items * 2 * kBlock * 4);
    L->part_corr = mode == MRA_APPROX_FULL ? take(BH * (size_t)L->max_items * corr_stride(d.head_dim) * 4) : 0;
    L->park = take(BH * (size_t)attn_grid_waves_per_head(L->BH, L->K, d.head_dim) * park_floats(d.head_dim) * 4);
    L->cand = take(BH * (size_t)kSelCap * 8);
    L->ncand = take(BH * kCandStride * 4);
    L->st_m = take(BH * (size_t)L->N * 4);
    L->st_linv = take(BH * (size_t)L->N * 4);
    L->total = o;
    return true;
}

// The backward pass's own workspace (mra_attention_bwd).
struct BwdLayout {
    int32_t maxch;
    size_t st_d, ct_ptr, ct_row, rch, cch, rmul, cmul, count, part_dq, part_dk, part_dv, g, c, et, wt, dqh, dkh,
        dvh, total;
};

void carve_bwd(const Layout& L, int32_t mode, BwdLayout* W) {
    const size_t BH = (size_t)L.BH, nb = (size_t)L.nb;
    W->maxch = bwd_max_chunks(L.nb, L.K);
    const size_t slots = BH * (size_t)W->maxch, tile = (size_t)kBlock * L.d * 4;
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o = up256(o + bytes); return at; };
    W->st_d = take(BH * (size_t)L.N * 4);
    W->ct_ptr = take(BH * (nb + 1) * 4);
    W->ct_row = take(BH * (size_t)L.K * 4);
    W->rch = take(slots * 16);
    W->cch = take(slots * 16);
    W->rmul = take(BH * nb * 16);
    W->cmul = take(BH * nb * 16);
    W->count = take(BH * 16);
    W->part_dq = take(slots * tile);
    W->part_dk = take(slots * tile);
    W->part_dv = take(slots * tile);
    const bool full = mode == MRA_APPROX_FULL;
    const size_t blk = BH * nb * (size_t)L.d * 4, cell = BH * nb * nb * 4;
    W->g = full ? take(blk) : 0;
    W->c = full ? take(BH * nb * 4) : 0;
    W->et = full ? take(cell) : 0;
    W->wt = full ? take(cell) : 0;
    W->dqh = full ? take(blk) : 0;
    W->dkh = full ? take(blk) : 0;
    W->dvh = full ? take(blk) : 0;
    W->total = o;
}

mra_status check_dims(const mra_dims* d) {
    if (!d) return MRA_ERR_NULL;
    if (d->batch < 1 || d->heads < 1) return MRA_ERR_SHAPE;
    if (d->seq_len < kBlock || d->seq_len % kBlock != 0 || d->seq_len > kMaxSeqLen) return MRA_ERR_SEQ_LEN;
    if (d->head_dim != kHeadDim && d->head_dim != kMaxHeadDim) return MRA_ERR_HEAD_DIM;
    if (d->scale_dim < 0 || d->scale_dim > d->head_dim) return MRA_ERR_HEAD_DIM;
    if (d->dtype != MRA_F32 && d->dtype != MRA_BF16) return MRA_ERR_DTYPE;
    if ((int64_t)d->batch * d->heads > (1 << 20)) return MRA_ERR_SHAPE;
    return MRA_OK;
}

mra_status check_params(int32_t bpr, int32_t mode, int32_t pf, int32_t pd) {
    if (mode != MRA_APPROX_FULL && mode != MRA_APPROX_SPARSE) return MRA_ERR_MODE;
    if (bpr < 1) return MRA_ERR_BUDGET;
    if (pf < 0 || pd < 0) return MRA_ERR_PRIOR;
    return MRA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

Params make_params(const mra_dims& d, const Layout& L, int32_t mode, int32_t pf, int32_t pd, const void* q,
                   const void* k, const void* v, const uint8_t* mask, void* out, void* ws, int32_t ranking = 0,
                   int32_t band = MRA_BAND_SYMMETRIC, int32_t save_stats = 0) {
    Params p;
    memset(&p, 0, sizeof(p));
    unsigned char* w = static_cast<unsigned char*>(ws);
    p.B = L.B; p.H = L.H; p.N = L.N; p.d = L.d; p.nb = L.nb; p.BH = L.BH;
    p.dscale = d.scale_dim > 0 ? d.scale_dim : d.head_dim;
    p.words = (L.nb + 31) / 32;
    p.K = L.K;
    p.mode = mode;
    p.dtype = d.dtype;
    p.prior_first = pf;
    p.prior_diag = pd;
    p.rank_raw = ranking == MRA_RANK_RAW_LOGITS ? 1 : 0;
    p.band_exact = band == MRA_BAND_EXACT ? 1 : 0;
    p.save_stats = save_stats ? 1 : 0;
    p.max_items = L.max_items;
    p.attn_wph = attn_grid_waves_per_head(L.BH, L.K, L.d);
    p.attn_seq = attn_heads_in_turn(L.BH, L.K, L.d) ? 1 : 0;
    attn_segments(L.BH, L.K, L.d, &p.seg_whole, &p.chunk);
    p.v_in_logits = v != nullptr && v_pooled_in_logits(mode, L.BH, L.nb, L.d) ? 1 : 0;
    p.q = q; p.k = k; p.v = v; p.mask = mask; p.out = out;
    p.qhat = reinterpret_cast<float*>(w + L.qhat);
    p.khat = reinterpret_cast<float*>(w + L.khat);
    p.vhat = L.vhat ? reinterpret_cast<float*>(w + L.vhat) : nullptr;
    p.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
    p.mbits = reinterpret_cast<uint32_t*>(w + L.mbits);
    p.logits = reinterpret_cast<float*>(w + L.logits);
    p.keys = reinterpret_cast<uint32_t*>(w + L.keys);
    p.rowmax = reinterpret_cast<float*>(w + L.rowmax);
    p.hist = reinterpret_cast<uint32_t*>(w + L.hist);
    p.thresh = reinterpret_cast<uint64_t*>(w + L.thresh);
    p.row_ptr = reinterpret_cast<int32_t*>(w + L.row_ptr);
    p.col = reinterpret_cast<int32_t*>(w + L.col);
    p.selbits = reinterpret_cast<uint32_t*>(w + L.selbits);
    p.item_ptr = reinterpret_cast<int32_t*>(w + L.item_ptr);
    p.recs = reinterpret_cast<BlkRec*>(w + L.recs);
    p.merge_rows = reinterpret_cast<int4*>(w + L.merge_rows);
    p.n_merge = reinterpret_cast<int32_t*>(w + L.n_merge);
    p.join_cnt = reinterpret_cast<uint32_t*>(w + L.join_cnt);
    p.lo_all = L.lo_all ? reinterpret_cast<float*>(w + L.lo_all) : nullptr;
    p.ll_all = L.ll_all ? reinterpret_cast<float*>(w + L.ll_all) : nullptr;
    p.part_o = reinterpret_cast<float*>(w + L.part_o);
    p.part_ml = reinterpret_cast<float*>(w + L.part_ml);
    p.part_corr = L.part_corr ? reinterpret_cast<float*>(w + L.part_corr) : nullptr;
    p.park = reinterpret_cast<float*>(w + L.park);
    p.cand = reinterpret_cast<uint64_t*>(w + L.cand);
    p.ncand = reinterpret_cast<uint32_t*>(w + L.ncand);
    p.st_m = reinterpret_cast<float*>(w + L.st_m);
    p.st_linv = reinterpret_cast<float*>(w + L.st_linv);
    p.error = reinterpret_cast<int32_t*>(w);
    return p;
}

// Common checks of mra_attention_fwd and mra_debug_stages.
mra_status check_call(const mra_dims* dims, const void* q, const void* k, const void* v, const uint8_t* mask,
                      int32_t bpr, int32_t mode, int32_t pf, int32_t pd, const void* out, const void* ws,
                      size_t ws_bytes, bool need_out, Layout* L) {
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    st = check_params(bpr, mode, pf, pd);
    if (st != MRA_OK) return st;
    if (!q || !k || !v || (need_out && !out)) return MRA_ERR_NULL;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(mask) || (out && misaligned(out)))
        return MRA_ERR_ALIGN;
    if (!carve(*dims, bpr, mode, L)) return MRA_ERR_SEQ_LEN;
    if (!ws || ws_bytes < L->total) return MRA_ERR_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return MRA_ERR_ALIGN;
    const size_t esz = dims->dtype == MRA_BF16 ? 2 : 4;
    const size_t tb = (size_t)dims->batch * dims->heads * dims->seq_len * dims->head_dim * esz;
    const size_t mb = (size_t)dims->batch * dims->seq_len;
    if (out && (overlaps(out, tb, q, tb) || overlaps(out, tb, k, tb) || overlaps(out, tb, v, tb) ||
                overlaps(out, tb, mask, mb) || overlaps(out, tb, ws, ws_bytes)))
        return MRA_ERR_ALIAS;
    // the kernels write the workspace while the inputs are still being read
    if (overlaps(ws, ws_bytes, q, tb) || overlaps(ws, ws_bytes, k, tb) || overlaps(ws, ws_bytes, v, tb) ||
        overlaps(ws, ws_bytes, mask, mb))
        return MRA_ERR_ALIAS;
    return MRA_OK;
}

__global__ void csr_to_flat_kernel(const int32_t* row_ptr, const int32_t* col, int nb, int64_t K, int BH,
                                   int32_t* sel) {
    const int x = blockIdx.x * blockDim.x + threadIdx.x;
    if (x >= BH * nb) return;
    const int bh = x / nb, i = x - bh * nb;
    const int32_t* rp = row_ptr + (size_t)bh * (nb + 1);
    for (int e = rp[i]; e < rp[i + 1]; e++) {
        if (e >= 0 && e < K) sel[(size_t)bh * K + e] = i * nb + col[(size_t)bh * K + e];
    }
}

}  // namespace
}  // namespace mra

using namespace mra;

MRA_API int32_t mra_abi_version(void) { return kAbiVersion; }

MRA_API const char* mra_status_string(int32_t s) {
    switch (s) {
        case MRA_OK: return "ok";
        case MRA_ERR_NULL: return "a required pointer is NULL";
        case MRA_ERR_SHAPE: return "batch/heads out of range";
        case MRA_ERR_SEQ_LEN: return "seq_len must be a multiple of 32 in [32, 16384]";
        case MRA_ERR_HEAD_DIM: return "head_dim must be 64 or 128 and scale_dim 0 or 1 .. head_dim";
        case MRA_ERR_DTYPE: return "dtype must be MRA_F32 or MRA_BF16";
        case MRA_ERR_MODE: return "approx_mode must be full (0) or sparse (1)";
        case MRA_ERR_BUDGET: return "block_per_row must be >= 1";
        case MRA_ERR_PRIOR: return "prior counts must be >= 0";
        case MRA_ERR_ALIAS: return "out overlaps an input or the workspace";
        case MRA_ERR_WORKSPACE: return "workspace missing or too small";
        case MRA_ERR_HIP: return "a HIP launch failed";
        case MRA_ERR_ALIGN: return "a pointer is not aligned (tensors 16 bytes, workspace 256 bytes)";
        case MRA_ERR_STAGE: return "stage cannot be replayed (3 only) or count < 1";
        case MRA_ERR_SCRATCH: return "the sizes need more workspace than the allocation-free entry point holds";
        default: return "unknown status";
    }
}

MRA_API int64_t mra_num_block(int32_t seq_len, int32_t block_per_row) {
    if (seq_len < kBlock || seq_len % kBlock != 0 || block_per_row < 1) return -1;
    const int64_t nb = seq_len / kBlock;
    const int64_t k = nb * (int64_t)block_per_row, cap = nb * nb;
    return k < cap ? k : cap;
}

MRA_API mra_status mra_workspace_size(const mra_dims* dims, int32_t block_per_row, int32_t approx_mode,
                                      size_t* bytes) {
    if (!bytes) return MRA_ERR_NULL;
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    st = check_params(block_per_row, approx_mode, 0, 0);
    if (st != MRA_OK) return st;
    Layout L;
    if (!carve(*dims, block_per_row, approx_mode, &L)) return MRA_ERR_SEQ_LEN;
    *bytes = L.total;
    return MRA_OK;
}

static mra_status run_front(const Params& p, hipStream_t s) {
    if (launch_pool(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_logits(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_premark(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_select(p, s) != hipSuccess) return MRA_ERR_HIP;
    return MRA_OK;
}

static bool bad_ranking(int32_t r) { return r != MRA_RANK_ROW_NORMALIZED && r != MRA_RANK_RAW_LOGITS; }
static bool bad_band(int32_t b) { return b != MRA_BAND_SYMMETRIC && b != MRA_BAND_EXACT; }

// The launch sequence; ev (8 events or null) brackets each of the four stages.
static mra_status run_forward(const mra_dims* dims, const void* q, const void* k, const void* v,
                              const uint8_t* mask, int32_t block_per_row, int32_t approx_mode, int32_t prior_first,
                              int32_t prior_diag, void* out, void* workspace, size_t workspace_bytes, void* stream,
                              void* const* ev, int32_t ranking = MRA_RANK_ROW_NORMALIZED,
                              int32_t band = MRA_BAND_SYMMETRIC, int32_t save_stats = 0) {
    Layout L;
    mra_status st = check_call(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out,
                               workspace, workspace_bytes, true, &L);
    if (st != MRA_OK) return st;
    if (bad_ranking(ranking)) return MRA_ERR_MODE;
    if (bad_band(band)) return MRA_ERR_PRIOR;
    const Params p = make_params(*dims, L, approx_mode, prior_first, prior_diag, q, k, v, mask, out, workspace,
                                 ranking, band, save_stats);
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int idx) {
        return (ev && ev[idx]) ? hipEventRecord(static_cast<hipEvent_t>(ev[idx]), s) : hipSuccess;
    };
    hipError_t e = mark(0);
    if (e == hipSuccess) e = launch_pool(p, s);
    if (e == hipSuccess) e = mark(1);
    if (e == hipSuccess) e = mark(2);
    if (e == hipSuccess) e = launch_logits(p, s);
    if (e == hipSuccess) e = mark(3);
    if (e == hipSuccess) e = mark(4);
    if (e == hipSuccess) e = launch_premark(p, s);
    if (e == hipSuccess) e = launch_select(p, s);
    if (e == hipSuccess) e = mark(5);
    if (e == hipSuccess) e = mark(6);
    if (e == hipSuccess) e = launch_attn(p, s);
    if (e == hipSuccess) e = mark(7);
    return e == hipSuccess ? MRA_OK : MRA_ERR_HIP;
}

MRA_API mra_status mra_attention_fwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                                     const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                     int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return run_forward(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out, workspace,
                       workspace_bytes, stream, nullptr);
}

MRA_API mra_status mra_attention_fwd_ex(const mra_dims* dims, const void* q, const void* k, const void* v,
                                        const uint8_t* mask, const mra_options* opts, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    if (!opts) return MRA_ERR_NULL;
    return run_forward(dims, q, k, v, mask, opts->block_per_row, opts->approx_mode, opts->prior_first,
                       opts->prior_diag, out, workspace, workspace_bytes, stream, nullptr, opts->score_ranking,
                       opts->diag_band, opts->save_stats);
}

MRA_API mra_status mra_attention_fwd_profiled(const mra_dims* dims, const void* q, const void* k, const void* v,
                                              const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                              int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                                              size_t workspace_bytes, void* stream, void* const* events) {
    return run_forward(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out, workspace,
                       workspace_bytes, stream, events);
}

MRA_API mra_status mra_backward_workspace_size(const mra_dims* dims, int32_t block_per_row, int32_t approx_mode,
                                               size_t* bytes) {
    if (!bytes) return MRA_ERR_NULL;
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    st = check_params(block_per_row, approx_mode, 0, 0);
    if (st != MRA_OK) return st;
    Layout L;
    if (!carve(*dims, block_per_row, approx_mode, &L)) return MRA_ERR_SEQ_LEN;
    BwdLayout W;
    carve_bwd(L, approx_mode, &W);
    *bytes = W.total;
    return MRA_OK;
}

// The backward pass on a forward call's workspace; dyn: the forward was a
// static layout (mra_bigbird_fwd) whose stream length is its row_ptr[nb].
static mra_status run_bwd(const mra_dims* dims, const void* q, const void* k, const void* v, const uint8_t* mask,
                          int32_t block_per_row, int32_t approx_mode, int32_t prior_first, int32_t prior_diag,
                          bool dyn, const void* out, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes, void* stream) {
    Layout L;
    mra_status st = check_call(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out,
                               workspace, workspace_bytes, true, &L);
    if (st != MRA_OK) return st;
    if (!dout || !dq || !dk || !dv) return MRA_ERR_NULL;
    if (misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv)) return MRA_ERR_ALIGN;
    BwdLayout W;
    carve_bwd(L, approx_mode, &W);
    if (!bwd_workspace || bwd_workspace_bytes < W.total) return MRA_ERR_WORKSPACE;
    if (misaligned(bwd_workspace)) return MRA_ERR_ALIGN;
    const size_t tb = (size_t)dims->batch * dims->heads * dims->seq_len * dims->head_dim *
                      (dims->dtype == MRA_BF16 ? 2 : 4);
    const void* ins[] = {q, k, v, out, dout, workspace, mask};
    const size_t insz[] = {tb, tb, tb, tb, tb, workspace_bytes, (size_t)dims->batch * dims->seq_len};
    void* outs[] = {dq, dk, dv, bwd_workspace};
    const size_t outsz[] = {tb, tb, tb, bwd_workspace_bytes};
    for (int a = 0; a < 4; a++) {
        for (int c = 0; c < 7; c++)
            if (overlaps(outs[a], outsz[a], ins[c], insz[c])) return MRA_ERR_ALIAS;
        for (int c = a + 1; c < 4; c++)
            if (overlaps(outs[a], outsz[a], outs[c], outsz[c])) return MRA_ERR_ALIAS;
    }
    Params p = make_params(*dims, L, approx_mode, prior_first, prior_diag, q, k, v, mask, const_cast<void*>(out),
                           workspace);
    p.fout = out;
    p.dout = dout;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    char* bw = static_cast<char*>(bwd_workspace);
    p.st_d = reinterpret_cast<float*>(bw + W.st_d);
    p.ct_ptr = reinterpret_cast<int32_t*>(bw + W.ct_ptr);
    p.ct_row = reinterpret_cast<int32_t*>(bw + W.ct_row);
    p.bwd_maxch = W.maxch;
    p.bwd_rch = reinterpret_cast<int4*>(bw + W.rch);
    p.bwd_cch = reinterpret_cast<int4*>(bw + W.cch);
    p.bwd_rmul = reinterpret_cast<int4*>(bw + W.rmul);
    p.bwd_cmul = reinterpret_cast<int4*>(bw + W.cmul);
    p.bwd_count = reinterpret_cast<int4*>(bw + W.count);
    p.bwd_part_dq = reinterpret_cast<float*>(bw + W.part_dq);
    p.bwd_part_dk = reinterpret_cast<float*>(bw + W.part_dk);
    p.bwd_part_dv = reinterpret_cast<float*>(bw + W.part_dv);
    p.attn_dyn = dyn ? 1 : 0;
    auto fl = [&](size_t off) { return off ? reinterpret_cast<float*>(bw + off) : nullptr; };
    p.bwd_g = fl(W.g);
    p.bwd_c = fl(W.c);
    p.bwd_et = fl(W.et);
    p.bwd_wt = fl(W.wt);
    p.bwd_dqh = fl(W.dqh);
    p.bwd_dkh = fl(W.dkh);
    p.bwd_dvh = fl(W.dvh);
    return launch_bwd(p, static_cast<hipStream_t>(stream)) == hipSuccess ? MRA_OK : MRA_ERR_HIP;
}

MRA_API mra_status mra_attention_bwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                                     const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                     int32_t prior_first, int32_t prior_diag, const void* out, const void* dout,
                                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                     void* bwd_workspace, size_t bwd_workspace_bytes, void* stream) {
    return run_bwd(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, false, out, dout, dq,
                   dk, dv, workspace, workspace_bytes, bwd_workspace, bwd_workspace_bytes, stream);
}

// ---------------------------------------------------------------- BigBird
// Largest number of 32-token cells a BigBird pattern can select per head:
// global rows attend every pattern block, the others at most 3 + 2 + r.
static bool bigbird_budget(const mra_dims* d, int32_t block_size, int32_t r, int32_t* bpr) {
    if (block_size < kBlock || block_size % kBlock != 0 || block_size > 4 * kBlock) return false;
    if (d->seq_len % block_size != 0 || d->seq_len < block_size) return false;
    const int64_t f = block_size / kBlock, nbb = d->seq_len / block_size, nb = d->seq_len / kBlock;
    int64_t cells = 0;
    for (int64_t I = 0; I < nbb; I++) {
        const int64_t row = (I == 0 || I == nbb - 1) ? nbb : std::min<int64_t>(nbb, 5 + (int64_t)r);
        cells += f * f * row;
    }
    cells = std::min<int64_t>(cells, nb * nb);
    *bpr = (int32_t)((cells + nb - 1) / nb);   // mra_num_block(N, bpr) >= cells
    return true;
}

static mra_status check_bigbird(const mra_dims* dims, int32_t block_size, int32_t r, int32_t* bpr) {
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    if (r < 1) return MRA_ERR_BUDGET;
    if (!bigbird_budget(dims, block_size, r, bpr)) return MRA_ERR_SEQ_LEN;
    return MRA_OK;
}

MRA_API mra_status mra_bigbird_workspace_size(const mra_dims* dims, int32_t block_size, int32_t num_random_blocks,
                                              size_t* bytes) {
    if (!bytes || !dims) return MRA_ERR_NULL;
    int32_t bpr = 0;
    const mra_status st = check_bigbird(dims, block_size, num_random_blocks, &bpr);
    if (st != MRA_OK) return st;
    Layout L;
    if (!carve(*dims, bpr, MRA_APPROX_SPARSE, &L)) return MRA_ERR_SEQ_LEN;
    *bytes = L.total;
    return MRA_OK;
}

MRA_API mra_status mra_bigbird_fwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                                   const uint8_t* mask, int32_t block_size, int32_t num_random_blocks,
                                   const int32_t* rand_blocks, void* out, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (!dims) return MRA_ERR_NULL;
    int32_t bpr = 0;
    mra_status st = check_bigbird(dims, block_size, num_random_blocks, &bpr);
    if (st != MRA_OK) return st;
    Layout L;
    st = check_call(dims, q, k, v, mask, bpr, MRA_APPROX_SPARSE, 0, 0, out, workspace, workspace_bytes, true, &L);
    if (st != MRA_OK) return st;
    if (!rand_blocks) return MRA_ERR_NULL;
    if (((uintptr_t)rand_blocks & 3u) != 0) return MRA_ERR_ALIGN;
    const size_t rbytes = (size_t)L.BH * (dims->seq_len / block_size) * num_random_blocks * 4;
    if (overlaps(out, (size_t)L.BH * L.N * L.d * (dims->dtype == MRA_BF16 ? 2 : 4), rand_blocks, rbytes) ||
        overlaps(workspace, workspace_bytes, rand_blocks, rbytes))
        return MRA_ERR_ALIAS;
    // the backward pass of a BigBird call reads its statistics: always kept
    Params p = make_params(*dims, L, MRA_APPROX_SPARSE, 0, 0, q, k, v, mask, out, workspace, MRA_RANK_ROW_NORMALIZED,
                           MRA_BAND_SYMMETRIC, 1);
    p.attn_dyn = 1;
    p.bb_f = block_size / kBlock;
    p.bb_r = num_random_blocks;
    p.bb_rand = rand_blocks;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_bigbird_layout(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_attn(p, s) != hipSuccess) return MRA_ERR_HIP;
    return MRA_OK;
}

MRA_API mra_status mra_bigbird_backward_workspace_size(const mra_dims* dims, int32_t block_size,
                                                       int32_t num_random_blocks, size_t* bytes) {
    if (!bytes || !dims) return MRA_ERR_NULL;
    int32_t bpr = 0;
    const mra_status st = check_bigbird(dims, block_size, num_random_blocks, &bpr);
    if (st != MRA_OK) return st;
    Layout L;
    if (!carve(*dims, bpr, MRA_APPROX_SPARSE, &L)) return MRA_ERR_SEQ_LEN;
    BwdLayout W;
    carve_bwd(L, MRA_APPROX_SPARSE, &W);
    *bytes = W.total;
    return MRA_OK;
}

MRA_API mra_status mra_bigbird_bwd(const mra_dims* dims, const void* q, const void* k, const void* v,
                                   const uint8_t* mask, int32_t block_size, int32_t num_random_blocks,
                                   const void* out, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                   size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                                   void* stream) {
    if (!dims) return MRA_ERR_NULL;
    int32_t bpr = 0;
    const mra_status st = check_bigbird(dims, block_size, num_random_blocks, &bpr);
    if (st != MRA_OK) return st;
    return run_bwd(dims, q, k, v, mask, bpr, MRA_APPROX_SPARSE, 0, 0, true, out, dout, dq, dk, dv, workspace,
                   workspace_bytes, bwd_workspace, bwd_workspace_bytes, stream);
}

// ------------------------------------------------------ allocation-free forward
// A fixed device array serves as the workspace of mra_attention_fwd_noalloc.
// Host code never uses the array's name as an address: each device's copy is
// looked up once with hipGetSymbolAddress (with that device current) and
// only that pointer is passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static void* g_scratch_ptr[kMaxDevices];
static hipError_t g_scratch_err[kMaxDevices];
static std::once_flag g_scratch_once[kMaxDevices];

// This device's copy of the scratch array (null when the lookup failed).
static void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    return g_scratch_ptr[dev];
}

MRA_API mra_status mra_attention_fwd_noalloc(const mra_dims* dims, const void* q, const void* k, const void* v,
                                             const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                             int32_t prior_first, int32_t prior_diag, void* out, void* stream) {
    // sizes first, so that an oversized call is refused before anything else
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    st = check_params(block_per_row, approx_mode, prior_first, prior_diag);
    if (st != MRA_OK) return st;
    Layout L;
    if (!carve(*dims, block_per_row, approx_mode, &L)) return MRA_ERR_SEQ_LEN;
    if (L.total > kScratchBytes) return MRA_ERR_SCRATCH;
    void* ws = scratch_for_current_device();
    if (!ws) return MRA_ERR_HIP;
    return run_forward(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out, ws,
                       kScratchBytes, stream, nullptr);
}

MRA_API mra_status mra_workspace_error(const void* workspace, size_t workspace_bytes, void* stream,
                                       uint32_t* error) {
    if (!workspace || !error) return MRA_ERR_NULL;
    if (workspace_bytes < 256) return MRA_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return MRA_ERR_HIP;
    uint32_t word = 0;
    if (hipMemcpy(&word, workspace, 4, hipMemcpyDeviceToHost) != hipSuccess) return MRA_ERR_HIP;
    *error = word;
    return MRA_OK;
}

MRA_API mra_status mra_debug_replay(const mra_dims* dims, const void* q, const void* k, const void* v,
                                    const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                    int32_t prior_first, int32_t prior_diag, void* out, void* workspace,
                                    size_t workspace_bytes, int32_t stage, int32_t count, void* stream) {
    Layout L;
    mra_status st = check_call(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag, out,
                               workspace, workspace_bytes, true, &L);
    if (st != MRA_OK) return st;
    if (stage != 3 || count < 1) return MRA_ERR_STAGE;
    const Params p = make_params(*dims, L, approx_mode, prior_first, prior_diag, q, k, v, mask, out, workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t c = 0; c < count; c++)
        if (launch_attn(p, s) != hipSuccess) return MRA_ERR_HIP;
    return MRA_OK;
}

MRA_API mra_status mra_debug_stages(const mra_dims* dims, const void* q, const void* k, const void* v,
                                    const uint8_t* mask, int32_t block_per_row, int32_t approx_mode,
                                    int32_t prior_first, int32_t prior_diag, int32_t score_ranking,
                                    int32_t diag_band, float* qhat, float* khat, float* vhat, int32_t* count,
                                    float* logits, float* rowmax, int32_t* sel, int32_t* error, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    Layout L;
    mra_status st = check_call(dims, q, k, v, mask, block_per_row, approx_mode, prior_first, prior_diag,
                               nullptr, workspace, workspace_bytes, false, &L);
    if (st != MRA_OK) return st;
    if (bad_ranking(score_ranking)) return MRA_ERR_MODE;
    if (bad_band(diag_band)) return MRA_ERR_PRIOR;
    const Params p = make_params(*dims, L, approx_mode, prior_first, prior_diag, q, k, v, mask, nullptr,
                                 workspace, score_ranking, diag_band);
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = run_front(p, s);
    if (st != MRA_OK) return st;
    const size_t BH = (size_t)L.BH, nb = (size_t)L.nb, dd = (size_t)L.d;
    hipError_t e = hipSuccess;
    auto cp = [&](void* dst, const void* src, size_t bytes) {
        if (dst && e == hipSuccess) e = hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
    };
    cp(qhat, p.qhat, BH * nb * dd * 4);
    cp(khat, p.khat, BH * nb * dd * 4);
    if (p.vhat) cp(vhat, p.vhat, BH * nb * dd * 4);
    cp(count, p.cnt, (size_t)L.B * nb * 4);
    cp(logits, p.logits, BH * nb * nb * 4);
    cp(rowmax, p.rowmax, BH * nb * 4);
    cp(error, p.error, 4);
    if (e != hipSuccess) return MRA_ERR_HIP;
    if (sel) {
        const int total = L.BH * L.nb;
        hipLaunchKernelGGL(csr_to_flat_kernel, dim3((total + 255) / 256), dim3(256), 0, s, p.row_ptr, p.col, L.nb,
                           L.K, L.BH, sel);
        if (hipGetLastError() != hipSuccess) return MRA_ERR_HIP;
    }
    return MRA_OK;
}

MRA_API mra_status mra_debug_wait_timeout(const mra_dims* dims, const void* q, const void* k, const void* v,
                                          int32_t block_per_row, int32_t approx_mode, uint32_t polls,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    Layout L;
    mra_status st = check_call(dims, q, k, v, nullptr, block_per_row, approx_mode, 0, 0, nullptr, workspace,
                               workspace_bytes, false, &L);
    if (st != MRA_OK) return st;
    if (polls < 1 || polls > (1u << 16)) return MRA_ERR_STAGE;
    if (!fused_select(L.BH, L.nb, L.d, approx_mode)) return MRA_ERR_SEQ_LEN;
    Params p = make_params(*dims, L, approx_mode, 0, 0, q, k, v, nullptr, nullptr, workspace);
    p.wait_polls = polls;
    p.wait_extra = 1;
    return run_front(p, static_cast<hipStream_t>(stream));
}

MRA_API mra_status mra_debug_select(const mra_dims* dims, const float* logits, const int32_t* count,
                                    int32_t block_per_row, int32_t prior_first, int32_t prior_diag,
                                    int32_t score_ranking, int32_t diag_band, int32_t* sel, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    mra_status st = check_dims(dims);
    if (st != MRA_OK) return st;
    st = check_params(block_per_row, MRA_APPROX_SPARSE, prior_first, prior_diag);
    if (st != MRA_OK) return st;
    if (bad_ranking(score_ranking)) return MRA_ERR_MODE;
    if (bad_band(diag_band)) return MRA_ERR_PRIOR;
    if (!logits || !count || !sel) return MRA_ERR_NULL;
    Layout L;
    if (!carve(*dims, block_per_row, MRA_APPROX_SPARSE, &L)) return MRA_ERR_SEQ_LEN;
    if (!workspace || workspace_bytes < L.total) return MRA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return MRA_ERR_ALIGN;
    Params p = make_params(*dims, L, MRA_APPROX_SPARSE, prior_first, prior_diag, nullptr, nullptr, nullptr,
                           nullptr, nullptr, workspace, score_ranking, diag_band);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t BH = (size_t)L.BH, nb = (size_t)L.nb;
    hipError_t e = hipMemcpyAsync(p.logits, logits, BH * nb * nb * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(p.cnt, count, (size_t)L.B * nb * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemsetAsync(p.hist, 0, BH * kHistBins * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(p.ncand, 0, BH * kCandStride * 4, s);
    if (e == hipSuccess) e = hipMemsetAsync(p.error, 0, 4, s);
    if (e != hipSuccess) return MRA_ERR_HIP;
    p.logits_given = 1;
    if (launch_logits_given(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_premark(p, s) != hipSuccess) return MRA_ERR_HIP;
    if (launch_select(p, s) != hipSuccess) return MRA_ERR_HIP;
    const int total = L.BH * L.nb;
    hipLaunchKernelGGL(csr_to_flat_kernel, dim3((total + 255) / 256), dim3(256), 0, s, p.row_ptr, p.col, L.nb, L.K,
                       L.BH, sel);
    if (hipGetLastError() != hipSuccess) return MRA_ERR_HIP;
    return MRA_OK;
}
