"""Pins for the CPU oracle: each test ties it to something other than itself.

These tests use the pages' worked example, closed forms, invariants,
special cases that reduce to a library routine (torch's fp64 CPU
scaled-dot-product attention, numpy's lexsort), and brute force on tiny
inputs.  Each pin is chosen so that a plausible mistake in the oracle fails
it: a dropped term, a wrong sign or index, or a transposed operand.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sdpa64(q, k, v, allowed=None):
    """torch fp64 CPU softmax(q k^T / sqrt(d)) v; allowed: bool [.., N, N] or None."""
    tq, tk, tv = (torch.from_numpy(np.asarray(x, np.float64)) for x in (q, k, v))
    m = None if allowed is None else torch.from_numpy(allowed)
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m).numpy()


def rand_qkv(B, H, N, d=64, seed=0, scale=1.0):
    rng = np.random.default_rng(seed)
    return [(rng.standard_normal((B, H, N, d)) * scale).astype(np.float32) for _ in range(3)]


# ---------------------------------------------------------------- budget ----
def test_budget_matches_worked_examples():
    ex = json.load(open(os.path.join(GOLDEN, "budget_examples.json")))["examples"]
    for e in ex:
        assert e["seq_len"] // 32 == e["num_blocks_per_row"]
        assert (e["seq_len"] // 32) ** 2 == e["full_grid"]
        assert oracle.num_block(e["seq_len"], e["block_per_row"]) == e["num_block"]


@pytest.mark.parametrize("N,bpr,expect", [
    (16384, 8, 4096), (4096, 4, 512), (512, 16, 256), (512, 17, 256), (32, 1, 1), (32, 5, 1),
    (48, 4, -1), (0, 4, -1), (512, 0, -1), (-32, 4, -1)])
def test_budget_closed_form(N, bpr, expect):
    assert oracle.num_block(N, bpr) == expect


# ---------------------------------------------------------------- pooling ---
def test_pool_hand_example():
    N, d = 64, 4
    x = np.tile(np.arange(N, dtype=np.float32)[:, None], (1, d))
    x[:, 1] *= -1
    mask = np.zeros(N, np.uint8)
    mask[[0, 5, 31]] = 1          # block 0: tokens 0, 5, 31
    mask[32:64] = 1               # block 1: all valid
    xh, cnt = oracle.pool_f32(x, mask)
    assert cnt.tolist() == [3, 32]
    assert xh[0].tolist() == [12.0, -12.0, 12.0, 12.0]
    assert xh[1, 0] == np.float32(np.mean(np.arange(32, 64)))
    # an empty block pools to zeros
    mask[:32] = 0
    xh, cnt = oracle.pool_f32(x, mask)
    assert cnt.tolist() == [0, 32] and np.all(xh[0] == 0)


def test_pool_matches_fp64_mean():
    rng = np.random.default_rng(7)
    N, d = 256, 64
    x = rng.standard_normal((N, d)).astype(np.float32)
    mask = (rng.random(N) < 0.6).astype(np.uint8)
    mask[64:96] = 0
    xh, cnt = oracle.pool_f32(x, mask)
    xh64 = oracle.pool_f64(x, mask)
    for i in range(N // 32):
        sel = mask[32 * i: 32 * i + 32].astype(bool)
        assert cnt[i] == sel.sum()
        ref = x[32 * i: 32 * i + 32][sel].astype(np.float64).mean(0) if sel.any() else np.zeros(d)
        np.testing.assert_allclose(xh64[i], ref, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(xh[i], ref, rtol=0, atol=4e-7 * max(1, np.abs(x).max()))


# ---------------------------------------------------------------- logits ----
def test_logits_match_scaled_matmul():
    rng = np.random.default_rng(3)
    nb, d = 24, 64
    qh = rng.standard_normal((nb, d)).astype(np.float32)
    kh = rng.standard_normal((nb, d)).astype(np.float32)
    S = oracle.lowres_logits_f32(qh, kh)
    ref = qh.astype(np.float64) @ kh.astype(np.float64).T / math.sqrt(d)
    np.testing.assert_allclose(S, ref, rtol=0, atol=2e-5)
    # not transposed: row i belongs to query block i
    qh2 = qh.copy()
    qh2[0] = 0
    assert np.all(oracle.lowres_logits_f32(qh2, kh)[0] == 0)
    assert np.any(oracle.lowres_logits_f32(qh2, kh)[:, 0] != 0)


def test_logits_exact_on_small_integers():
    # small integers: every product and partial sum is exact in fp32
    rng = np.random.default_rng(4)
    nb, d = 8, 64
    qh = rng.integers(-8, 9, (nb, d)).astype(np.float32)
    kh = rng.integers(-8, 9, (nb, d)).astype(np.float32)
    S = oracle.lowres_logits_f32(qh, kh)
    exact = (qh.astype(np.int64) @ kh.astype(np.int64).T).astype(np.float64) / 8.0
    assert np.array_equal(S.astype(np.float64), exact)


# ---------------------------------------------------------------- scores ----
def test_scores_rowmax_priors_and_empty_blocks():
    nb = 8
    rng = np.random.default_rng(5)
    S = rng.standard_normal((nb, nb)).astype(np.float32)
    cnt = np.full(nb, 32, np.int32)
    cnt[6] = 0
    rowmax, sc = oracle.scores_f32(S, cnt, prior_first=2, prior_diag=3)
    for i in range(nb):
        valid = cnt > 0
        assert rowmax[i] == S[i, valid].max()
        for j in range(nb):
            if cnt[i] == 0 or cnt[j] == 0:
                assert sc[i, j] == -np.inf
                continue
            nprior = int(abs(i - j) <= 1) + int(i < 2) + int(j < 2)
            s = np.float32(S[i, j] - rowmax[i])
            for _ in range(nprior):
                s = np.float32(s + np.float32(5000.0))
            assert sc[i, j] == s, (i, j)
    # each non-empty row's best block scores exactly 0 before priors
    _, sc0 = oracle.scores_f32(S, cnt)
    for i in range(nb):
        if cnt[i]:
            assert sc0[i].max() == 0.0 and not np.signbit(sc0[i].max())


@pytest.mark.parametrize("g,half", [(1, 0), (2, 1), (3, 1), (5, 2)])
def test_diagonal_band_width(g, half):
    nb = 9
    S = np.zeros((nb, nb), np.float32)
    cnt = np.full(nb, 32, np.int32)
    _, sc = oracle.scores_f32(S, cnt, prior_diag=g)
    band = np.abs(np.subtract.outer(np.arange(nb), np.arange(nb))) <= half
    assert np.array_equal(sc == 5000.0, band) and np.all(sc[~band] == 0.0)


@pytest.mark.parametrize("g,lo,hi", [(1, 0, 0), (2, 0, 1), (3, -1, 1), (4, -1, 2), (5, -2, 2), (6, -2, 3)])
def test_diagonal_band_exact_width(g, lo, hi):
    # reading R7': the band is exactly g blocks wide, offsets j - i in
    # [-floor((g-1)/2), floor(g/2)]; an interior block row holds g band cells
    nb = 11
    S = np.zeros((nb, nb), np.float32)
    cnt = np.full(nb, 32, np.int32)
    _, sc = oracle.scores_f32(S, cnt, prior_diag=g, band="exact")
    off = np.subtract.outer(np.arange(nb), np.arange(nb)) * -1   # off[i, j] = j - i
    band = (off >= lo) & (off <= hi)
    assert np.array_equal(sc == 5000.0, band) and np.all(sc[~band] == 0.0)
    assert all(int((sc[i] == 5000.0).sum()) == g for i in range(3, nb - 3))
    if g % 2 == 1:   # odd widths: both readings give the same band
        _, sym = oracle.scores_f32(S, cnt, prior_diag=g)
        assert np.array_equal(sym, sc)


@pytest.mark.parametrize("band,g,bpr", [("exact", 2, 2), ("exact", 4, 4), ("symmetric", 2, 3),
                                        ("symmetric", 4, 5)])
def test_band_prior_sets_closed_form(band, g, bpr):
    # equal logits: the budget takes every band cell (+5000) and fills the
    # rest with the smallest flat indices outside the band
    nb = 16
    cells = [(i, j) for i in range(nb) for j in range(nb)
             if (-((g - 1) // 2) <= j - i <= g // 2 if band == "exact" else abs(i - j) <= g // 2)]
    K = nb * bpr
    assert len(cells) <= K
    inside = sorted(i * nb + j for i, j in cells)
    outside = [f for f in range(nb * nb) if f not in set(inside)][: K - len(cells)]
    sel = oracle.select_from_logits(np.zeros((nb, nb), np.float32), np.full(nb, 32, np.int32), K,
                                    prior_diag=g, band=band)
    assert sel.tolist() == sorted(inside + outside)


# ---------------------------------------------------------------- selection -
def test_selection_matches_lexsort_with_ties():
    rng = np.random.default_rng(11)
    for nb, K in [(16, 64), (32, 100), (8, 64), (8, 1)]:
        score = rng.integers(-5, 3, (nb, nb)).astype(np.float32)   # many ties
        score[0, 3] = -np.inf
        flat = np.arange(nb * nb)
        order = np.lexsort((flat, -score.reshape(-1)))
        ref = np.sort(order[:K])
        assert np.array_equal(oracle.select_top(score, K), ref)


def test_selection_all_equal_takes_first_flat_indices():
    nb = 16
    sel = oracle.select_top(np.zeros((nb, nb), np.float32), 37)
    assert sel.tolist() == list(range(37))


def test_selection_one_per_row_is_row_argmax():
    # bpr = 1, no priors: each row's maximum scores exactly 0 and every other
    # cell is negative, so the nb selected cells are the row argmaxes.
    rng = np.random.default_rng(12)
    nb = 16
    S = rng.standard_normal((nb, nb)).astype(np.float32)
    sel = oracle.select_from_logits(S, np.full(nb, 32, np.int32), nb)
    assert np.array_equal(sel, np.arange(nb) * nb + S.argmax(1))


# ------------------------------------------- raw-logit ranking (reading R2') --
def test_raw_ranking_scores_are_the_logits_plus_priors():
    # R2' ranks S_ij itself: no row max is subtracted; priors, empty blocks
    # and the -0 fold behave as under R2
    rng = np.random.default_rng(13)
    nb = 12
    S = rng.standard_normal((nb, nb)).astype(np.float32)
    S[2, 5] = -0.0
    cnt = np.full(nb, 32, np.int32)
    cnt[7] = 0
    _, sc = oracle.scores_f32(S, cnt, prior_first=2, prior_diag=3, ranking="raw_logits")
    want = S.copy()
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    for m in ((np.abs(i - j) <= 1), (i < 2), (j < 2)):   # fp32 adds in the order diagonal, row, column
        want = np.where(m, want + np.float32(5000.0), want).astype(np.float32)
    want[7, :] = -np.inf
    want[:, 7] = -np.inf
    want[want == 0] = 0.0
    assert np.array_equal(sc, want) and not np.signbit(sc[2, 5])


def test_raw_ranking_selection_matches_lexsort():
    rng = np.random.default_rng(14)
    for nb, K in [(16, 64), (8, 8), (32, 96)]:
        S = np.round(rng.standard_normal((nb, nb)) * 4).astype(np.float32) / 4   # ties
        cnt = np.full(nb, 32, np.int32)
        flat = np.arange(nb * nb)
        ref = np.sort(np.lexsort((flat, -S.reshape(-1)))[:K])
        assert np.array_equal(oracle.select_from_logits(S, cnt, K, ranking="raw_logits"), ref)


def test_rankings_differ_on_rows_of_different_level():
    # S_ij = 10 i + j / 100: under R2 every row's best cell scores 0, so bpr 1
    # takes the last column; under R2' the K = nb largest logits are the
    # whole last row
    nb = 16
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    S = (10.0 * i + j / 100.0).astype(np.float32)
    cnt = np.full(nb, 32, np.int32)
    r2 = oracle.select_from_logits(S, cnt, nb)
    r2p = oracle.select_from_logits(S, cnt, nb, ranking="raw_logits")
    assert r2.tolist() == [r * nb + nb - 1 for r in range(nb)]
    assert r2p.tolist() == [(nb - 1) * nb + c for c in range(nb)]


def test_raw_ranking_sparse_forward_is_block_masked_dense():
    # block-constant rows of q: the raw low-res logits are ordered by key
    # block, the same in every row; with bpr 2 and no priors R2' takes whole
    # key-block columns (the highest-logit ones), so sparse mode is dense
    # attention masked to those columns
    rng = np.random.default_rng(15)
    N, nb, d = 256, 8, 64
    k = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    qrow = rng.standard_normal(d).astype(np.float32)
    q = np.broadcast_to(qrow, (1, 1, N, d)).copy()
    v = rng.standard_normal((1, 1, N, d)).astype(np.float32)
    out, sel = oracle.mra_forward(q, k, v, None, 2, "sparse", ranking="raw_logits", return_selection=True)
    cells = sel[0, 0]
    cols = sorted(set((cells % nb).tolist()))
    assert len(cells) == 2 * nb and len(cols) == 2
    assert all(((c // nb) * nb + cc) in set(cells.tolist()) for c in cells for cc in cols)
    kh = k[0, 0].reshape(nb, 32, d).mean(1)
    assert cols == sorted(np.argsort(-(kh @ qrow))[:2].tolist())
    blk = np.arange(N) // 32
    allowed = np.isin(blk, cols)[None, :].repeat(N, 0)
    np.testing.assert_allclose(out, sdpa64(q, k, v, allowed), rtol=0, atol=1e-12)


# -------------------------------------------------------- closed-form sets --
@pytest.mark.parametrize("pf,pd,bpr,cells", [
    (0, 1, 1, lambda i, j: i == j),
    (4, 0, 7, lambda i, j: i < 4 or j < 4),
    (8, 0, 12, lambda i, j: i < 8 or j < 8),
])
def test_prior_sets_fill_budget_exactly(pf, pd, bpr, cells):
    q, k, v = rand_qkv(1, 2, 512, seed=21)
    out, sel = oracle.mra_forward(q, k, v, block_per_row=bpr, approx_mode="sparse",
                                  prior_first=pf, prior_diag=pd, return_selection=True)
    nb = 16
    ref = [i * nb + j for i in range(nb) for j in range(nb) if cells(i, j)]
    assert len(ref) == oracle.num_block(512, bpr)
    for h in range(2):
        assert sel[0, h].tolist() == ref


# ----------------------------------------------------- reductions to dense --
@pytest.mark.parametrize("mode", ["full", "sparse"])
@pytest.mark.parametrize("N,bpr", [(512, 16), (64, 4)])
def test_all_blocks_selected_equals_dense(mode, N, bpr):
    q, k, v = rand_qkv(1, 2, N, seed=31)
    assert oracle.num_block(N, bpr) == (N // 32) ** 2
    out = oracle.mra_forward(q, k, v, block_per_row=bpr, approx_mode=mode)
    np.testing.assert_allclose(out, sdpa64(q, k, v), rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.dense_forward(q, k, v), sdpa64(q, k, v), rtol=0, atol=1e-12)


def test_all_pairs_selected_with_mask_equals_masked_dense():
    N = 256
    q, k, v = rand_qkv(2, 2, N, seed=32)
    mask = np.ones((2, N), np.uint8)
    mask[0, 200:] = 0
    mask[1, ::3] = 0
    allowed = np.broadcast_to(mask[:, None, None, :].astype(bool), (2, 2, N, N)).copy()
    ref = sdpa64(q, k, v, allowed)
    ref[mask[:, None, :, None].repeat(2, 1).repeat(64, 3) == 0] = 0
    for mode in ("full", "sparse"):
        out = oracle.mra_forward(q, k, v, mask, block_per_row=8, approx_mode=mode)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(oracle.dense_forward(q, k, v, mask), ref, rtol=0, atol=1e-12)


def test_priors_only_sparse_equals_block_masked_dense():
    N, nb = 512, 16
    q, k, v = rand_qkv(1, 2, N, seed=33)
    out = oracle.mra_forward(q, k, v, block_per_row=7, approx_mode="sparse", prior_first=4)
    blk = np.arange(N) // 32
    allowed = (blk[:, None] < 4) | (blk[None, :] < 4)
    np.testing.assert_allclose(out, sdpa64(q, k, v, allowed), rtol=0, atol=1e-12)


@pytest.mark.parametrize("masked", [False, True])
def test_block_constant_qk_full_equals_dense(masked):
    # Q and K constant over the valid tokens of each block: the exact logits of
    # an unselected block all equal its low-res logit, so full mode must equal
    # dense attention whatever the selection (pins the cnt_j weights and the merge).
    N, nb, d = 256, 8, 64
    rng = np.random.default_rng(34)
    qb = rng.standard_normal((1, 2, nb, d)).astype(np.float32)
    kb = rng.standard_normal((1, 2, nb, d)).astype(np.float32)
    q = np.repeat(qb, 32, axis=2)
    k = np.repeat(kb, 32, axis=2)
    v = rng.standard_normal((1, 2, N, d)).astype(np.float32)
    mask = None
    allowed = None
    if masked:
        mask = (rng.random((1, N)) < 0.7).astype(np.uint8)
        mask[0, 64:96] = 0
        allowed = np.broadcast_to(mask[:, None, None, :].astype(bool), (1, 2, N, N)).copy()
    ref = sdpa64(q, k, v, allowed)
    if masked:
        ref[:, :, mask[0] == 0, :] = 0
    for bpr, pf, pd in [(1, 0, 0), (2, 1, 3), (3, 0, 1)]:
        out = oracle.mra_forward(q, k, v, mask, block_per_row=bpr, approx_mode="full",
                                 prior_first=pf, prior_diag=pd)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)


# ------------------------------------------------------------ brute force ---
def brute_force(q, k, v, mask, sel, mode):
    """Materialise the N x N approximate weight matrix of one head: exact
    exp(s) on selected blocks, exp(low-res logit) on every valid key of an
    unselected block (full mode), nothing elsewhere."""
    N, d = q.shape
    nb = N // 32
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    m = np.ones(N, bool) if mask is None else mask.astype(bool)
    chosen = np.zeros((nb, nb), bool)
    chosen.reshape(-1)[sel] = True
    logit = np.full((N, N), -np.inf)
    exact = q64 @ k64.T / math.sqrt(d)
    blk = np.arange(N) // 32
    cnt = np.array([m[32 * j:32 * j + 32].sum() for j in range(nb)])
    pooled = lambda x: np.stack([x[32 * j:32 * j + 32][m[32 * j:32 * j + 32]].mean(0)
                                 if cnt[j] else np.zeros(d) for j in range(nb)])
    low = pooled(q64) @ pooled(k64).T / math.sqrt(d)
    for t in range(N):
        for u in range(N):
            if not m[u]:
                continue
            if chosen[blk[t], blk[u]]:
                logit[t, u] = exact[t, u]
            elif mode == "full":
                logit[t, u] = low[blk[t], blk[u]]
    out = np.zeros((N, d))
    for t in range(N):
        if not m[t] or np.all(logit[t] == -np.inf):
            continue
        w = np.exp(logit[t] - logit[t].max())
        out[t] = w @ v64 / w.sum()
    return out


@pytest.mark.parametrize("mode,bpr,pf,pd,masked", [
    ("full", 2, 0, 0, False), ("full", 3, 1, 1, True), ("sparse", 2, 0, 3, False),
    ("sparse", 1, 0, 0, True), ("full", 1, 0, 0, False)])
def test_brute_force_materialisation(mode, bpr, pf, pd, masked):
    N = 256
    q, k, v = rand_qkv(1, 2, N, seed=41 + bpr)
    mask = None
    if masked:
        rng = np.random.default_rng(5)
        mask = (rng.random((1, N)) < 0.8).astype(np.uint8)
        mask[0, 32:64] = 0
    out, sel = oracle.mra_forward(q, k, v, mask, block_per_row=bpr, approx_mode=mode,
                                  prior_first=pf, prior_diag=pd, return_selection=True)
    for h in range(2):
        ref = brute_force(q[0, h], k[0, h], v[0, h], None if mask is None else mask[0],
                          sel[0, h], mode)
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=1e-12)


# 128-channel heads: nothing in the oracle is tied to 64 channels
@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_head128_all_blocks_selected_equals_dense(mode):
    q, k, v = rand_qkv(1, 2, 256, d=128, seed=37)
    out = oracle.mra_forward(q, k, v, block_per_row=8, approx_mode=mode)
    np.testing.assert_allclose(out, sdpa64(q, k, v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode,pf,pd,masked", [("full", 0, 1, True), ("sparse", 1, 3, False)])
def test_head128_brute_force_materialisation(mode, pf, pd, masked):
    N = 256
    q, k, v = rand_qkv(1, 2, N, d=128, seed=43)
    mask = None
    if masked:
        mask = (np.random.default_rng(6).random((1, N)) < 0.8).astype(np.uint8)
    out, sel = oracle.mra_forward(q, k, v, mask, block_per_row=2, approx_mode=mode, prior_first=pf, prior_diag=pd,
                                  return_selection=True)
    for h in range(2):
        ref = brute_force(q[0, h], k[0, h], v[0, h], None if mask is None else mask[0], sel[0, h], mode)
        np.testing.assert_allclose(out[0, h], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------- invariants ---
@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_value_shift_and_scale_invariance(mode):
    N = 512
    q, k, v = rand_qkv(1, 2, N, seed=51)
    # V on a 1/64 grid and shifts on a 1/4 grid keep v + c exact in fp32
    v = (np.random.default_rng(9).integers(-256, 256, v.shape) / 64).astype(np.float32)
    kw = dict(block_per_row=3, approx_mode=mode, prior_first=1, prior_diag=1)
    base, sel = oracle.mra_forward(q, k, v, return_selection=True, **kw)
    c = (np.arange(64) / 4 - 8).astype(np.float32)
    shifted = oracle.mra_forward(q, k, v + c, **kw)
    rows = np.any(base != 0, axis=-1)          # rows that attend to something
    np.testing.assert_allclose(shifted[rows], (base + c)[rows], rtol=0, atol=1e-12)
    scaled = oracle.mra_forward(q, k, v * np.float32(4.0), **kw)
    np.testing.assert_allclose(scaled, 4 * base, rtol=1e-14, atol=1e-13)


def test_sparse_rows_in_convex_hull_of_selected_values():
    N, nb = 512, 16
    q, k, v = rand_qkv(1, 1, N, seed=52)
    out, sel = oracle.mra_forward(q, k, v, block_per_row=2, approx_mode="sparse",
                                  return_selection=True)
    chosen = np.zeros((nb, nb), bool)
    chosen.reshape(-1)[sel[0, 0]] = True
    for i in range(nb):
        cols = np.nonzero(chosen[i])[0]
        rows = slice(32 * i, 32 * i + 32)
        if len(cols) == 0:
            assert np.all(out[0, 0, rows] == 0)     # nothing selected: 0/0 -> 0
            continue
        vv = np.concatenate([v[0, 0, 32 * j:32 * j + 32] for j in cols])
        assert np.all(out[0, 0, rows] <= vv.max(0) + 1e-12)
        assert np.all(out[0, 0, rows] >= vv.min(0) - 1e-12)


def test_masked_query_rows_are_zero_and_selection_skips_empty_blocks():
    N, nb = 256, 8
    q, k, v = rand_qkv(1, 1, N, seed=53)
    mask = np.ones((1, N), np.uint8)
    mask[0, 192:] = 0                       # blocks 6, 7 empty
    mask[0, 5] = 0
    out, sel = oracle.mra_forward(q, k, v, mask, block_per_row=4, return_selection=True)
    assert np.all(out[0, 0, 192:] == 0) and np.all(out[0, 0, 5] == 0)
    i, j = sel[0, 0] // nb, sel[0, 0] % nb
    assert np.all(i < 6) and np.all(j < 6)   # 32 = K <= 36 valid pairs


def test_selection_reading_on_named_workload_ties():
    # The long sparse workload with priors (first 2, diagonal 3) has 884 prior
    # cells for a budget of 512; the top of the order is always the priors.
    w = workloads.iid("t", 1, 1, 4096, seed=3, scale=0.5, approx_mode="sparse",
                      prior_first=2, prior_diag=3)
    nb = 128
    qh, cnt = oracle.pool_f32(w.q[0, 0])
    kh, _ = oracle.pool_f32(w.k[0, 0])
    S = oracle.lowres_logits_f32(qh, kh)
    _, sc = oracle.scores_f32(S, cnt, 2, 3)
    sel = oracle.select_top(sc, 512)
    ii, jj = np.divmod(sel, nb)
    prior = (np.abs(ii - jj) <= 1) | (ii < 2) | (jj < 2)
    assert np.all(prior)
    assert (sc > 2500).sum() == 884      # logit spread is far below the 5000 bias


# ------------------------------------------------------------- gradients --
# The oracle's backward (oracle_mra_bwd): gradients of the forward with the
# selection held fixed ([MRA] step 3), through the low-res branch and the block
# means in full mode ([MRA] step 4).
def sdpa64_grads(q, k, v, dout, allowed=None):
    """torch fp64 CPU autograd of softmax(q k^T / sqrt(d)) v against dout."""
    tq, tk, tv = (torch.from_numpy(np.asarray(x, np.float64)).requires_grad_(True) for x in (q, k, v))
    m = None if allowed is None else torch.from_numpy(allowed)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m)
    out.backward(torch.from_numpy(np.asarray(dout, np.float64)))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def rand_dout(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_bwd_all_blocks_selected_equals_dense_autograd(mode):
    N, bpr = 128, 4
    q, k, v = rand_qkv(1, 2, N, seed=41)
    g = rand_dout(q.shape, 42)
    assert oracle.num_block(N, bpr) == (N // 32) ** 2
    got = oracle.mra_backward(q, k, v, g, block_per_row=bpr, approx_mode=mode)
    for a, b in zip(got, sdpa64_grads(q, k, v, g)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_bwd_all_pairs_selected_with_mask_equals_masked_dense_autograd():
    N = 128
    q, k, v = rand_qkv(2, 1, N, seed=43)
    mask = np.ones((2, N), np.uint8)
    mask[0, 100:] = 0
    mask[1, ::5] = 0
    g = rand_dout(q.shape, 44)
    g[mask[:, None, :] == 0] = 0.0            # padded rows output 0: no gradient flows from them
    allowed = np.broadcast_to(mask[:, None, None, :].astype(bool), (2, 1, N, N)).copy()
    ref = sdpa64_grads(q, k, v, g, allowed)
    for mode in ("full", "sparse"):
        got = oracle.mra_backward(q, k, v, g, mask, block_per_row=4, approx_mode=mode)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_bwd_priors_only_sparse_equals_block_masked_dense_autograd():
    N = 512
    q, k, v = rand_qkv(1, 1, N, seed=45)
    g = rand_dout(q.shape, 46)
    got = oracle.mra_backward(q, k, v, g, block_per_row=7, approx_mode="sparse", prior_first=4)
    blk = np.arange(N) // 32
    allowed = (blk[:, None] < 4) | (blk[None, :] < 4)
    assert oracle.num_block(N, 7) == int(allowed[::32, ::32].sum())
    for a, b in zip(got, sdpa64_grads(q, k, v, g, allowed)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_bwd_value_gradients_sum_to_output_gradients(mode):
    # every valid output row is a convex combination of values (and, in full
    # mode, of block means whose weights each spread 1/cnt over cnt tokens),
    # so the value gradients of one head sum to its rows' output gradients
    N = 256
    q, k, v = rand_qkv(2, 2, N, seed=47)
    mask = np.ones((2, N), np.uint8)
    mask[1, 150:] = 0
    g = rand_dout(q.shape, 48)
    _, _, dv = oracle.mra_backward(q, k, v, g, mask, block_per_row=2, approx_mode=mode)
    want = (g.astype(np.float64) * mask[:, None, :, None]).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), want, rtol=0, atol=1e-10)


@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_bwd_matches_central_differences(mode):
    # loss = sum(out * g) with the fp64 forward oracle; central differences on
    # sampled coordinates where the selection stays the same
    B, H, N, d = 1, 1, 128, 8
    rng = np.random.default_rng(49)
    q, k, v = (rng.standard_normal((B, H, N, d)).astype(np.float32) for _ in range(3))
    mask = np.ones((B, N), np.uint8)
    mask[0, 120:] = 0                          # one partial block
    g = rand_dout(q.shape, 50)
    kw = dict(block_per_row=1, approx_mode=mode, prior_diag=1)
    grads = oracle.mra_backward(q, k, v, g, mask, **kw)
    _, sel0 = oracle.mra_forward(q, k, v, mask, return_selection=True, **kw)
    checked = 0
    for which in range(3):
        for _ in range(10):
            t, c = int(rng.integers(0, 120)), int(rng.integers(0, d))
            vals = []
            for sgn in (1, -1):
                x = [q.copy(), k.copy(), v.copy()]
                x[which][0, 0, t, c] = np.float32(x[which][0, 0, t, c] + sgn * np.float32(1e-3))
                out, sel = oracle.mra_forward(*x, mask, return_selection=True, **kw)
                vals.append((float((out * g).sum()), x[which][0, 0, t, c], np.array_equal(sel, sel0)))
            if not (vals[0][2] and vals[1][2]):
                continue
            fd = (vals[0][0] - vals[1][0]) / (float(vals[0][1]) - float(vals[1][1]))
            assert abs(fd - grads[which][0, 0, t, c]) <= 1e-5 * (1 + abs(fd)), (which, t, c, fd)
            checked += 1
    assert checked >= 24


# ------------------------------------------------------- BigBird pattern ----
def bigbird_allowed(N, bs, rand_bh):
    """[N, N] bool from the pattern's three parts, built with numpy broadcasts."""
    nbb = N // bs
    I = np.arange(nbb)[:, None]
    J = np.arange(nbb)[None, :]
    blk = (np.abs(I - J) <= 1) | (I == 0) | (I == nbb - 1) | (J == 0) | (J == nbb - 1)
    for i in range(nbb):
        for x in rand_bh[i]:
            if 0 <= x < nbb:
                blk[i, x] = True
    return np.repeat(np.repeat(blk, bs, 0), bs, 1)


def test_bigbird_equals_block_masked_sdpa():
    B, H, N, bs = 2, 2, 512, 64
    q, k, v = rand_qkv(B, H, N, seed=61)
    rand = workloads.bigbird_rand(B, H, N, bs, 2, seed=62)
    mask = np.ones((B, N), np.uint8)
    mask[1, 400:] = 0
    got = oracle.bigbird_forward(q, k, v, rand, mask, bs)
    for b in range(B):
        for h in range(H):
            allowed = bigbird_allowed(N, bs, rand[b, h]) & mask[b][None, :].astype(bool)
            ref = sdpa64(q[b, h], k[b, h], v[b, h], allowed)
            valid = mask[b].astype(bool)
            np.testing.assert_allclose(got[b, h][valid], ref[valid], rtol=0, atol=1e-12)
            assert np.all(got[b, h][~valid] == 0)


def test_bigbird_short_sequence_is_dense():
    # three blocks or fewer: the window and the two global blocks cover every pair
    q, k, v = rand_qkv(1, 2, 192, seed=63)
    got = oracle.bigbird_forward(q, k, v, np.full((1, 2, 3, 2), -1, np.int32), None, 64)
    np.testing.assert_allclose(got, sdpa64(q, k, v), rtol=0, atol=1e-12)


def test_bigbird_rows_see_only_their_blocks():
    # a block row's output moves when an attended block's values change and
    # stays bit-identical when a block outside its pattern changes
    N, bs, nbb = 1024, 64, 16
    q, k, v = rand_qkv(1, 1, N, seed=64)
    rand = np.full((1, 1, nbb, 3), -1, np.int32)
    rand[0, 0, 7] = [3, 12, 12]                     # a repeated pick names the block once
    base = oracle.bigbird_forward(q, k, v, rand, None, bs)
    rows = slice(7 * bs, 8 * bs)
    for J, moves in [(3, True), (12, True), (6, True), (0, True), (15, True), (10, False), (4, False)]:
        v2 = v.copy()
        v2[0, 0, J * bs:(J + 1) * bs] += 1.0
        out = oracle.bigbird_forward(q, k, v2, rand, None, bs)
        assert (not np.array_equal(out[0, 0, rows], base[0, 0, rows])) == moves, J
    # the global rows see every block
    v2 = v.copy()
    v2[0, 0, 5 * bs:6 * bs] += 1.0
    out = oracle.bigbird_forward(q, k, v2, rand, None, bs)
    assert not np.array_equal(out[0, 0, :bs], base[0, 0, :bs])
    assert not np.array_equal(out[0, 0, -bs:], base[0, 0, -bs:])


def test_bigbird_picks_outside_the_grid_name_nothing():
    q, k, v = rand_qkv(1, 1, 512, seed=65)
    none = oracle.bigbird_forward(q, k, v, np.full((1, 1, 8, 2), -1, np.int32), None, 64)
    bad = np.full((1, 1, 8, 2), 8, np.int32)
    bad[..., 1] = -5
    assert np.array_equal(oracle.bigbird_forward(q, k, v, bad, None, 64), none)
    # picks inside the window or on a global block change nothing either
    inside = np.zeros((1, 1, 8, 2), np.int32)
    inside[0, 0, :, 1] = np.clip(np.arange(8) + 1, 0, 7)
    assert np.array_equal(oracle.bigbird_forward(q, k, v, inside, None, 64), none)


def test_bigbird_generator_draws_outside_window_and_globals():
    rand = workloads.bigbird_rand(2, 3, 4096, 64, 3, seed=66)
    nbb = 64
    for I in range(nbb):
        picks = rand[:, :, I].reshape(-1, 3)
        assert np.all(picks >= 1) and np.all(picks <= nbb - 2)
        assert np.all(np.abs(picks - I) > 1)
        assert all(len(set(p.tolist())) == 3 for p in picks)


def test_bigbird_gradients_equal_block_masked_autograd():
    B, H, N, bs = 1, 2, 512, 64
    q, k, v = rand_qkv(B, H, N, seed=67)
    rand = workloads.bigbird_rand(B, H, N, bs, 2, seed=68)
    mask = np.ones((B, N), np.uint8)
    mask[0, 450:] = 0
    g = rand_dout(q.shape, 69) * mask[:, None, :, None].astype(np.float32)   # padded rows output 0
    got = oracle.bigbird_backward(q, k, v, rand, g, mask, bs)
    for h in range(H):
        allowed = bigbird_allowed(N, bs, rand[0, h]) & mask[0][None, :].astype(bool)
        allowed[~mask[0].astype(bool)] = True   # padded query rows: any finite row (their dO is 0)
        ref = sdpa64_grads(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], g[:, h:h + 1], allowed[None, None])
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a[:, h:h + 1], b, rtol=0, atol=1e-11)
