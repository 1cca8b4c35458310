"""128-channel heads on the GPU: the forward kernels built for 128 channels
against the CPU oracle at the same head size.

* Stages 1-2 (pooled blocks, counts, low-res logits, row maxima, selected
  block sets) bit for bit: the fp32 sums run over 128 channels in the same
  order on both sides.
* Outputs: fp32 within 1e-4 max-abs; bf16 within 2e-2 max-abs and 1e-2
  mean-relative over valid query rows; padded query rows exactly 0.
Cases cover both modes and dtypes, ragged masks, priors, a fully masked
sequence, the one-block sequence and the N = 4096 and 16384 shapes of the
named workloads.  The backward pass at 128 channels is checked against the
oracle's gradients with the bounds of tests/test_gpu_backward.py.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_backward import TOL_BWD, TOL_BWD32, check, run_case

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-4, mean_rel=None), "bf16": dict(max_abs=2e-2, mean_rel=1e-2)}


@pytest.fixture(scope="module")
def mra():
    import block_sparse_approximate_amd as m
    m.lib()
    return m


def dev(w, name):
    x = w.raw(name)
    if w.dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def dev_mask(w):
    return None if w.mask is None else torch.from_numpy(w.mask).cuda()


def kwargs(w):
    return dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode,
                initial_prior_first_n_blocks=w.prior_first, initial_prior_diagonal_n_blocks=w.prior_diag)


def bits_equal(a, b):
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def ragged_mask(B, N, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((B, N), np.uint8)
    for b in range(B):
        m[b, :int(rng.integers(N // 2, N + 1))] = 1
    m[0, 40:45] = 0   # a hole inside a block
    return m


def assert_close(w, got, ref):
    valid = np.ones((w.B, w.N), bool) if w.mask is None else w.mask.astype(bool)
    vrows = np.broadcast_to(valid[:, None, :], (w.B, w.H, w.N))
    assert np.all(got[~vrows] == 0), "padded query rows must be 0"
    g, r = got[vrows], ref[vrows]
    err = np.abs(g - r)
    tol = TOL[w.dtype]
    max_abs = float(err.max()) if err.size else 0.0
    mean_rel = float(err.sum() / max(np.abs(r).sum(), 1e-300))
    print("  %s: max_abs %.3e mean_rel %.3e" % (w.name, max_abs, mean_rel), flush=True)
    assert max_abs <= tol["max_abs"]
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"]


def check_stages(mra, w):
    r = mra.debug_stages(dev(w, "q"), dev(w, "k"), dev(w, "v"), dev_mask(w), **kwargs(w))
    torch.cuda.synchronize()
    g = {k: (None if v is None else v.cpu().numpy()) for k, v in r.items()}
    assert int(g["error"][0]) == 0
    K = oracle.num_block(w.N, w.block_per_row)
    for b in range(w.B):
        m = None if w.mask is None else w.mask[b]
        for h in range(w.H):
            qh, cnt = oracle.pool_f32(w.q[b, h], m)
            kh, _ = oracle.pool_f32(w.k[b, h], m)
            S = oracle.lowres_logits_f32(qh, kh)
            rm, sc = oracle.scores_f32(S, cnt, w.prior_first, w.prior_diag)
            assert np.array_equal(g["count"][b], cnt)
            assert bits_equal(g["qhat"][b, h], qh) and bits_equal(g["khat"][b, h], kh)
            assert bits_equal(g["logits"][b, h], S) and bits_equal(g["rowmax"][b, h], rm)
            if w.approx_mode == "full":
                vh, _ = oracle.pool_f32(w.v[b, h], m)
                assert bits_equal(g["vhat"][b, h], vh)
            assert np.array_equal(g["sel"][b, h], oracle.select_top(sc, K))


def check_output(mra, w):
    out = mra.attention(dev(w, "q"), dev(w, "k"), dev(w, "v"), dev_mask(w), **kwargs(w))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.mra_forward(w.q, w.k, w.v, w.mask, w.block_per_row, w.approx_mode, w.prior_first, w.prior_diag)
    assert_close(w, got, ref)


CASES = [
    # name, B, H, N, dtype, mode, bpr, prior_first, prior_diag, masked
    ("bf16-full-mask", 2, 3, 1024, "bf16", "full", 4, 0, 0, True),
    ("bf16-sparse-priors", 2, 3, 1024, "bf16", "sparse", 3, 1, 3, False),
    ("f32-full-diag", 1, 2, 512, "f32", "full", 4, 0, 1, True),
    ("f32-sparse", 1, 3, 512, "f32", "sparse", 2, 0, 0, False),
    ("bf16-full-ragged-tail", 2, 2, 800, "bf16", "full", 5, 2, 2, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_head128_stages_and_output(mra, case):
    name, B, H, N, dtype, mode, bpr, pf, pd, masked = case
    w = workloads.iid("d128-" + name, B, H, N, d=128, dtype=dtype, seed=N + bpr, scale=0.7, block_per_row=bpr,
                      approx_mode=mode, prior_first=pf, prior_diag=pd,
                      mask=ragged_mask(B, N, 3) if masked else None)
    print("case", w, flush=True)
    check_stages(mra, w)
    check_output(mra, w)


@pytest.mark.parametrize("mode", ["full", "sparse"])
def test_head128_single_block_and_empty_sequence(mra, mode):
    w = workloads.iid("d128-one-block", 1, 2, 32, d=128, dtype="bf16", seed=5, block_per_row=1, approx_mode=mode)
    print("case", w, flush=True)
    check_output(mra, w)
    mask = np.ones((2, 256), np.uint8)
    mask[1] = 0
    w = workloads.iid("d128-empty-seq", 2, 2, 256, d=128, dtype="f32", seed=6, block_per_row=2, approx_mode=mode,
                      mask=mask)
    print("case", w, flush=True)
    check_output(mra, w)


@pytest.mark.parametrize("mode,pf,pd", [("full", 0, 0), ("sparse", 2, 3)])
def test_head128_n4096(mra, mode, pf, pd):
    w = workloads.iid("d128-N4096-" + mode, 2, 4, 4096, d=128, dtype="bf16", seed=41, scale=0.5, block_per_row=4,
                      approx_mode=mode, prior_first=pf, prior_diag=pd)
    print("case", w, flush=True)
    check_stages(mra, w)
    check_output(mra, w)


def test_head128_n16384(mra):
    w = workloads.iid("d128-N16384-full", 1, 2, 16384, d=128, dtype="bf16", seed=42, scale=0.5, block_per_row=8,
                      approx_mode="full", prior_diag=1)
    print("case", w, flush=True)
    check_stages(mra, w)
    check_output(mra, w)


def test_head128_matches_padded_head64_path(mra):
    # 64-channel heads zero-padded to 128 with the 64-channel logit scale:
    # the zeros change no sum, so the 128-channel kernels must give the
    # 64-channel kernels' selection and, within rounding, their output
    w = workloads.iid("d64", 2, 3, 1024, d=64, dtype="bf16", seed=9, scale=0.8, block_per_row=3, approx_mode="full",
                      prior_diag=1)
    q, k, v = dev(w, "q"), dev(w, "k"), dev(w, "v")
    pad = lambda t: torch.nn.functional.pad(t, (0, 64)).contiguous()
    kw = kwargs(w)
    s64 = mra.debug_stages(q, k, v, None, **kw)
    s128 = mra.debug_stages(pad(q), pad(k), pad(v), None, scale_dim=64, **kw)
    o64 = mra.attention(q, k, v, None, **kw)
    o128 = mra.attention(pad(q), pad(k), pad(v), None, scale_dim=64, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s64["sel"], s128["sel"])
    assert torch.equal(s64["logits"], s128["logits"])
    assert torch.all(o128[..., 64:] == 0)
    assert (o128[..., :64].float() - o64.float()).abs().max().item() <= 2e-2


BWD_CASES = [
    # name, B, H, N, dtype, mode, bpr, prior_first, prior_diag, masked
    ("bf16-sparse-priors", 1, 3, 1024, "bf16", "sparse", 3, 1, 3, False),
    ("bf16-full-mask", 2, 2, 1024, "bf16", "full", 4, 0, 1, True),
    ("f32-sparse-mask", 1, 2, 512, "f32", "sparse", 3, 0, 3, True),
    ("f32-full", 1, 2, 512, "f32", "full", 4, 1, 0, False),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_head128_backward(mra, case):
    name, B, H, N, dtype, mode, bpr, pf, pd, masked = case
    w = workloads.iid("d128-bwd-" + name, B, H, N, d=128, dtype=dtype, seed=N + 7 * bpr, scale=0.7,
                      block_per_row=bpr, approx_mode=mode, prior_first=pf, prior_diag=pd,
                      mask=ragged_mask(B, N, 4) if masked else None)
    print("case", w, flush=True)
    got, ref = run_case(mra, w)
    check(w.name, got, ref, TOL_BWD if dtype == "bf16" else TOL_BWD32)


@pytest.mark.parametrize("mode,pf,pd", [("sparse", 2, 3), ("full", 0, 0)])
def test_head128_backward_n4096(mra, mode, pf, pd):
    w = workloads.iid("d128-bwd-N4096-" + mode, 1, 4, 4096, d=128, dtype="bf16", seed=77, scale=0.5,
                      block_per_row=4, approx_mode=mode, prior_first=pf, prior_diag=pd)
    print("case", w, flush=True)
    got, ref = run_case(mra, w)
    check(w.name, got, ref)


def test_head128_bigbird_forward_and_backward(mra):
    bb = workloads.bigbird("d128-BB-bs64-r2", B=1, H=2, N=2048, block_size=64, r=2, seed=13, d=128,
                           mask=ragged_mask(1, 2048, 8))
    w = bb.w
    print("case", bb, flush=True)
    mask = torch.from_numpy(w.mask).cuda()
    q, k, v = dev(w, "q"), dev(w, "k"), dev(w, "v")
    r = bb.rand.shape[3]
    ws = torch.zeros(mra.bigbird_workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, bb.block_size, r),
                     dtype=torch.uint8, device="cuda")
    out = mra.bigbird_attention(q, k, v, torch.from_numpy(bb.rand).cuda(), mask, bb.block_size, workspace=ws)
    g16 = torch.from_numpy(np.random.default_rng(14).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
    grads = mra.bigbird_backward(q, k, v, out, g16.cuda(), ws, r, mask, bb.block_size)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "device error word"
    assert_close(w, out.float().cpu().numpy().astype(np.float64),
                 oracle.bigbird_forward(w.q, w.k, w.v, bb.rand, w.mask, bb.block_size))
    ref = oracle.bigbird_backward(w.q, w.k, w.v, bb.rand, g16.float().numpy(), w.mask, bb.block_size)
    check(w.name, [t.float().cpu().numpy() for t in grads], ref)
