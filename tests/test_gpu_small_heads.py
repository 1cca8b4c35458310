"""Heads narrower than 64 channels on the GPU: zero-padded to the kernels'
64 with the logit scale of their own size (mra_dims.scale_dim), against the
CPU oracle run at the true head size.  Zero channels add exact zeros to every
pooled mean, logit and product, so the selection must match bit for bit and
the outputs to the usual tolerance; the padded channels of the results must
be exactly zero.  The smallest case is the page's test configuration
(hidden size 16 over 2 heads: head size 8, sequence 64)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {"f32": dict(max_abs=1e-4, mean_rel=None), "bf16": dict(max_abs=2e-2, mean_rel=1e-2)}


@pytest.fixture(scope="module")
def mra():
    import block_sparse_approximate_amd as m
    m.lib()
    return m


def padded(w, name):
    x = np.zeros(w.q.shape[:3] + (64,), np.float32)
    x[..., :w.d] = getattr(w, name)
    t = torch.from_numpy(x)
    return (t.to(torch.bfloat16) if w.dtype == "bf16" else t).cuda()


def close(w, got, ref):
    err = np.abs(got - ref)
    tol = TOL[w.dtype]
    mean_rel = float(err.sum() / max(np.abs(ref).sum(), 1e-300))
    print("  %s: max_abs %.3e mean_rel %.3e" % (w.name, err.max(), mean_rel), flush=True)
    assert err.max() <= tol["max_abs"]
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"]


@pytest.mark.parametrize("d,dtype,mode", [(8, "bf16", "full"), (16, "bf16", "sparse"), (32, "bf16", "full"),
                                          (32, "f32", "sparse"), (48, "f32", "full"), (32, "bf16", "sparse")])
def test_small_heads_forward(mra, d, dtype, mode):
    w = workloads.iid("d%d" % d, 2, 3, 1024, d=d, dtype=dtype, seed=d, scale=1.0, block_per_row=3,
                      approx_mode=mode, prior_first=1 if mode == "sparse" else 0, prior_diag=3)
    print("case", w, flush=True)
    q, k, v = padded(w, "q"), padded(w, "k"), padded(w, "v")
    kw = dict(block_per_row=w.block_per_row, approx_mode=mode, initial_prior_first_n_blocks=w.prior_first,
              initial_prior_diagonal_n_blocks=w.prior_diag, scale_dim=d)
    st = mra.debug_stages(q, k, v, None, **kw)
    out = mra.attention(q, k, v, None, **kw)
    torch.cuda.synchronize()
    ref, sel = oracle.mra_forward(w.q, w.k, w.v, None, w.block_per_row, mode, w.prior_first, w.prior_diag,
                                  return_selection=True)
    assert int(st["error"][0].item()) == 0
    assert np.array_equal(st["sel"].cpu().numpy(), sel)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(got[..., d:] == 0)
    close(w, got[..., :d], ref)


@pytest.mark.parametrize("dtype,mode", [("bf16", "full"), ("f32", "sparse")])
def test_small_heads_backward(mra, dtype, mode):
    d = 32
    w = workloads.iid("bwd-d32", 1, 2, 1024, d=d, dtype=dtype, seed=3, scale=1.0, block_per_row=3,
                      approx_mode=mode, prior_diag=3)
    q, k, v = padded(w, "q"), padded(w, "k"), padded(w, "v")
    kw = dict(block_per_row=w.block_per_row, approx_mode=mode, initial_prior_diagonal_n_blocks=w.prior_diag,
              scale_dim=d)
    dt = q.dtype
    ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, 64, dt, w.block_per_row, mode), dtype=torch.uint8,
                     device="cuda")
    out = mra.attention(q, k, v, None, workspace=ws, save_stats=True, **kw)
    g = np.zeros(q.shape, np.float32)
    g[..., :d] = np.random.default_rng(4).standard_normal(w.q.shape).astype(np.float32)
    gt = torch.from_numpy(g).to(dt)
    grads = mra.attention_backward(q, k, v, out, gt.cuda(), ws, None, **kw)
    torch.cuda.synchronize()
    ref = oracle.mra_backward(w.q, w.k, w.v, gt.float().numpy()[..., :d], None, w.block_per_row, mode, 0,
                              w.prior_diag)
    from test_gpu_backward import TOL_BWD, TOL_BWD32
    t = TOL_BWD if dtype == "bf16" else TOL_BWD32
    tol = (t["max_rel_to_scale"], t["mean_rel"])
    for label, a, b in zip(("dq", "dk", "dv"), grads, ref):
        a = a.float().cpu().numpy()
        assert np.all(a[..., d:] == 0), label
        err = np.abs(a[..., :d] - b)
        rel, mean_rel = err.max() / np.abs(b).max(), err.sum() / np.abs(b).sum()
        print("  %s %s: %.3e %.3e" % (dtype, label, rel, mean_rel), flush=True)
        assert rel <= tol[0] and mean_rel <= tol[1], (label, rel, mean_rel)


def test_page_test_shape_through_the_layer(mra):
    # hidden 16 over 2 heads (head size 8), sequence 64, as in the page's tests
    from block_sparse_approximate_amd.layer import MraSelfAttention
    torch.manual_seed(5)
    mod = MraSelfAttention(16, 2, block_per_row=4, approx_mode="full").cuda()
    x = torch.randn(3, 64, 16, device="cuda", requires_grad=True)
    y = mod(x)
    y.sum().backward()
    torch.cuda.synchronize()
    with torch.no_grad():
        heads = lambda t: t.view(3, 64, 2, 8).transpose(1, 2).cpu().numpy()
        q, k, v = heads(mod.query(x)), heads(mod.key(x)), heads(mod.value(x))
    ref = oracle.mra_forward(q, k, v, None, 4, "full").transpose(0, 2, 1, 3).reshape(3, 64, 16)
    err = np.abs(y.detach().cpu().numpy() - ref)
    print("  layer d=8: max_abs %.3e" % err.max(), flush=True)
    assert err.max() <= 1e-4
    assert torch.isfinite(x.grad).all() and x.grad.abs().sum() > 0
