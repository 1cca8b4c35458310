"""GPU parity of BigBird block-sparse attention (mra_bigbird_fwd through the
C ABI) against the CPU oracle (oracle.bigbird_forward): the pattern of the
BigBird page (window of three blocks, first and last blocks global, given
random blocks) run through the same block-attention and join kernels as
MRA's sparse mode."""
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


def dev(w, name):
    x = w.raw(name)
    if w.dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def run(mra, bb):
    w = bb.w
    mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ws = torch.zeros(mra.bigbird_workspace_size(w.B, w.H, w.N, w.d, dt, bb.block_size, bb.rand.shape[3]),
                     dtype=torch.uint8, device="cuda")
    ws[:4] = 0xFF                  # a stale error word: the call must clear it
    out = mra.bigbird_attention(dev(w, "q"), dev(w, "k"), dev(w, "v"), torch.from_numpy(bb.rand).cuda(), mask,
                                bb.block_size, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "device error word"
    got = out.float().cpu().numpy().astype(np.float64)
    ref = oracle.bigbird_forward(w.q, w.k, w.v, bb.rand, w.mask, bb.block_size)
    valid = np.ones((w.B, w.N), bool) if w.mask is None else w.mask.astype(bool)
    vrows = np.broadcast_to(valid[:, None, :], (w.B, w.H, w.N))
    assert np.all(got[~vrows] == 0)
    err = np.abs(got[vrows] - ref[vrows])
    tol = TOL[w.dtype]
    mean_rel = float(err.sum() / np.abs(ref[vrows]).sum())
    print("  %s: max_abs %.3e mean_rel %.3e" % (w.name, err.max(), mean_rel), flush=True)
    assert err.max() <= tol["max_abs"]
    if tol["mean_rel"] is not None:
        assert mean_rel <= tol["mean_rel"]
    return got


def test_bigbird_named_workload(mra):
    bb = workloads.bigbird()     # bf16 B=2 H=12 N=4096, block 64, 3 random blocks
    print("case", bb, flush=True)
    run(mra, bb)


def ragged_mask(B, N, seed):
    rng = np.random.default_rng(seed)
    m = np.ones((B, N), np.uint8)
    for b in range(B):
        m[b, int(rng.integers(N // 2, N)):] = 0
    m[0, 70] = 0
    return m


@pytest.mark.parametrize("name,kw", [
    ("bs32", dict(B=1, H=2, N=1024, block_size=32, r=2)),
    ("bs64-masked", dict(B=2, H=2, N=2048, block_size=64, r=3, mask=ragged_mask(2, 2048, 5))),
    ("bs128", dict(B=1, H=3, N=2048, block_size=128, r=1)),
    ("fp32", dict(B=1, H=2, N=1024, block_size=64, r=2, dtype="f32")),
    ("short-dense", dict(B=1, H=2, N=192, block_size=64, r=1)),
    ("two-blocks", dict(B=1, H=1, N=128, block_size=64, r=2)),
    ("long-16k", dict(B=1, H=2, N=16384, block_size=64, r=3)),
])
def test_bigbird_shapes(mra, name, kw):
    kw = dict(kw)
    bb = workloads.bigbird(name, seed=7, **kw)
    print("case", bb, flush=True)
    run(mra, bb)


def test_bigbird_picks_outside_grid_and_repeats(mra):
    # picks outside [0, nbb) name nothing; repeats and picks inside the
    # window or on a global block are attended once
    bb = workloads.bigbird("odd-picks", B=1, H=2, N=1024, block_size=64, r=4, seed=8)
    rng = np.random.default_rng(9)
    rand = bb.rand.copy()
    rand[..., 0] = -1
    rand[..., 1] = 16 + rng.integers(0, 5, rand.shape[:3])
    rand[..., 2] = rand[..., 3]
    rand[0, 0, 5, 3] = 5
    rand[0, 1, 6, 3] = 0
    bb.rand = rand
    run(mra, bb)


def test_bigbird_matches_mra_sparse_on_the_same_cells(mra):
    # the same kernels: a short sequence's pattern covers every cell, so the
    # output equals MRA sparse mode with every block selected
    bb = workloads.bigbird("cover", B=1, H=2, N=192, block_size=64, r=1, seed=10)
    got = run(mra, bb)
    w = bb.w
    out = mra.attention(dev(w, "q"), dev(w, "k"), dev(w, "v"), None, block_per_row=6, approx_mode="sparse")
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), got)



from test_gpu_backward import TOL_BWD  # noqa: E402  (the bf16 gradient bounds, derived there)


@pytest.mark.parametrize("name,kw", [
    ("bwd-named", dict()),
    ("bwd-bs32-masked", dict(B=2, H=2, N=1024, block_size=32, r=2, mask=ragged_mask(2, 1024, 6))),
    ("bwd-bs128", dict(B=1, H=2, N=2048, block_size=128, r=1)),
])
def test_bigbird_backward_matches_oracle(mra, name, kw):
    bb = workloads.bigbird(name, seed=11, **kw) if kw else workloads.bigbird()
    w = bb.w
    print("case", bb, flush=True)
    mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
    q, k, v = dev(w, "q"), dev(w, "k"), dev(w, "v")
    rand = torch.from_numpy(bb.rand).cuda()
    ws = torch.zeros(mra.bigbird_workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, bb.block_size,
                                                bb.rand.shape[3]), dtype=torch.uint8, device="cuda")
    out = mra.bigbird_attention(q, k, v, rand, mask, bb.block_size, workspace=ws)
    g16 = torch.from_numpy(np.random.default_rng(12).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
    dq, dk, dv = mra.bigbird_backward(q, k, v, out, g16.cuda(), ws, bb.rand.shape[3], mask, bb.block_size)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0, "device error word"
    ref = oracle.bigbird_backward(w.q, w.k, w.v, bb.rand, g16.float().numpy(), w.mask, bb.block_size)
    for label, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        a = a.float().cpu().numpy()
        err = np.abs(a - b)
        rel = float(err.max()) / float(np.abs(b).max())
        mean_rel = float(err.sum() / np.abs(b).sum())
        print("  %s %s: max|err|/max|ref| %.3e  mean_rel %.3e" % (name, label, rel, mean_rel), flush=True)
        assert np.isfinite(a).all()
        assert rel <= TOL_BWD["max_rel_to_scale"] and mean_rel <= TOL_BWD["mean_rel"], (label, rel, mean_rel)
