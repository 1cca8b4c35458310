"""GPU parity of the backward pass (mra_attention_bwd, through the C ABI)
against the CPU oracle's gradients (oracle.mra_backward), in sparse and full
mode.

The gradients run in bf16 operands with fp32 accumulation: the inputs, P and
dS enter the products rounded to bf16 (unit roundoff u = 2^-9 each), and
D_t = dO_t . O_t uses the forward's bf16 output.  Each gradient element is a
sum of terms carrying about two such roundings (P or dS, and D through the
cancellation in dP - D), so its error relative to the tensor's scale is a few
u: the bounds below are max |err| <= 8u max |ref| and
sum |err| / sum |ref| <= 3u (TOL_BWD).  Measured over every bf16 case in the
GPU suite: at most 4.6u (C4's dq) and 2.0u.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

U_BF16 = 2.0 ** -9
TOL_BWD = dict(max_rel_to_scale=8 * U_BF16, mean_rel=3 * U_BF16)
# fp32 inputs: fp32 products and sums (unit roundoff 2^-24, over contractions
# of 64 channels or 32 tokens per block and a few hundred blocks), the
# hardware exp2 (about 2^-22 relative) and the cancellation in dP - D;
# relative to each tensor's scale, max |err| <= 2^-17 max |ref| and
# sum |err| / sum |ref| <= 2^-20.  Measured: at most 2.7e-6 and 3.6e-7.
TOL_BWD32 = dict(max_rel_to_scale=2.0 ** -17, mean_rel=2.0 ** -20)


@pytest.fixture(scope="module")
def mra():
    import block_sparse_approximate_amd as m
    m.lib()
    return m


def to_dev(x_bits):
    return torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_of(w, name):
    if w.dtype == "bf16":
        return to_dev(w.raw(name))
    return torch.from_numpy(np.ascontiguousarray(w.raw(name))).cuda()


def bf16_round(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def run_case(mra, w, seed=7, bwd_workspace=None):
    q, k, v = dev_of(w, "q"), dev_of(w, "k"), dev_of(w, "v")
    dt = q.dtype
    mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
    kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode, initial_prior_first_n_blocks=w.prior_first,
              initial_prior_diagonal_n_blocks=w.prior_diag)
    ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, w.d, dt, w.block_per_row, w.approx_mode),
                     dtype=torch.uint8, device="cuda")
    out = mra.attention(q, k, v, mask, workspace=ws, save_stats=True, **kw)
    g = np.random.default_rng(seed).standard_normal(q.shape).astype(np.float32)
    g = bf16_round(g) if dt == torch.bfloat16 else torch.from_numpy(g)
    dq, dk, dv = mra.attention_backward(q, k, v, out, g.to(dt).cuda(), ws, mask, bwd_workspace=bwd_workspace, **kw)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy() for t in (dq, dk, dv)]
    ref = oracle.mra_backward(w.q, w.k, w.v, g.float().numpy(), w.mask, w.block_per_row, w.approx_mode,
                              w.prior_first, w.prior_diag)
    return got, ref


def check(name, got, ref, tol=TOL_BWD):
    for label, a, b in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(a - b)
        scale = float(np.abs(b).max())
        rel = float(err.max()) / scale if scale > 0 else float(err.max())
        mean_rel = float(err.sum() / np.abs(b).sum()) if scale > 0 else 0.0
        print("  %s %s: max|err|/max|ref| %.3e  mean_rel %.3e  (max|ref| %.3e)" % (name, label, rel, mean_rel, scale),
              flush=True)
        assert np.isfinite(a).all(), label
        if scale == 0:
            assert err.max() == 0, label
            continue
        assert rel <= tol["max_rel_to_scale"], (label, rel)
        assert mean_rel <= tol["mean_rel"], (label, mean_rel)


def small(name, B, H, N, seed=0, mask=None, mode="sparse", dtype="bf16", **kw):
    return workloads.iid(name, B, H, N, dtype=dtype, seed=seed, scale=0.7, mask=mask, approx_mode=mode, **kw)


def ragged_mask(B, N, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((B, N), np.uint8)
    for b in range(B):
        m[b, : int(rng.integers(N // 2, N))] = 1
    m[0, 5] = 0
    return m


CASES = [
    ("one-block", dict(B=1, H=2, N=32)),
    ("nb8-bpr2", dict(B=1, H=3, N=256, block_per_row=2)),
    ("ragged-nb13-masked", dict(B=2, H=1, N=416, block_per_row=3, mask=ragged_mask(2, 416, 3))),
    ("priors", dict(B=1, H=2, N=1024, block_per_row=3, prior_first=2, prior_diag=3)),
    ("all-selected", dict(B=1, H=2, N=256, block_per_row=8)),
    ("long-rows", dict(B=1, H=2, N=2048, block_per_row=2, prior_first=1)),
]


@pytest.mark.parametrize("mode", ["sparse", "full"])
@pytest.mark.parametrize("name,kw", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(mra, name, kw, mode):
    w = small(name, mode=mode, **kw)
    print("case", name, mode, w, flush=True)
    got, ref = run_case(mra, w)
    check(name, got, ref)


@pytest.mark.parametrize("cfg", ["C3", "C4", "C2"])
def test_backward_named_workload(mra, cfg):
    # C3: bf16 B=2 H=12 N=4096 sparse with priors; C4: the same shape in full
    # mode on clustered inputs; C2: bf16 B=8 H=12 N=512 full mode, ragged mask
    w = workloads.get(cfg)
    print("case", w, flush=True)
    got, ref = run_case(mra, w)
    check(cfg, got, ref)


def test_backward_all_selected_equals_dense_autograd(mra):
    # every block selected: the gradients are those of dense attention
    # (torch autograd in fp64 on the CPU, a library routine)
    w = small("dense", B=1, H=2, N=256, block_per_row=8, seed=5)
    got, _ = run_case(mra, w, seed=9)
    g = bf16_round(np.random.default_rng(9).standard_normal((1, 2, 256, 64)).astype(np.float32)).double()
    tq, tk, tv = (torch.from_numpy(np.asarray(x, np.float64)).requires_grad_(True) for x in (w.q, w.k, w.v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).backward(g)
    check("dense", got, [t.grad.numpy() for t in (tq, tk, tv)])


@pytest.mark.parametrize("mode", ["sparse", "full"])
def test_backward_is_deterministic(mra, mode):
    w = small("det", B=1, H=2, N=1024, block_per_row=3, seed=4, prior_first=1, mode=mode)
    a, _ = run_case(mra, w)
    b, _ = run_case(mra, w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_full_block_constant_qk_matches_dense_along_blocks(mra):
    # rows of q and k equal within each 32-token block: there the low-res
    # branch is exact, so full mode coincides with dense attention on the
    # subspace of block-constant q and k.  Derivatives along that subspace
    # agree: dv everywhere (P is constant across a key block) and dq, dk
    # summed over each block (the per-token parts off the subspace differ:
    # a block mean spreads its gradient evenly).  Dense gradients: torch
    # autograd in fp64 on the CPU.
    rng = np.random.default_rng(21)
    B, H, N, d = 1, 2, 256, 64
    qb = np.repeat(rng.standard_normal((B, H, N // 32, d)).astype(np.float32) * 0.7, 32, axis=2)
    kb = np.repeat(rng.standard_normal((B, H, N // 32, d)).astype(np.float32) * 0.7, 32, axis=2)
    vv = rng.standard_normal((B, H, N, d)).astype(np.float32)
    w = workloads.from_arrays("blockconst", qb, kb, vv, dtype="bf16", block_per_row=2, approx_mode="full")
    got, _ = run_case(mra, w, seed=22)
    g = bf16_round(np.random.default_rng(22).standard_normal((B, H, N, d)).astype(np.float32)).double()
    tq, tk, tv = (torch.from_numpy(np.asarray(x, np.float64)).requires_grad_(True) for x in (w.q, w.k, w.v))
    torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).backward(g)
    dense = [t.grad.numpy() for t in (tq, tk, tv)]
    bsum = lambda x: x.reshape(B, H, N // 32, 32, d).sum(axis=3)
    check("blockconst", [bsum(got[0]), bsum(got[1]), got[2]], [bsum(dense[0]), bsum(dense[1]), dense[2]])


def test_backward_reused_workspace_matches_fresh(mra):
    # a backward workspace left over from a larger call holds stale chunk
    # lists and partials; nothing of it may leak into the next call
    big = small("big", B=1, H=2, N=2048, block_per_row=3, prior_first=2, seed=11, mode="full")
    little = small("little", B=1, H=3, N=512, block_per_row=2, prior_diag=3, seed=12, mode="full")
    bw = torch.empty(mra.backward_workspace_size(1, 2, 2048, block_per_row=3, approx_mode="full"),
                     dtype=torch.uint8, device="cuda")
    run_case(mra, big, bwd_workspace=bw)
    reused, ref = run_case(mra, little, bwd_workspace=bw)
    fresh, _ = run_case(mra, little)
    for x, y in zip(reused, fresh):
        assert np.array_equal(x, y)
    check("little", reused, ref)



@pytest.mark.parametrize("mode", ["sparse", "full"])
@pytest.mark.parametrize("name,kw", [c for c in CASES if c[0] in ("one-block", "ragged-nb13-masked", "priors",
                                                                  "long-rows")], ids=lambda x: x if isinstance(x, str) else "")
def test_backward_fp32_matches_oracle(mra, name, kw, mode):
    w = small(name + "-f32", mode=mode, dtype="f32", **kw)
    print("case", name, mode, w, flush=True)
    got, ref = run_case(mra, w)
    check(name, got, ref, TOL_BWD32)


def test_backward_fp32_named_workload(mra):
    w = workloads.get("C1")   # fp32, B=1, H=2, N=512, full mode
    print("case", w, flush=True)
    got, ref = run_case(mra, w)
    check("C1", got, ref, TOL_BWD32)
