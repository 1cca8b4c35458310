"""GPU tests of the torch modules around the kernels (block_sparse_approximate_amd.layer):
the autograd function against the oracle's forward and gradients, the
self-attention module's padding of seq_len to a multiple of 32, and one
encoder layer against the same layer with dense attention where every block
is selected (there MRA-2 is dense attention, [MRA] 第三步 with nothing left
for the low-res branch)."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

from test_gpu_backward import TOL_BWD  # noqa: E402  (the bf16 gradient bounds, derived there)

# The whole layer in bf16 against the same layer with dense attention: the
# projections, LayerNorm and feed-forward block add bf16 roundings of their
# own on both sides, and the weight gradients sum over every token.  Measured:
# output and input gradient at most 6.7e-3 / 3.3e-3 (max / mean relative),
# weight gradients 4.6e-3 / 4.8e-3.
TOL_LAYER = dict(max_rel=2.0 ** -6, mean_rel=2.0 ** -7)
TOL_LAYER_WEIGHTS = dict(max_rel=2.0 ** -6, mean_rel=2.0 ** -6)


@pytest.fixture(scope="module")
def layer():
    import block_sparse_approximate_amd as m
    m.lib()
    from block_sparse_approximate_amd import layer as L
    return L


def close(name, got, ref, max_rel=TOL_BWD["max_rel_to_scale"], mean_rel=TOL_BWD["mean_rel"]):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    scale = float(np.abs(ref).max())
    r = float(err.max()) / scale
    m = float(err.sum() / np.abs(ref).sum())
    print("  %s: max|err|/max|ref| %.3e  mean_rel %.3e" % (name, r, m), flush=True)
    assert np.isfinite(got).all(), name
    assert r <= max_rel and m <= mean_rel, (name, r, m)


def bf16_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("mode", ["sparse", "full"])
def test_function_forward_and_gradients_match_oracle(layer, mode):
    w = workloads.iid("fn-" + mode, 1, 2, 512, dtype="bf16", seed=31, scale=0.7, block_per_row=3,
                      approx_mode=mode, prior_first=1, prior_diag=3)
    q, k, v = (bf16_dev(x).requires_grad_(True) for x in (w.q, w.k, w.v))
    out = layer.mra_attention(q, k, v, None, w.block_per_row, mode, w.prior_first, w.prior_diag)
    g = np.random.default_rng(32).standard_normal(q.shape).astype(np.float32)
    g16 = torch.from_numpy(g).to(torch.bfloat16)
    out.backward(g16.cuda())
    ref_out = oracle.mra_forward(w.q, w.k, w.v, None, w.block_per_row, mode, w.prior_first, w.prior_diag)
    err = np.abs(out.detach().float().cpu().numpy() - ref_out)
    assert err.max() <= 2e-2 and err.sum() / np.abs(ref_out).sum() <= 1e-2
    ref = oracle.mra_backward(w.q, w.k, w.v, g16.float().numpy(), None, w.block_per_row, mode, w.prior_first,
                              w.prior_diag)
    for name, t, r in zip(("dq", "dk", "dv"), (q, k, v), ref):
        close(name, t.grad.float().cpu().numpy(), r)


@pytest.mark.parametrize("d", [96, 128])
def test_wide_heads_match_oracle(layer, d):
    # heads of 65 to 128 channels: zero-padded to the 128-channel kernels
    # with their own logit scale, forward and gradients
    w = workloads.iid("wide-%d" % d, 1, 2, 512, d=d, dtype="bf16", seed=d, scale=0.7, block_per_row=3,
                      approx_mode="full", prior_diag=1)
    q, k, v = (bf16_dev(x).requires_grad_(True) for x in (w.q, w.k, w.v))
    out = layer.mra_attention(q, k, v, None, w.block_per_row, "full", 0, w.prior_diag)
    ref = oracle.mra_forward(w.q, w.k, w.v, None, w.block_per_row, "full", 0, w.prior_diag)
    assert out.shape == q.shape
    err = np.abs(out.detach().float().cpu().numpy() - ref)
    assert err.max() <= 2e-2 and err.sum() / np.abs(ref).sum() <= 1e-2
    g = np.random.default_rng(d + 1).standard_normal(q.shape).astype(np.float32)
    g16 = torch.from_numpy(g).to(torch.bfloat16)
    out.backward(g16.cuda())
    refg = oracle.mra_backward(w.q, w.k, w.v, g16.float().numpy(), None, w.block_per_row, "full", 0, w.prior_diag)
    for name, t, r in zip(("dq", "dk", "dv"), (q, k, v), refg):
        assert t.grad.shape == t.shape
        close(name, t.grad.float().cpu().numpy(), r)


def test_self_attention_pads_to_a_block_multiple(layer):
    torch.manual_seed(0)
    B, N, hidden = 2, 100, 128
    mod = layer.MraSelfAttention(hidden, 2, block_per_row=2, approx_mode="full").cuda().to(torch.bfloat16)
    x = torch.randn(B, N, hidden, device="cuda").to(torch.bfloat16)
    am = torch.ones(B, N, dtype=torch.uint8, device="cuda")
    am[1, 70:] = 0
    with torch.no_grad():
        got = mod(x, am).float().cpu().numpy()
        # the inputs the kernels see: the same projections of the zero-padded sequence
        xp = torch.nn.functional.pad(x, (0, 0, 0, 28))
        heads = lambda t: t.view(B, 128, 2, 64).transpose(1, 2).float().cpu().numpy()
        q, k, v = heads(mod.query(xp)), heads(mod.key(xp)), heads(mod.value(xp))
    assert got.shape == (B, N, hidden)
    mask = np.zeros((B, 128), np.uint8)
    mask[0, :100] = 1
    mask[1, :70] = 1
    ref = oracle.mra_forward(q, k, v, mask, 2, "full")              # [B, H, 128, 64]
    ref = ref.transpose(0, 2, 1, 3).reshape(B, 128, hidden)[:, :N]
    err = np.abs(got - ref)
    print("  padded: max_abs %.3e" % err.max(), flush=True)
    assert err.max() <= 2e-2 and err.sum() / np.abs(ref).sum() <= 1e-2
    assert np.all(got[1, 70:] == 0)                                  # padded query rows output 0


def dense_layer_reference(mod, x):
    """The same encoder layer on the CPU in fp32 with dense softmax attention
    (torch scaled_dot_product_attention), weights copied from mod."""
    ref = type(mod)(hidden_size=x.shape[-1], num_attention_heads=mod.attention.num_attention_heads,
                    intermediate_size=mod.intermediate.out_features)
    ref.load_state_dict({k: t.float().cpu() for k, t in mod.state_dict().items()})
    xr = x.detach().float().cpu().requires_grad_(True)
    B, N, Hd = xr.shape
    H = ref.attention.num_attention_heads
    split = lambda t: t.view(B, N, H, Hd // H).transpose(1, 2)
    a = torch.nn.functional.scaled_dot_product_attention(split(ref.attention.query(xr)), split(ref.attention.key(xr)),
                                                         split(ref.attention.value(xr)))
    a = a.transpose(1, 2).reshape(B, N, Hd)
    h = ref.attn_norm(ref.attn_out(a) + xr)
    y = ref.out_norm(ref.out(torch.nn.functional.gelu(ref.intermediate(h))) + h)
    return ref, xr, y


def test_layer_with_every_block_selected_matches_dense_layer(layer):
    torch.manual_seed(1)
    B, N, hidden = 2, 128, 256           # nb = 4, bpr 4: all 16 cells selected
    mod = layer.MraLayer(hidden, 4, intermediate_size=512, block_per_row=4, approx_mode="full").cuda()
    mod = mod.to(torch.bfloat16)
    x = (torch.randn(B, N, hidden, device="cuda") * 0.5).to(torch.bfloat16).requires_grad_(True)
    y = mod(x)
    gy = torch.randn(B, N, hidden).to(torch.bfloat16)
    y.backward(gy.cuda())
    ref, xr, yr = dense_layer_reference(mod, x)
    yr.backward(gy.float())
    close("y", y.detach().float().cpu().numpy(), yr.detach().numpy(), **TOL_LAYER)
    close("dx", x.grad.float().cpu().numpy(), xr.grad.numpy(), **TOL_LAYER)
    for name in ("attention.query.weight", "attention.key.weight", "attention.value.weight"):
        got = dict(mod.named_parameters())[name].grad.float().cpu().numpy()
        want = dict(ref.named_parameters())[name].grad.numpy()
        close(name, got, want, **TOL_LAYER_WEIGHTS)
