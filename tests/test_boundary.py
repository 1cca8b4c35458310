"""CPU tests of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before queueing any
GPU work (so these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import block_sparse_approximate_amd as mra
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mra.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mra_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = mra.lib()
    names = declared_functions()
    assert len(names) == 19
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mra.SIGNATURES)
    assert L.mra_abi_version() == 4


def test_status_strings():
    for s in range(0, 15):
        assert mra.lib().mra_status_string(s)
    assert mra.lib().mra_status_string(99) == b"unknown status"


@pytest.mark.parametrize("N,bpr", [(512, 4), (64, 4), (4096, 4), (16384, 8), (32, 1), (96, 100),
                                   (48, 4), (0, 1), (512, 0), (-64, 2)])
def test_num_block_matches_oracle(N, bpr):
    assert mra.num_block(N, bpr) == oracle.num_block(N, bpr)


def test_workspace_size_grows_and_validates():
    small = mra.workspace_size(1, 2, 512)
    big = mra.workspace_size(2, 12, 4096)
    assert 0 < small < big
    assert mra.workspace_size(2, 12, 4096, approx_mode="sparse") < big
    with pytest.raises(mra.MraError) as e:
        mra.workspace_size(1, 1, 100)
    assert e.value.status == 3
    with pytest.raises(mra.MraError) as e:
        mra.workspace_size(1, 1, 512, head_dim=32)
    assert e.value.status == 4
    # 128-channel heads
    assert mra.workspace_size(2, 12, 4096, head_dim=128) > big
    assert mra.backward_workspace_size(1, 1, 512, head_dim=128) > mra.backward_workspace_size(1, 1, 512)
    assert mra.bigbird_backward_workspace_size(1, 1, 512, head_dim=128) > 0
    assert mra.bigbird_workspace_size(1, 1, 512, head_dim=128) > 0
    with pytest.raises(mra.MraError) as e:
        mra.backward_workspace_size(1, 1, 512, head_dim=96)
    assert e.value.status == 4
    with pytest.raises(mra.MraError) as e:
        mra.workspace_size(1, 1, 512, block_per_row=0)
    assert e.value.status == 7
    with pytest.raises(mra.MraError) as e:
        mra.workspace_size(1, 1, 512, approx_mode="bogus")
    assert e.value.status == 6
    with pytest.raises(mra.MraError) as e:
        mra.workspace_size(1, 1, 32768)
    assert e.value.status == 3


# Fake, aligned, non-null "device" addresses: every call below fails its
# host-side checks, so no address is ever dereferenced.
Q, K, V, O, W = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def call(dims=(1, 2, 512, 64, 1), q=Q, k=K, v=V, mask=None, bpr=4, mode=0, pf=0, pd=0, out=O, ws=W,
         ws_bytes=None):
    d = mra._Dims(*dims)
    if ws_bytes is None:
        ws_bytes = 1 << 40 if ws else 0
    return mra.lib().mra_attention_fwd(ctypes.byref(d), q, k, v, mask, bpr, mode, pf, pd, out, ws, ws_bytes,
                                       None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(dims=(0, 2, 512, 64, 1)), 2), (dict(dims=(1, 0, 512, 64, 1)), 2),
    (dict(dims=(1, 2, 500, 64, 1)), 3), (dict(dims=(1, 2, 0, 64, 1)), 3),
    (dict(dims=(1, 2, 32768, 64, 1)), 3),
    (dict(dims=(1, 2, 512, 96, 1)), 4), (dict(dims=(1, 2, 512, 32, 1)), 4), (dict(dims=(1, 2, 512, 64, 7)), 5),
    (dict(mode=2), 6), (dict(mode=-1), 6), (dict(bpr=0), 7), (dict(pf=-1), 8), (dict(pd=-2), 8),
    (dict(out=Q), 9), (dict(out=W), 9), (dict(out=Q + 4096), 9),
    (dict(ws=None), 10), (dict(ws_bytes=1024), 10),
    (dict(q=Q + 8), 12), (dict(mask=0x60000004), 12), (dict(ws=W + 16), 12),
    # the workspace is written while the inputs are read: it may overlap none of them
    (dict(ws=Q - 256), 9), (dict(ws=V + 4096, ws_bytes=4 << 20), 9), (dict(mask=W + 4096), 9),
])
def test_attention_fwd_rejects_bad_arguments(kw, status):
    assert call(**kw) == status


def call_ex(opts=(4, 0, 0, 0, 1), **kw):
    d = mra._Dims(*kw.get("dims", (1, 2, 512, 64, 1)))
    o = None if opts is None else ctypes.byref(mra._Options(*opts))
    return mra.lib().mra_attention_fwd_ex(ctypes.byref(d), Q, K, V, None, o, kw.get("out", O), W, 1 << 40, None)


@pytest.mark.parametrize("opts,status", [
    (None, 1), ((4, 0, 0, 0, 2), 6), ((4, 0, 0, 0, -1), 6), ((4, 3, 0, 0, 1), 6), ((0, 0, 0, 0, 1), 7),
    ((4, 1, -1, 0, 1), 8), ((4, 0, 0, 2, 0, 2, 0), 8), ((4, 0, 0, 2, 0, -1, 1), 8),
])
def test_attention_fwd_ex_rejects_bad_options(opts, status):
    assert call_ex(opts) == status


def test_attention_fwd_ex_checks_like_fwd():
    assert call_ex(out=None) == 1
    assert call_ex(out=Q) == 9
    assert call_ex(dims=(1, 2, 500, 64, 1)) == 3


def test_null_dims_rejected():
    L = mra.lib()
    assert L.mra_attention_fwd(None, Q, K, V, None, 4, 0, 0, 0, O, W, 1 << 40, None) == 1
    n = ctypes.c_size_t(0)
    assert L.mra_workspace_size(None, 4, 0, ctypes.byref(n)) == 1


def test_debug_select_rejects_bad_arguments():
    L = mra.lib()
    d = mra._Dims(1, 1, 512, 64, 1)
    assert L.mra_debug_select(ctypes.byref(d), None, K, 4, 0, 0, 0, 0, O, W, 1 << 40, None) == 1
    assert L.mra_debug_select(ctypes.byref(d), Q, K, 4, 0, 0, 0, 0, O, W, 16, None) == 10
    assert L.mra_debug_select(ctypes.byref(d), Q, K, 0, 0, 0, 0, 0, O, W, 1 << 40, None) == 7
    assert L.mra_debug_select(ctypes.byref(d), Q, K, 4, -1, 0, 0, 0, O, W, 1 << 40, None) == 8
    assert L.mra_debug_select(ctypes.byref(d), Q, K, 4, 0, 0, 2, 0, O, W, 1 << 40, None) == 6
    assert L.mra_debug_select(ctypes.byref(d), Q, K, 4, 0, 2, 0, 3, O, W, 1 << 40, None) == 8


def test_debug_wait_timeout_rejects_bad_arguments():
    L = mra.lib()
    d = mra._Dims(1, 2, 4096, 64, 1)
    assert L.mra_debug_wait_timeout(None, Q, K, V, 4, 0, 8, W, 1 << 40, None) == 1
    assert L.mra_debug_wait_timeout(ctypes.byref(d), Q, K, V, 4, 0, 8, W, 16, None) == 10
    assert L.mra_debug_wait_timeout(ctypes.byref(d), Q, K, V, 4, 0, 0, W, 1 << 40, None) == 13
    assert L.mra_debug_wait_timeout(ctypes.byref(d), Q, K, V, 4, 0, (1 << 16) + 1, W, 1 << 40, None) == 13
    # only heads of 64 or 128 block rows form logits and select in one launch
    # (and without a device no size does)
    for n in (1024, 8192, 4096):
        d = mra._Dims(1, 2, n, 64, 1)
        assert L.mra_debug_wait_timeout(ctypes.byref(d), Q, K, V, 4, 0, 8, W, 1 << 40, None) == 3


def test_debug_replay_rejects_bad_arguments():
    L = mra.lib()
    d = mra._Dims(1, 2, 512, 64, 1)
    args = lambda stage, count, ws_bytes=1 << 40: (ctypes.byref(d), Q, K, V, None, 4, 0, 0, 0, O, W, ws_bytes,
                                                   stage, count, None)
    for stage in (0, 1, 2, 4, 5, -1):
        assert L.mra_debug_replay(*args(stage, 1)) == 13
    assert L.mra_debug_replay(*args(3, 0)) == 13
    assert L.mra_debug_replay(*args(3, 1, 16)) == 10
    assert L.mra_debug_replay(ctypes.byref(d), Q, K, V, None, 4, 0, 0, 0, None, W, 1 << 40, 3, 1, None) == 1


DO, DQ, DK, DV, BW = 0x70000000, 0x80000000, 0x90000000, 0xA0000000, 0xB0000000


MK = 0x60000000


def call_bwd(dims=(1, 2, 512, 64, 1), mode=1, dout=DO, dq=DQ, dk=DK, dv=DV, bw=BW, bw_bytes=None, out=O,
             ws=W, mask=None):
    d = mra._Dims(*dims)
    ws_bytes = mra.workspace_size(1, 2, 512, approx_mode="full")   # enough for either mode
    if bw_bytes is None:
        bw_bytes = mra.backward_workspace_size(1, 2, 512)
    return mra.lib().mra_attention_bwd(ctypes.byref(d), Q, K, V, mask, 4, mode, 0, 0, out, dout, dq, dk, dv, ws,
                                       ws_bytes, bw, bw_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), 1), (dict(dout=None), 1), (dict(dq=None), 1), (dict(dv=None), 1),
    (dict(mode=2), 6), (dict(mode=-1), 6), (dict(dims=(1, 2, 512, 64, 7)), 5), (dict(ws=None), 10),
    (dict(dims=(1, 2, 512, 96, 1)), 4),
    (dict(bw=None), 10), (dict(bw_bytes=4096), 10),
    (dict(dq=Q), 9), (dict(dk=O + 64), 9), (dict(dv=DQ), 9), (dict(dq=BW), 9), (dict(bw=DO), 9),
    (dict(dq=DQ + 8), 12), (dict(bw=BW + 8), 12),
    # no output of the backward may overlap the mask it reads
    (dict(mask=MK, dq=MK - 1024), 9), (dict(mask=MK, bw=MK - 256), 9), (dict(mask=DV + 64), 9),
])
def test_attention_bwd_rejects_bad_arguments(kw, status):
    assert call_bwd(**kw) == status


def test_backward_workspace_size_grows_and_validates():
    small = mra.backward_workspace_size(1, 2, 512)
    big = mra.backward_workspace_size(2, 12, 4096)
    assert 0 < small < big
    assert mra.backward_workspace_size(2, 12, 4096, block_per_row=8) > big
    assert mra.backward_workspace_size(2, 12, 4096, approx_mode="full") > big   # the low-res terms' buffers
    with pytest.raises(mra.MraError) as e:
        mra.backward_workspace_size(1, 1, 100)
    assert e.value.status == 3
    with pytest.raises(mra.MraError) as e:
        mra.backward_workspace_size(1, 1, 512, block_per_row=0)
    assert e.value.status == 7


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError):
        mra.attention(q, q, q)


def test_bigbird_workspace_and_argument_checks():
    assert mra.bigbird_workspace_size(2, 12, 4096) > 0
    for kw, status in [(dict(seq_len=4000), 3), (dict(block_size=48), 3), (dict(block_size=256), 3),
                       (dict(num_random_blocks=0), 7), (dict(seq_len=100), 3)]:
        args = dict(batch=1, heads=2, seq_len=512, block_size=64, num_random_blocks=3)
        args.update(kw)
        with pytest.raises(mra.MraError) as e:
            mra.bigbird_workspace_size(args["batch"], args["heads"], args["seq_len"], block_size=args["block_size"],
                                       num_random_blocks=args["num_random_blocks"])
        assert e.value.status == status, kw
    L = mra.lib()
    d = mra._Dims(1, 2, 512, 64, 1)
    RB = 0xC0000000
    ws = mra.bigbird_workspace_size(1, 2, 512)
    call = lambda **kw: L.mra_bigbird_fwd(ctypes.byref(d), kw.get("q", Q), K, V, None, kw.get("bs", 64),
                                          kw.get("r", 3), kw.get("rand", RB), kw.get("out", O), W,
                                          kw.get("ws_bytes", ws), None)
    assert call(rand=None) == 1
    assert call(q=None) == 1
    assert call(rand=RB + 2) == 12
    assert call(rand=O) == 9
    assert call(out=Q) == 9
    assert call(ws_bytes=64) == 10
    assert call(r=0) == 7
    assert call(bs=96) == 3
    assert L.mra_bigbird_fwd(None, Q, K, V, None, 64, 3, RB, O, W, ws, None) == 1


def test_bigbird_backward_checks():
    assert mra.bigbird_backward_workspace_size(2, 12, 4096) > 0
    with pytest.raises(mra.MraError) as e:
        mra.bigbird_backward_workspace_size(1, 2, 512, num_random_blocks=0)
    assert e.value.status == 7
    L = mra.lib()
    d = mra._Dims(1, 2, 512, 64, 1)
    ws = mra.bigbird_workspace_size(1, 2, 512)
    bw = mra.bigbird_backward_workspace_size(1, 2, 512)
    DO2, DQ2, DK2, DV2, BW2 = 0x70000000, 0x80000000, 0x90000000, 0xA0000000, 0xB0000000
    call = lambda **kw: L.mra_bigbird_bwd(ctypes.byref(d), Q, K, V, None, kw.get("bs", 64), kw.get("r", 3), O,
                                          kw.get("dout", DO2), kw.get("dq", DQ2), DK2, DV2, W, ws,
                                          kw.get("bw", BW2), kw.get("bw_bytes", bw), None)
    assert call(dout=None) == 1
    assert call(bw=None) == 10
    assert call(bw_bytes=256) == 10
    assert call(dq=Q) == 9
    assert call(r=0) == 7
    assert call(bs=96) == 3
    dbad = mra._Dims(1, 2, 512, 64, 7)
    assert L.mra_bigbird_bwd(ctypes.byref(dbad), Q, K, V, None, 64, 3, O, DO2, DQ2, DK2, DV2, W, 1 << 30, BW2,
                             1 << 30, None) == 5


def test_scale_dim_checks():
    for sd, status in [(-1, 4), (65, 4)]:
        d = mra._Dims(1, 2, 512, 64, 1, sd)
        assert mra.lib().mra_attention_fwd(ctypes.byref(d), Q, K, V, None, 4, 0, 0, 0, O, W, 1 << 40, None) == status
    d = mra._Dims(1, 2, 512, 64, 1, 32)
    assert mra.lib().mra_attention_fwd(ctypes.byref(d), Q, K, V, None, 4, 0, 0, 0, None, W, 1 << 40, None) == 1


def test_workspace_error_checks_arguments():
    # host-side checks only: none of these reaches the HIP runtime
    L = mra.lib()
    word = ctypes.c_uint32(7)
    assert L.mra_workspace_error(None, 1 << 20, None, ctypes.byref(word)) == 1
    assert L.mra_workspace_error(W, 1 << 20, None, None) == 1
    assert L.mra_workspace_error(W, 128, None, ctypes.byref(word)) == 10
    assert word.value == 7


def test_device_error_bits_are_named():
    # every bit the header documents has a name in the binding
    text = open(HEADER).read()
    bits = {int(v) for v in re.findall(r"MRA_DEVERR_[A-Z_]+ = (\d+)", text)}
    assert bits == set(mra.DEVICE_ERRORS) == {1, 2, 4, 8, 16, 32}


def test_head_count_cap():
    # batch * heads up to 2^20 pass the host checks (the kernels index the
    # per-head histograms, BH * 4096 words, in 64 bits); more is rejected
    n = ctypes.c_size_t(0)
    d = mra._Dims(1 << 10, 1 << 10, 32, 64, 1)
    assert mra.lib().mra_workspace_size(ctypes.byref(d), 1, 0, ctypes.byref(n)) == 0
    assert n.value > (1 << 20) * 4096 * 4
    d = mra._Dims(1 << 10, (1 << 10) + 1, 32, 64, 1)
    assert mra.lib().mra_workspace_size(ctypes.byref(d), 1, 0, ctypes.byref(n)) == 2
