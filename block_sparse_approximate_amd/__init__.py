"""MI355X-native MRA-2 multi-resolution approximate self-attention (forward).

A thin binding over ``libmra.so`` (hand-written HIP kernels for gfx950 behind
the C ABI in ``include/mra.h``).  This module only marshals arguments: torch
supplies device memory and the current HIP stream; every step of the method
runs in the library's kernels.  There is no CPU or PyTorch fallback: if the
library is missing, importing the binding's entry points raises.

Method: the page "A deep dive into the MRA model in Transformers"
(深入解析 Transformers 中的 MRA 模型), steps 1-4 and the MraConfig section,
whose parameter names the keyword arguments below keep.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["attention", "attention_profiled", "prepare", "num_block", "workspace_size", "debug_stages", "debug_select",
           "debug_replay", "attention_backward", "workspace_error", "MraDeviceError",
           "MraError", "library_path", "lib"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmra.so")
_lib = None

MODES = {"full": 0, "sparse": 1}
# step 2's ranking: the row-max-normalised logits (default) or the raw logits
RANKINGS = {"row_normalized": 0, "raw_logits": 1}
# width of the diagonal prior band for even n: |i - j| <= n // 2 ("symmetric")
# or exactly n blocks, offsets -((n - 1) // 2) .. n // 2 ("exact")
BANDS = {"symmetric": 0, "exact": 1}
# bits of a workspace's device error word (include/mra.h MRA_DEVERR_*)
DEVICE_ERRORS = {1: "selector candidate list", 2: "selection or segment count", 4: "attention record window",
                 8: "backward plan", 16: "forward kept no softmax statistics",
                 32: "selector wait for the head's logits"}
# When set (environment MRA_CHECK_DEVICE_ERRORS=1, or assigned), every forward
# and backward call waits for its stream and raises MraDeviceError if a
# kernel flagged an inconsistency.  Off by default: the check synchronises.
CHECK_DEVICE_ERRORS = os.environ.get("MRA_CHECK_DEVICE_ERRORS", "0") == "1"
DTYPES = {torch.float32: 0, torch.bfloat16: 1}

# Entry points declared in include/mra.h, with their ctypes signatures.
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "mra_abi_version": ([], _I32),
    "mra_status_string": ([_I32], ctypes.c_char_p),
    "mra_num_block": ([_I32, _I32], _I64),
    "mra_workspace_size": ([_P, _I32, _I32, ctypes.POINTER(_SZ)], ctypes.c_int),
    "mra_attention_fwd": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P], ctypes.c_int),
    "mra_attention_fwd_profiled": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P, _P],
                                   ctypes.c_int),
    "mra_attention_fwd_ex": ([_P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "mra_debug_stages": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P,
                          _P, _P, _SZ, _P], ctypes.c_int),
    "mra_debug_select": ([_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _P, _SZ, _P], ctypes.c_int),
    "mra_debug_wait_timeout": ([_P, _P, _P, _P, _I32, _I32, ctypes.c_uint32, _P, _SZ, _P], ctypes.c_int),
    "mra_workspace_error": ([_P, _SZ, _P, ctypes.POINTER(ctypes.c_uint32)], ctypes.c_int),
    "mra_attention_fwd_noalloc": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P], ctypes.c_int),
    "mra_bigbird_workspace_size": ([_P, _I32, _I32, ctypes.POINTER(_SZ)], ctypes.c_int),
    "mra_bigbird_fwd": ([_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _SZ, _P], ctypes.c_int),
    "mra_bigbird_backward_workspace_size": ([_P, _I32, _I32, ctypes.POINTER(_SZ)], ctypes.c_int),
    "mra_bigbird_bwd": ([_P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _P], ctypes.c_int),
    "mra_backward_workspace_size": ([_P, _I32, _I32, ctypes.POINTER(_SZ)], ctypes.c_int),
    "mra_attention_bwd": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ,
                           _P], ctypes.c_int),
    "mra_debug_replay": ([_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _SZ, _I32, _I32, _P], ctypes.c_int),
}


class MraError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: status %d (%s)" % (what, status, _status_text(status)))
        self.status = status


class MraDeviceError(RuntimeError):
    """A kernel flagged an inconsistency in its bookkeeping: the call's
    outputs are undefined.  `word` holds the device error word's bits."""

    def __init__(self, word: int, what: str):
        names = [n for b, n in DEVICE_ERRORS.items() if word & b]
        super().__init__("%s: device error word 0x%x (%s)" % (what, word, ", ".join(names) or "?"))
        self.word = word


class _Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale_dim", ctypes.c_int32)]


class _Options(ctypes.Structure):
    _fields_ = [("block_per_row", ctypes.c_int32), ("approx_mode", ctypes.c_int32),
                ("prior_first", ctypes.c_int32), ("prior_diag", ctypes.c_int32),
                ("score_ranking", ctypes.c_int32), ("diag_band", ctypes.c_int32),
                ("save_stats", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmra.so; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libmra.so is not built (run `python -m block_sparse_approximate_amd.build`"
                              " or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _status_text(status: int) -> str:
    try:
        return lib().mra_status_string(status).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise MraError(status, what)


def workspace_error(workspace: torch.Tensor) -> int:
    """The device error word of a forward call's workspace (and of the
    backward passes that read it), after the current stream has finished its
    queued work; 0 when every kernel's bookkeeping added up."""
    word = ctypes.c_uint32(0)
    _check(lib().mra_workspace_error(_ptr(workspace), workspace.numel(), _stream(workspace), ctypes.byref(word)),
           "mra_workspace_error")
    return int(word.value)


def _check_device(workspace: torch.Tensor, what: str):
    if CHECK_DEVICE_ERRORS:
        word = workspace_error(workspace)
        if word:
            raise MraDeviceError(word, what)


def num_block(seq_len: int, block_per_row: int) -> int:
    return int(lib().mra_num_block(seq_len, block_per_row))


def _dims(B, H, N, d, dtype_code, scale_dim=0) -> _Dims:
    return _Dims(B, H, N, d, dtype_code, scale_dim)


def workspace_size(batch, heads, seq_len, head_dim=64, dtype=torch.bfloat16, block_per_row=4,
                   approx_mode="full") -> int:
    n = _SZ(0)
    dims = _dims(batch, heads, seq_len, head_dim, DTYPES.get(dtype, -1))
    _check(lib().mra_workspace_size(ctypes.byref(dims), block_per_row, MODES.get(approx_mode, -1),
                                    ctypes.byref(n)), "mra_workspace_size")
    return n.value


def backward_workspace_size(batch, heads, seq_len, head_dim=64, dtype=torch.bfloat16, block_per_row=4,
                            approx_mode="sparse") -> int:
    n = _SZ(0)
    dims = _dims(batch, heads, seq_len, head_dim, DTYPES.get(dtype, -1))
    _check(lib().mra_backward_workspace_size(ctypes.byref(dims), block_per_row, MODES.get(approx_mode, -1),
                                             ctypes.byref(n)), "mra_backward_workspace_size")
    return n.value


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_inputs(q, k, v, mask):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if t.dim() != 4 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous [batch, heads, seq_len, head_dim] tensor" % name)
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if q.dtype not in DTYPES:
        raise ValueError("dtype must be float32 or bfloat16")
    if mask is not None:
        if mask.dtype == torch.bool:
            raise ValueError("pass the mask as uint8 (1 = valid token)")
        if (mask.dtype != torch.uint8 or mask.shape != (q.shape[0], q.shape[2]) or not mask.is_contiguous()
                or mask.device != q.device):
            raise ValueError("mask must be a contiguous uint8 [batch, seq_len] tensor on q's device")


def attention(q, k, v, mask=None, block_per_row=4, approx_mode="full", initial_prior_first_n_blocks=0,
              initial_prior_diagonal_n_blocks=0, out=None, workspace=None, score_ranking="row_normalized", scale_dim=0,
              diag_band="symmetric", save_stats=False):
    """MRA-2 forward on [batch, heads, seq_len, head_dim] tensors (bf16 or fp32).
    mask: uint8 [batch, seq_len] (1 = valid) or None.  score_ranking:
    "row_normalized" (default) or "raw_logits", what step 2's top-k ranks.
    diag_band: "symmetric" (default, |i - j| <= n // 2) or "exact" (a band of
    exactly n blocks).  save_stats: keep each token's softmax statistics in
    the workspace for attention_backward.  Returns `out`."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    if score_ranking == "row_normalized" and diag_band == "symmetric" and not save_stats:
        st = lib().mra_attention_fwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row,
                                     MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                                     initial_prior_diagonal_n_blocks, _ptr(out), _ptr(workspace),
                                     workspace.numel(), _stream(q))
        _check(st, "mra_attention_fwd")
    else:
        opts = _Options(block_per_row, MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                        initial_prior_diagonal_n_blocks, RANKINGS.get(score_ranking, -1), BANDS.get(diag_band, -1),
                        1 if save_stats else 0)
        st = lib().mra_attention_fwd_ex(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                                        ctypes.byref(opts), _ptr(out), _ptr(workspace), workspace.numel(), _stream(q))
        _check(st, "mra_attention_fwd_ex")
    _check_device(workspace, "mra_attention_fwd")
    return out


def attention_noalloc(q, k, v, mask=None, block_per_row=4, approx_mode="full", initial_prior_first_n_blocks=0,
                      initial_prior_diagonal_n_blocks=0, out=None, scale_dim=0):
    """attention() through mra_attention_fwd_noalloc: the library's own fixed
    device scratch (64 MiB per GPU) serves as the workspace, so the library
    allocates nothing; calls on one GPU must not overlap.  Returns `out`."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    st = lib().mra_attention_fwd_noalloc(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row,
                                         MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                                         initial_prior_diagonal_n_blocks, _ptr(out), _stream(q))
    _check(st, "mra_attention_fwd_noalloc")
    return out


def prepare(q, k, v, mask=None, block_per_row=4, approx_mode="full", initial_prior_first_n_blocks=0,
            initial_prior_diagonal_n_blocks=0, out=None, workspace=None, scale_dim=0):
    """Check and marshal the arguments once; returns (call, out) where call()
    queues one forward pass on the current stream through the C ABI.  The
    tensors must stay alive and unchanged in shape while call is used."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    fn = lib().mra_attention_fwd
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row, MODES.get(approx_mode, -1),
            initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks, _ptr(out), _ptr(workspace),
            workspace.numel(), _stream(q))
    keep = (dims, q, k, v, mask, out, workspace)

    def call():
        st = fn(*args)
        if st != 0:
            raise MraError(st, "mra_attention_fwd")
        _check_device(workspace, "mra_attention_fwd")
        return keep[5]

    return call, out


STAGES = ("pool", "logits", "select", "attn")


def attention_profiled(q, k, v, events, mask=None, block_per_row=4, approx_mode="full",
                       initial_prior_first_n_blocks=0, initial_prior_diagonal_n_blocks=0, out=None,
                       workspace=None, scale_dim=0):
    """attention() plus HIP event records around each kernel launch.
    events: 8 torch.cuda.Event(enable_timing=True) (already recorded once, so
    that their handles exist), entry 2s / 2s+1 bracketing stage STAGES[s]."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
    ws_bytes = workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    arr = (ctypes.c_void_p * 8)(*[e.cuda_event if e is not None else None for e in events])
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    st = lib().mra_attention_fwd_profiled(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask),
                                          block_per_row, MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                                          initial_prior_diagonal_n_blocks, _ptr(out), _ptr(workspace),
                                          workspace.numel(), _stream(q), arr)
    _check(st, "mra_attention_fwd_profiled")
    return out


def prepare_backward(q, k, v, out, dout, workspace, mask=None, block_per_row=4, approx_mode="sparse",
                     initial_prior_first_n_blocks=0, initial_prior_diagonal_n_blocks=0, dq=None, dk=None, dv=None,
                     bwd_workspace=None, scale_dim=0):
    """Check and marshal the arguments of attention_backward once; returns
    (call, (dq, dk, dv)) where call() queues one backward pass on the current
    stream through the C ABI.  `out` and `workspace` are a forward call's
    output and workspace (the selection and softmax statistics are read from
    it); the other arguments must be the ones it was made with.
    `bwd_workspace` (uint8, backward_workspace_size bytes) is allocated when
    not given.  Both modes, bf16 or fp32."""
    _check_inputs(q, k, v, mask)
    for t in (out, dout):
        if not (t.is_cuda and t.dtype == q.dtype and t.shape == q.shape and t.is_contiguous()):
            raise ValueError("out and dout must be contiguous device tensors shaped and typed like q")
    B, H, N, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if not (t.is_cuda and t.dtype == q.dtype and t.shape == q.shape and t.is_contiguous()):
            raise ValueError("dq, dk and dv must be contiguous device tensors shaped and typed like q")
    bw_bytes = backward_workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    if bwd_workspace is None or bwd_workspace.numel() < bw_bytes:
        bwd_workspace = torch.empty(bw_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    fn = lib().mra_attention_bwd
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row, MODES.get(approx_mode, -1),
            initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks, _ptr(out), _ptr(dout), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), _ptr(bwd_workspace), bwd_workspace.numel(),
            _stream(q))
    keep = (dims, q, k, v, mask, out, dout, dq, dk, dv, workspace, bwd_workspace)

    def call():
        st = fn(*args)
        if st != 0:
            raise MraError(st, "mra_attention_bwd")
        _check_device(workspace, "mra_attention_bwd")
        return keep[7:10]

    return call, (dq, dk, dv)


def attention_backward(q, k, v, out, dout, workspace, mask=None, block_per_row=4, approx_mode="sparse",
                       initial_prior_first_n_blocks=0, initial_prior_diagonal_n_blocks=0, dq=None, dk=None,
                       dv=None, bwd_workspace=None, scale_dim=0):
    """Gradients (dq, dk, dv) of a forward call's output with respect to q, k,
    v given dout; arguments as for prepare_backward."""
    call, grads = prepare_backward(q, k, v, out, dout, workspace, mask, block_per_row, approx_mode,
                                   initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks, dq, dk, dv,
                                   bwd_workspace, scale_dim)
    call()
    return grads


def debug_replay(q, k, v, stage, count, mask=None, block_per_row=4, approx_mode="full",
                 initial_prior_first_n_blocks=0, initial_prior_diagonal_n_blocks=0, out=None, workspace=None, scale_dim=0):
    """Relaunch stage STAGES[stage] (3 attn only) `count` times on
    the current stream, on a workspace and out that a forward call with the
    same arguments has filled; for timing the kernel alone."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    st = lib().mra_debug_replay(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row,
                                MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                                initial_prior_diagonal_n_blocks, _ptr(out), _ptr(workspace),
                                0 if workspace is None else workspace.numel(), stage, count, _stream(q))
    _check(st, "mra_debug_replay")
    return out


def debug_stages(q, k, v, mask=None, block_per_row=4, approx_mode="full", initial_prior_first_n_blocks=0,
                 initial_prior_diagonal_n_blocks=0, score_ranking="row_normalized", scale_dim=0,
                 diag_band="symmetric"):
    """Steps 1-2 of the same kernels; returns a dict of device tensors:
    qhat, khat, vhat (full mode), count, logits, rowmax, sel, error."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    nb = N // 32
    K = num_block(N, block_per_row)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    r = {
        "qhat": torch.empty(B, H, nb, d, **f32),
        "khat": torch.empty(B, H, nb, d, **f32),
        "vhat": torch.empty(B, H, nb, d, **f32) if approx_mode == "full" else None,
        "count": torch.empty(B, nb, dtype=torch.int32, device=dev),
        "logits": torch.empty(B, H, nb, nb, **f32),
        "rowmax": torch.empty(B, H, nb, **f32),
        "sel": torch.empty(B, H, max(K, 1), dtype=torch.int32, device=dev),
        "error": torch.zeros(1, dtype=torch.int32, device=dev),
    }
    ws_bytes = workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    st = lib().mra_debug_stages(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_per_row,
                                MODES.get(approx_mode, -1), initial_prior_first_n_blocks,
                                initial_prior_diagonal_n_blocks, RANKINGS.get(score_ranking, -1),
                                BANDS.get(diag_band, -1), _ptr(r["qhat"]), _ptr(r["khat"]),
                                _ptr(r["vhat"]), _ptr(r["count"]), _ptr(r["logits"]), _ptr(r["rowmax"]),
                                _ptr(r["sel"]), _ptr(r["error"]), _ptr(ws), ws_bytes, _stream(q))
    _check(st, "mra_debug_stages")
    r["sel"] = r["sel"][:, :, :K]
    return r


def debug_select(logits, count, batch, heads, block_per_row=4, initial_prior_first_n_blocks=0,
                 initial_prior_diagonal_n_blocks=0, score_ranking="row_normalized", diag_band="symmetric"):
    """The step-2 selector alone on given fp32 logits [B, H, nb, nb] and
    int32 counts [B, nb] (device tensors).  Returns sel [B, H, K] int32."""
    nb = logits.shape[-1]
    N = 32 * nb
    K = num_block(N, block_per_row)
    if logits.dtype != torch.float32 or not logits.is_contiguous() or logits.shape != (batch, heads, nb, nb):
        raise ValueError("logits must be contiguous fp32 [B, H, nb, nb]")
    if count.dtype != torch.int32 or not count.is_contiguous() or count.shape != (batch, nb):
        raise ValueError("count must be contiguous int32 [B, nb]")
    sel = torch.empty(batch, heads, max(K, 1), dtype=torch.int32, device=logits.device)
    ws_bytes = workspace_size(batch, heads, N, 64, torch.bfloat16, block_per_row, "sparse")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=logits.device)
    dims = _dims(batch, heads, N, 64, 1)
    st = lib().mra_debug_select(ctypes.byref(dims), _ptr(logits), _ptr(count), block_per_row,
                                initial_prior_first_n_blocks, initial_prior_diagonal_n_blocks,
                                RANKINGS.get(score_ranking, -1), BANDS.get(diag_band, -1), _ptr(sel), _ptr(ws),
                                ws_bytes, _stream(logits))
    _check(st, "mra_debug_select")
    return sel[:, :, :K]


def debug_wait_timeout(q, k, v, polls=16, block_per_row=4, approx_mode="full"):
    """Pooling and the logits-and-selection launch (seq_len 2048 or 4096)
    with every workgroup's wait for its head made to run out after `polls`
    polls; returns the workspace's device error word (MRA_DEVERR_WAIT is
    expected).  A test of the error path: the selection is not meant for use."""
    _check_inputs(q, k, v, None)
    B, H, N, d = q.shape
    ws_bytes = workspace_size(B, H, N, d, q.dtype, block_per_row, approx_mode)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], 0)
    _check(lib().mra_debug_wait_timeout(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), block_per_row,
                                        MODES.get(approx_mode, -1), polls, _ptr(ws), ws_bytes, _stream(q)),
           "mra_debug_wait_timeout")
    return workspace_error(ws)


def bigbird_workspace_size(batch, heads, seq_len, head_dim=64, dtype=torch.bfloat16, block_size=64,
                           num_random_blocks=3) -> int:
    n = _SZ(0)
    dims = _dims(batch, heads, seq_len, head_dim, DTYPES.get(dtype, -1))
    _check(lib().mra_bigbird_workspace_size(ctypes.byref(dims), block_size, num_random_blocks, ctypes.byref(n)),
           "mra_bigbird_workspace_size")
    return n.value


def prepare_bigbird(q, k, v, rand_blocks, mask=None, block_size=64, out=None, workspace=None, scale_dim=0):
    """Check and marshal BigBird block-sparse attention once (mra_bigbird_fwd);
    rand_blocks: int32 device tensor [B, H, seq_len / block_size, r] of the
    random key blocks drawn per query block.  Returns (call, out)."""
    _check_inputs(q, k, v, mask)
    B, H, N, d = q.shape
    if (not rand_blocks.is_cuda or rand_blocks.dtype != torch.int32 or rand_blocks.dim() != 4
            or not rand_blocks.is_contiguous() or tuple(rand_blocks.shape[:3]) != (B, H, N // block_size)):
        raise ValueError("rand_blocks must be a contiguous int32 device tensor [B, H, seq_len / block_size, r]")
    r = rand_blocks.shape[3]
    out = torch.empty_like(q) if out is None else out
    ws_bytes = bigbird_workspace_size(B, H, N, d, q.dtype, block_size, r)
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    fn = lib().mra_bigbird_fwd
    args = (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_size, r, _ptr(rand_blocks), _ptr(out),
            _ptr(workspace), workspace.numel(), _stream(q))
    keep = (dims, q, k, v, mask, rand_blocks, out, workspace)

    def call():
        st = fn(*args)
        if st != 0:
            raise MraError(st, "mra_bigbird_fwd")
        _check_device(workspace, "mra_bigbird_fwd")
        return keep[6]

    return call, out


def bigbird_attention(q, k, v, rand_blocks, mask=None, block_size=64, out=None, workspace=None, scale_dim=0):
    """BigBird block-sparse attention ([BigBird] pattern: window of three
    blocks, first and last blocks global, the given random blocks) on
    [batch, heads, seq_len, 64] tensors.  Returns `out`."""
    call, out = prepare_bigbird(q, k, v, rand_blocks, mask, block_size, out, workspace, scale_dim)
    call()
    return out


def bigbird_backward_workspace_size(batch, heads, seq_len, head_dim=64, dtype=torch.bfloat16, block_size=64,
                                    num_random_blocks=3) -> int:
    n = _SZ(0)
    dims = _dims(batch, heads, seq_len, head_dim, DTYPES.get(dtype, -1))
    _check(lib().mra_bigbird_backward_workspace_size(ctypes.byref(dims), block_size, num_random_blocks,
                                                     ctypes.byref(n)), "mra_bigbird_backward_workspace_size")
    return n.value


def bigbird_backward(q, k, v, out, dout, workspace, num_random_blocks, mask=None, block_size=64, dq=None,
                     dk=None, dv=None, bwd_workspace=None, scale_dim=0):
    """Gradients (dq, dk, dv) of a bigbird_attention call's output given
    dout; `out` and `workspace` are that call's (its layout is read from the
    workspace).  bf16 or fp32."""
    _check_inputs(q, k, v, mask)
    for t in (out, dout):
        if not (t.is_cuda and t.dtype == q.dtype and t.shape == q.shape and t.is_contiguous()):
            raise ValueError("out and dout must be contiguous device tensors shaped and typed like q")
    B, H, N, d = q.shape
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    bw_bytes = bigbird_backward_workspace_size(B, H, N, d, q.dtype, block_size, num_random_blocks)
    if bwd_workspace is None or bwd_workspace.numel() < bw_bytes:
        bwd_workspace = torch.empty(bw_bytes, dtype=torch.uint8, device=q.device)
    dims = _dims(B, H, N, d, DTYPES[q.dtype], scale_dim)
    st = lib().mra_bigbird_bwd(ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(mask), block_size,
                               num_random_blocks, _ptr(out), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                               _ptr(workspace), workspace.numel(), _ptr(bwd_workspace), bwd_workspace.numel(),
                               _stream(q))
    _check(st, "mra_bigbird_bwd")
    _check_device(workspace, "mra_bigbird_bwd")
    return dq, dk, dv
