"""CPU oracle for the MRA-2 forward pass (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does: it shares
no code with the oracle and fails loudly when its own HIP library is missing.

The arithmetic lives in ``mra_oracle.c`` (plain C, fp64 values, fp32
canonical selection); each function there cites the passage of the page
"A deep dive into the MRA model in Transformers" it follows.  This module only
compiles that file with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mra_oracle.c")
_LIB = os.path.join(_HERE, "libmra_oracle.so")
# A test that plants mistakes in copies of the oracle points this at a
# mutated build; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("MRA_ORACLE_LIB")
# -ffp-contract=off and no fast-math: the fp32 steps must be exactly the
# operations written in the C source.
CFLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-pthread"]

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            build()
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_num_block.argtypes = [i32, i32]
        L.oracle_num_block.restype = i64
        L.oracle_pool_f32.argtypes = [i32, i32, P, P, P, P]
        L.oracle_pool_f32.restype = None
        L.oracle_pool_f64.argtypes = [i32, i32, P, P, P]
        L.oracle_pool_f64.restype = None
        L.oracle_lowres_logits_f32.argtypes = [i32, i32, P, P, P]
        L.oracle_lowres_logits_f32.restype = None
        L.oracle_scores_f32.argtypes = [i32, P, P, i32, i32, i32, P, P]
        L.oracle_scores_f32.restype = None
        L.oracle_select_top.argtypes = [i32, P, i64, P]
        L.oracle_select_top.restype = ctypes.c_int
        L.oracle_select_from_logits.argtypes = [i32, P, P, i64, i32, i32, i32, P]
        L.oracle_select_from_logits.restype = ctypes.c_int
        L.oracle_mra_fwd.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, i32, i32, i32, i32,
                                     P, P, i32]
        L.oracle_mra_fwd.restype = ctypes.c_int
        L.oracle_dense_fwd.argtypes = [i32, i32, i32, i32, P, P, P, P, P, i32]
        L.oracle_dense_fwd.restype = ctypes.c_int
        L.oracle_mra_bwd.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, i32, i32, i32, i32, P, P, P, P, i32]
        L.oracle_mra_bwd.restype = ctypes.c_int
        L.oracle_bigbird_fwd.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, i32, P, P, i32]
        L.oracle_bigbird_fwd.restype = ctypes.c_int
        L.oracle_bigbird_bwd.argtypes = [i32, i32, i32, i32, P, P, P, P, i32, i32, P, P, P, P, P, i32]
        L.oracle_bigbird_bwd.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _mask(m):
    return None if m is None else np.ascontiguousarray(m, dtype=np.uint8)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


MODES = {"full": 0, "sparse": 1}
# how step 2 ranks the cells: "row_normalized" S_ij - rowmax_i (reading R2,
# the default) or "raw_logits" S_ij (reading R2')
RANKINGS = {"row_normalized": 0, "raw_logits": 1}
# width of the diagonal prior band for even n: |i - j| <= n // 2 ("symmetric", n + 1 wide)
# or exactly n wide, offsets -((n - 1) // 2) .. n // 2 ("exact")
BANDS = {"symmetric": 0, "exact": 2}


def _variant(ranking, band):
    return RANKINGS[ranking] | BANDS[band]



def num_block(seq_len: int, block_per_row: int) -> int:
    return int(lib().oracle_num_block(seq_len, block_per_row))


def pool_f32(x, mask=None):
    """x: [N, d] one head -> (xhat [nb, d] fp32, cnt [nb] int32)."""
    x = _f32(x)
    N, d = x.shape
    xh = np.zeros((N // 32, d), np.float32)
    cnt = np.zeros(N // 32, np.int32)
    m = _mask(mask)
    lib().oracle_pool_f32(N, d, _p(x), _p(m), _p(xh), _p(cnt))
    return xh, cnt


def pool_f64(x, mask=None):
    x = _f32(x)
    N, d = x.shape
    xh = np.zeros((N // 32, d), np.float64)
    m = _mask(mask)
    lib().oracle_pool_f64(N, d, _p(x), _p(m), _p(xh))
    return xh


def lowres_logits_f32(qhat, khat):
    qhat, khat = _f32(qhat), _f32(khat)
    nb, d = qhat.shape
    S = np.zeros((nb, nb), np.float32)
    lib().oracle_lowres_logits_f32(nb, d, _p(qhat), _p(khat), _p(S))
    return S


def scores_f32(S, cnt, prior_first=0, prior_diag=0, ranking="row_normalized", band="symmetric"):
    S = _f32(S)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    nb = S.shape[0]
    rowmax = np.zeros(nb, np.float32)
    score = np.zeros((nb, nb), np.float32)
    lib().oracle_scores_f32(nb, _p(S), _p(cnt), prior_first, prior_diag, _variant(ranking, band), _p(rowmax),
                            _p(score))
    return rowmax, score


def select_top(score, K):
    score = _f32(score)
    nb = score.shape[0]
    sel = np.zeros(max(K, 1), np.int32)
    rc = lib().oracle_select_top(nb, _p(score), K, _p(sel))
    if rc:
        raise ValueError("oracle_select_top failed: %d" % rc)
    return sel[:K]


def select_from_logits(S, cnt, K, prior_first=0, prior_diag=0, ranking="row_normalized", band="symmetric"):
    S = _f32(S)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    nb = S.shape[0]
    sel = np.zeros(max(K, 1), np.int32)
    rc = lib().oracle_select_from_logits(nb, _p(S), _p(cnt), K, prior_first, prior_diag,
                                         _variant(ranking, band), _p(sel))
    if rc:
        raise ValueError("oracle_select_from_logits failed: %d" % rc)
    return sel[:K]


def mra_forward(q, k, v, mask=None, block_per_row=4, approx_mode="full",
                prior_first=0, prior_diag=0, threads=None, return_selection=False, ranking="row_normalized",
                band="symmetric"):
    """q, k, v: [B, H, N, d] (fp32 values; bf16 inputs widened exactly).
    mask: [B, N] or None.  Returns out [B, H, N, d] fp64 (and sel [B, H, K])."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    K = num_block(N, block_per_row)
    if K < 0:
        raise ValueError("invalid sequence length / block_per_row")
    out = np.zeros((B, H, N, d), np.float64)
    sel = np.zeros((B, H, max(K, 1)), np.int32) if return_selection else None
    m = _mask(mask)
    rc = lib().oracle_mra_fwd(B, H, N, d, _p(q), _p(k), _p(v), _p(m), block_per_row,
                              MODES[approx_mode], prior_first, prior_diag, _variant(ranking, band), _p(out), _p(sel),
                              threads or default_threads())
    if rc:
        raise ValueError("oracle_mra_fwd failed: %d" % rc)
    if return_selection:
        return out, sel[:, :, :K]
    return out


def mra_backward(q, k, v, dout, mask=None, block_per_row=4, approx_mode="full",
                 prior_first=0, prior_diag=0, threads=None, ranking="row_normalized", band="symmetric"):
    """Gradients of mra_forward's output with respect to q, k, v given
    dout = dL/d out, with the selection held fixed ([MRA] step 3: the block
    products' backward reuses the kernels on transposed indices).  All
    [B, H, N, d]; returns (dq, dk, dv) fp64."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, N, d = q.shape
    if num_block(N, block_per_row) < 0:
        raise ValueError("invalid sequence length / block_per_row")
    dq = np.zeros((B, H, N, d), np.float64)
    dk = np.zeros_like(dq)
    dv = np.zeros_like(dq)
    m = _mask(mask)
    rc = lib().oracle_mra_bwd(B, H, N, d, _p(q), _p(k), _p(v), _p(m), block_per_row, MODES[approx_mode],
                              prior_first, prior_diag, _variant(ranking, band), _p(g), _p(dq), _p(dk), _p(dv),
                              threads or default_threads())
    if rc:
        raise ValueError("oracle_mra_bwd failed: %d" % rc)
    return dq, dk, dv


def dense_forward(q, k, v, mask=None, threads=None):
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    out = np.zeros((B, H, N, d), np.float64)
    m = _mask(mask)
    rc = lib().oracle_dense_fwd(B, H, N, d, _p(q), _p(k), _p(v), _p(m), _p(out),
                                threads or default_threads())
    if rc:
        raise ValueError("oracle_dense_fwd failed: %d" % rc)
    return out


def bigbird_forward(q, k, v, rand, mask=None, block_size=64, threads=None):
    """BigBird block-sparse attention ([BigBird]: 3-block window, the first
    and last blocks global, r random key blocks per query block given in
    rand [B, H, N / block_size, r]).  q, k, v: [B, H, N, d]; returns fp64."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, H, N, d = q.shape
    rand = np.ascontiguousarray(rand, dtype=np.int32)
    if rand.ndim != 4 or rand.shape[:3] != (B, H, N // block_size):
        raise ValueError("rand must be [B, H, N / block_size, r]")
    out = np.zeros((B, H, N, d), np.float64)
    rc = lib().oracle_bigbird_fwd(B, H, N, d, _p(q), _p(k), _p(v), _p(_mask(mask)), block_size, rand.shape[3],
                                  _p(rand), _p(out), threads or default_threads())
    if rc:
        raise ValueError("oracle_bigbird_fwd failed: %d" % rc)
    return out


def bigbird_backward(q, k, v, rand, dout, mask=None, block_size=64, threads=None):
    """Gradients of bigbird_forward's output with respect to q, k, v given
    dout = dL/d out (the pattern is a constant).  Returns (dq, dk, dv) fp64."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, H, N, d = q.shape
    rand = np.ascontiguousarray(rand, dtype=np.int32)
    if rand.ndim != 4 or rand.shape[:3] != (B, H, N // block_size):
        raise ValueError("rand must be [B, H, N / block_size, r]")
    dq, dk, dv = (np.zeros((B, H, N, d), np.float64) for _ in range(3))
    rc = lib().oracle_bigbird_bwd(B, H, N, d, _p(q), _p(k), _p(v), _p(_mask(mask)), block_size, rand.shape[3],
                                  _p(rand), _p(g), _p(dq), _p(dk), _p(dv), threads or default_threads())
    if rc:
        raise ValueError("oracle_bigbird_bwd failed: %d" % rc)
    return dq, dk, dv
