"""Seeded synthetic inputs for the MRA-2 forward pass.

This module only draws inputs; it holds none of the method's arithmetic, so
both the HIP path's tests and the CPU oracle may take their inputs from it.

Recipe (numpy ``default_rng(seed)``, PCG64):
  * Q, K, V are drawn in that order as ``standard_normal((B, H, N, d),
    float32) * scale``;
  * bf16 workloads are rounded on the host to bf16 with round-to-nearest-even;
    the same bits go to the GPU and, widened exactly to fp32, to the oracle;
  * masks are ``uint8 [B, N]`` (1 = valid token) or ``None``.

The five named workloads are the ones the method is measured on: a small fp32
case, the MRA-base layer shape with padded sequences, a long sparse-mode case
with first-n and diagonal priors (BigBird-like), a clustered long case and a
very long case.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even.
    Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str                 # "f32" or "bf16"
    block_per_row: int
    approx_mode: str           # "full" or "sparse"
    prior_first: int = 0
    prior_diag: int = 0
    q: np.ndarray = field(repr=False, default=None)   # fp32 values [B,H,N,d]
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    mask: np.ndarray | None = field(repr=False, default=None)  # uint8 [B,N]

    def raw(self, name: str) -> np.ndarray:
        """The tensor as it goes to the device: fp32 values or bf16 bits."""
        x = getattr(self, name)
        return bf16_bits(x) if self.dtype == "bf16" else x

    @property
    def tokens(self) -> int:
        return self.B * self.N


def _finish(w: Workload, q, k, v) -> Workload:
    if w.dtype == "bf16":
        q, k, v = (bf16_to_f32(bf16_bits(x)) for x in (q, k, v))
    w.q, w.k, w.v = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v))
    return w


def iid(name, B, H, N, d=64, dtype="bf16", scale=1.0, seed=0, block_per_row=4,
        approx_mode="full", prior_first=0, prior_diag=0, mask=None) -> Workload:
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    w = Workload(name, B, H, N, d, dtype, block_per_row, approx_mode, prior_first, prior_diag,
                 mask=mask)
    return _finish(w, q, k, v)


def from_arrays(name, q, k, v, dtype="bf16", block_per_row=4, approx_mode="full", prior_first=0, prior_diag=0,
                mask=None) -> Workload:
    """A workload from given [B, H, N, d] arrays (rounded to bf16 when dtype is bf16)."""
    B, H, N, d = q.shape
    w = Workload(name, B, H, N, d, dtype, block_per_row, approx_mode, prior_first, prior_diag, mask=mask)
    return _finish(w, q, k, v)


def c1() -> Workload:
    """fp32, B=1, H=2, N=512, d=64, N(0,1), no mask, bpr 4 (64 of 256), full."""
    return iid("C1-fp32-N512-full", 1, 2, 512, dtype="f32", scale=1.0, seed=1)


def c2() -> Workload:
    """MRA-base layer shape: bf16, B=8, H=12, N=512, N(0,1)*0.5; per-sequence
    valid length 32*ceil(U/32), U uniform in [256, 512]; tail masked; full."""
    rng = np.random.default_rng(2)
    B, H, N, d = 8, 12, 512, 64
    shape = (B, H, N, d)
    q = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.5)
    k = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.5)
    v = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.5)
    U = rng.integers(256, 513, size=B)
    L = 32 * ((U + 31) // 32)
    mask = (np.arange(N)[None, :] < L[:, None]).astype(np.uint8)
    w = Workload("C2-bf16-N512-full-masked", B, H, N, d, "bf16", 4, "full", mask=mask)
    return _finish(w, q, k, v)


def c3() -> Workload:
    """bf16, B=2, H=12, N=4096, N(0,1)*0.5, sparse mode, bpr 4 (512 per head),
    first-n prior 2, diagonal prior 3."""
    return iid("C3-bf16-N4096-sparse-priors", 2, 12, 4096, scale=0.5, seed=3,
               approx_mode="sparse", prior_first=2, prior_diag=3)


def c4() -> Workload:
    """Clustered: bf16, B=2, H=12, N=4096.  Per sequence, 15 distinct cut points
    in 1..N-1 split the tokens into 16 contiguous runs shared by its heads; per
    (b, h), 16 centroids ~ N(0, I); Q and K = centroid of the token's run +
    0.3 * N(0, 1) noise (drawn separately); V ~ N(0, 1).  bpr 4, full."""
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 12, 4096, 64
    q = np.empty((B, H, N, d), np.float32)
    k = np.empty((B, H, N, d), np.float32)
    for b in range(B):
        cuts = np.sort(rng.choice(np.arange(1, N), size=15, replace=False))
        run = np.searchsorted(cuts, np.arange(N), side="right")  # run id 0..15
        for h in range(H):
            cent = rng.standard_normal((16, d), dtype=np.float32)
            q[b, h] = cent[run] + np.float32(0.3) * rng.standard_normal((N, d), dtype=np.float32)
            k[b, h] = cent[run] + np.float32(0.3) * rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    w = Workload("C4-bf16-N4096-full-clustered", B, H, N, d, "bf16", 4, "full")
    return _finish(w, q, k, v)


def c5() -> Workload:
    """bf16, B=1, H=16, N=16384, N(0,1)*0.5, bpr 8 (4096 of 262144 per head),
    full, diagonal prior 1."""
    return iid("C5-bf16-N16384-full-diag1", 1, 16, 16384, scale=0.5, seed=5,
               block_per_row=8, prior_diag=1)


CONFIGS = {"C1": c1, "C2": c2, "C3": c3, "C4": c4, "C5": c5}


def get(name: str) -> Workload:
    return CONFIGS[name]()


def bigbird_rand(B, H, N, block_size=64, r=3, seed=0) -> np.ndarray:
    """The random key blocks a BigBird layer draws for each query block
    ([BigBird]: num_random_blocks per query block), drawn here and passed in
    as an input: r distinct blocks outside the block's 3-block window and the
    two global blocks (first and last), or -1 where fewer than r remain.
    Returns int32 [B, H, N / block_size, r]."""
    rng = np.random.default_rng(seed)
    nbb = N // block_size
    out = np.full((B, H, nbb, r), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for I in range(nbb):
                cand = [J for J in range(1, nbb - 1) if abs(I - J) > 1]
                if cand:
                    pick = rng.choice(cand, size=min(r, len(cand)), replace=False)
                    out[b, h, I, :len(pick)] = pick
    return out


@dataclass
class BigBirdWorkload:
    name: str
    w: Workload                 # q, k, v, mask and dtype (block_per_row, approx_mode unused)
    block_size: int
    rand: np.ndarray = field(repr=False, default=None)   # int32 [B, H, N / block_size, r]


def bigbird(name="BB-bf16-N4096-bs64-r3", B=2, H=12, N=4096, block_size=64, r=3, dtype="bf16", seed=6,
            scale=0.5, mask=None, d=64) -> BigBirdWorkload:
    """BigBird block-sparse workload: the page's defaults (block 64, three
    random blocks) at the N = 4096 sequence length it is built for, iid
    inputs of the same scale as the MRA workloads."""
    w = iid(name, B, H, N, d=d, dtype=dtype, scale=scale, seed=seed, approx_mode="sparse", mask=mask)
    return BigBirdWorkload(name, w, block_size, bigbird_rand(B, H, N, block_size, r, seed + 100))
