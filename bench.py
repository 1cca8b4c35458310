#!/usr/bin/env python3
"""Benchmark of the MRA-2 forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4]

A step is one call of the whole forward pass (pooling, low-res logits, top-k
selection, block attention with the low-res merge) on inputs already
resident in HBM.  The default workload is the clustered N=4096 bf16 full-mode
case (B=2, H=12, d=64, block_per_row=4), the one configuration at N=4096 that
runs every stage.  W untimed warm-up steps, then exactly K timed steps
bracketed by torch.cuda.synchronize(); rank 0 prints one JSON line.

Besides tokens/s the line carries:
  * per-kernel average durations, from HIP events recorded around each launch
    on the library's stream (a second loop of K calls through
    mra_attention_fwd_profiled, each call with its own events, one
    synchronisation at the end);
  * for the block attention, `replay_us`: the average of
    K back-to-back relaunches of that kernel alone (mra_debug_replay) between
    one pair of events on the same stream, which leaves out the cost of the
    events between the kernels of a call;
  * `roofline` for the kernel with the largest average duration: its
    algorithmic bytes per launch (every input it needs read once, every
    output written once) over its average duration (replay_us where there
    is one), against HBM; for the
    block attention, whose arithmetic intensity (4*32*32*d flop per selected
    block) is far below the MFMA ridge, the MFMA rate is given beside it;
  * `traffic`: HBM bytes per launch of that kernel from rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters committed under profiles/, scaled by the same
    counters' reading on a plain copy of known size; null when the kernel
    source changed since the counters were taken;
  * `cpu_baseline`: the CPU oracle on the host cores (the whole workload,
    repeated for about 10 s);
  * `backward`: the gradient pass (mra_attention_bwd) on the N=4096
    workloads C3 (sparse mode, priors) and C4 (full mode, clustered), K timed
    calls between HIP events on the library's stream after a forward call
    that left its selection and statistics in the workspace; its algorithmic
    bytes (Q, K, V, O, dO read once, dQ, dK, dV written once) and MFMA work
    (five 32x32x64 products per selected block: S, dP, dS K, dS^T Q, P^T dO;
    the low-res terms of full mode, 4 nb^2 d multiply-adds per head, are
    left out) over that time;
  * `bigbird`: BigBird block-sparse attention (mra_bigbird_fwd: the BigBird
    page's window of three blocks, two global blocks and three random blocks
    of 64 tokens) on B=2, H=12, N=4096 bf16, through the same attention
    kernels; algorithmic bytes Q, K, V read and O written once, MFMA work
    4 x 32 x 32 x 64 per attended 32-token cell; and its backward pass
    (mra_bigbird_bwd) timed the same way;
  * `head128`: the forward pass on 128-channel heads (B=2, H=12, N=4096,
    bf16, full mode, i.i.d. N(0,1)*0.5 inputs), timed the same way, with the
    same algorithmic bytes and MFMA work at d=128, and its backward pass;
  * `regimes`: for the three N >= 4096 workloads (C3 sparse with priors, C4
    full clustered, C5 N=16384), per-call durations of --calls calls (200 by
    default), each call between its own pair of HIP events: median, p10 and
    p90 in two regimes.  "warm": calls back to back, so inputs and workspace
    stay in the 256 MB last-level cache (MALL).  "cold": before each call
    (outside its events) a 1 GiB buffer is rewritten by a fill kernel, more
    than the MALL and the L2s hold, so the call starts from HBM;
  * `attn_cold`: the block attention kernel alone after the same 1 GiB write
    (a relaunch on the filled workspace), median of --calls launches, with
    its algorithmic HBM rate;
  * `copy_bandwidth`: a measured device-to-device copy of 1 GiB (bytes read
    plus bytes written over the median duration of 20 copies), the practical
    HBM ceiling the roofline fractions are also given against.
The headline `value` stays the wall-clock rate of the K timed steps.  Only
one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3     # MI355X fp32 matrix
METRIC = "MRA-2 fwd tokens/s and sparse-block MFMA % of peak, N=4096 bf16, 1 MI355X"
KERNEL_SOURCES = {
    "pool": "mra_pool.hip", "logits": "mra_select.hip", "select": "mra_select.hip",
    "logits+select": "mra_select.hip", "attn": "mra_attn.hip",
}


def kernel_hash(stage: str) -> str:
    csrc = os.path.join(ROOT, "block_sparse_approximate_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[stage], "mra_common.h"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic(w, stage: str, sel_blocks: int) -> tuple[float, str]:
    """(amount per launch, unit) for a stage: flops for the block attention,
    bytes for the memory-bound stages.  Bytes are what the method must move:
    every input read once and every output written once."""
    B, H, N, d = w.B, w.H, w.N, w.d
    BH, nb = B * H, N // 32
    es = 2 if w.dtype == "bf16" else 4
    full = w.approx_mode == "full"
    fused = nb in (64, 128)    # one launch forms the logits, selects and (full mode) pools V
    ntens = 3 if full and not fused else 2
    K = nb * w.block_per_row if nb * w.block_per_row < nb * nb else nb * nb
    mask_b = 0 if w.mask is None else B * N
    if stage == "attn":        # Q, K, V read once and O written once (its arithmetic intensity is far
        return 4 * BH * N * d * es, "byte"   # below the MFMA ridge, so HBM is its roofline)
    if stage == "pool":        # Q, K (V) in; pooled fp32 rows and block counts out
        return ntens * BH * N * d * es + mask_b + ntens * BH * nb * d * 4 + 2 * B * nb * 4, "byte"
    if stage == "logits":      # pooled Q, K (V) in; logits, row maxima (low-res row sums) out
        lowres = BH * nb * d * 4 + BH * nb * (d + 1) * 4 if full else 0
        return 2 * BH * nb * d * 4 + BH * nb * nb * 4 + BH * nb * 4 + lowres, "byte"
    if stage == "select":      # logits and row maxima in; K block indices out
        return BH * nb * nb * 4 + BH * nb * 4 + BH * K * 4, "byte"
    if stage == "logits+select":   # one launch for both (N = 2048, 4096), which also pools V in full mode
        v = BH * N * d * es + BH * nb * d * 4 if full else 0
        return algorithmic(w, "logits", sel_blocks)[0] + algorithmic(w, "select", sel_blocks)[0] + v, "byte"
    raise ValueError(stage)


def selected_valid_blocks(w) -> int:
    """Selected blocks whose query and key blocks both hold valid tokens (the
    useful ones); every selected block when there is no mask."""
    import numpy as np
    nb = w.N // 32
    K = min(nb * w.block_per_row, nb * nb)
    if w.mask is None:
        return w.B * w.H * K
    cnt = w.mask.reshape(w.B, nb, 32).sum(-1)
    valid = (cnt > 0).sum(-1)            # a fully valid-pair budget is min(K, valid^2)
    return int(sum(w.H * min(K, int(v) * int(v)) for v in valid))


SCRUB_BYTES = 1 << 30   # more than the 256 MB MALL plus the L2s


def percentiles(ts):
    import numpy as np
    a = np.asarray(ts, np.float64)
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "mean_us": round(float(a.mean()), 2),
            "calls": int(a.size)}


def time_each(call, n, scrub=None):
    """Durations (us) of n calls of `call`, each between its own pair of HIP
    events on the current stream.  With `scrub` (a device buffer), a fill
    kernel rewrites it before each call, outside the call's events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        if scrub is not None:
            scrub.fill_(i % 251 + 1)
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def copy_bandwidth():
    """Bytes read plus bytes written per second of a 1 GiB device-to-device
    copy (median of 20)."""
    import torch
    a = torch.full((SCRUB_BYTES,), 7, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ts = time_each(lambda: b.copy_(a), 20)
    import numpy as np
    med = float(np.median(ts)) * 1e-6
    del a, b
    return {"bytes_moved": 2 * SCRUB_BYTES, "median_us": round(med * 1e6, 1),
            "GBs": round(2 * SCRUB_BYTES / med / 1e9, 1), "kind": "torch copy_ of 1 GiB, device to device"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_regimes(mra, cfgs, calls: int, copy_gbs: float) -> dict:
    """Warm and cold per-call durations of the forward pass on the named
    workloads, and for the block attention alone after the cold write."""
    import numpy as np
    import torch

    import workloads

    scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
    res = {}
    attn_cold = {}
    for cfg in cfgs:
        w = workloads.get(cfg)
        q, k, v = (torch.from_numpy(w.raw(n).view(np.int16)).view(torch.bfloat16).cuda() for n in ("q", "k", "v"))
        mask = None if w.mask is None else torch.from_numpy(w.mask).cuda()
        kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode,
                  initial_prior_first_n_blocks=w.prior_first, initial_prior_diagonal_n_blocks=w.prior_diag)
        out = torch.empty_like(q)
        ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, w.d, q.dtype, w.block_per_row, w.approx_mode),
                         dtype=torch.uint8, device="cuda")
        call, _ = mra.prepare(q, k, v, mask, out=out, workspace=ws, **kw)
        for _ in range(20):
            call()
        warm = percentiles(time_each(call, calls))
        cold = percentiles(time_each(call, calls, scrub))
        tokens = w.B * w.N
        for r in (warm, cold):
            r["tokens_per_s"] = round(tokens / (r["median_us"] * 1e-6), 1)
        res[w.name] = {"warm": warm, "cold": cold}
        if cfg == "C4":
            replay = lambda: mra.debug_replay(q, k, v, 3, 1, mask, out=out, workspace=ws, **kw)
            a = percentiles(time_each(replay, calls, scrub))
            nbytes = 4.0 * w.B * w.H * w.N * w.d * 2
            gbs = nbytes / (a["median_us"] * 1e-6) / 1e9
            attn_cold = dict(a, workload=w.name, algorithmic_bytes=int(nbytes), achieved_GBs=round(gbs, 1),
                             frac_of_peak=round(gbs / PEAK_HBM_GBS, 4),
                             frac_of_measured_copy=round(gbs / copy_gbs, 4) if copy_gbs else None,
                             regime="cold: a 1 GiB write before each launch; Q, K, V and the workspace come "
                                    "from HBM")
        del q, k, v, out, ws
    del scrub
    return {"regimes": res, "attn_cold": attn_cold}


def load_traffic(stage: str, workload: str):
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path))
    except Exception:
        return None
    e = t.get(stage)
    if not e or e.get("workload") != workload or e.get("source_hash") != kernel_hash(stage):
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(w, seconds: float = 10.0):
    import oracle
    threads = oracle.default_threads()
    runs, t0 = 0, time.perf_counter()
    while True:
        oracle.mra_forward(w.q, w.k, w.v, w.mask, block_per_row=w.block_per_row, approx_mode=w.approx_mode,
                           prior_first=w.prior_first, prior_diag=w.prior_diag, threads=threads)
        runs += 1
        el = time.perf_counter() - t0
        if el >= seconds or runs >= 200:
            break
    return {"value": w.B * w.N * runs / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "the whole %s workload (%d heads), %d runs in %.1f s" % (w.name, w.B * w.H, runs, el)}


def bench_backward(mra, steps: int, warmup: int, cfg: str) -> dict:
    import numpy as np
    import torch

    import workloads

    w = workloads.get(cfg)
    to_dev = lambda n: torch.from_numpy(w.raw(n).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_dev("q"), to_dev("k"), to_dev("v")
    kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode, initial_prior_first_n_blocks=w.prior_first,
              initial_prior_diagonal_n_blocks=w.prior_diag)
    ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, w.block_per_row, w.approx_mode),
                     dtype=torch.uint8, device="cuda")
    out = mra.attention(q, k, v, None, workspace=ws, save_stats=True, **kw)
    g = torch.from_numpy(np.random.default_rng(1).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16).cuda()
    run, _ = mra.prepare_backward(q, k, v, out, g, ws, None, **kw)
    for _ in range(warmup):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    BH, K = w.B * w.H, mra.num_block(w.N, w.block_per_row)
    nbytes = 8.0 * BH * w.N * w.d * 2
    flops = 5.0 * 2 * 32 * 32 * w.d * BH * K
    return {"workload": w.name, "ms_per_call": round(ms, 5), "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
            "algorithmic_bytes": int(nbytes), "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def bench_bigbird(mra, steps: int, warmup: int) -> dict:
    """BigBird block-sparse attention (the BigBird page's pattern: window of
    three blocks, first and last blocks global, three random blocks, block
    64) on the N=4096 bf16 workload, through the same attention kernels."""
    import numpy as np
    import torch

    import workloads

    bb = workloads.bigbird()
    w = bb.w
    to_dev = lambda n: torch.from_numpy(w.raw(n).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_dev("q"), to_dev("k"), to_dev("v")
    rand = torch.from_numpy(bb.rand).cuda()
    run, out = mra.prepare_bigbird(q, k, v, rand, None, bb.block_size)
    for _ in range(warmup):
        run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # its backward pass (mra_bigbird_bwd) on the layout that forward left
    g = torch.from_numpy(np.random.default_rng(2).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
    g = g.cuda()
    r = int(bb.rand.shape[3])
    fws = torch.empty(mra.bigbird_workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, bb.block_size, r),
                      dtype=torch.uint8, device="cuda")
    out = mra.bigbird_attention(q, k, v, rand, None, bb.block_size, workspace=fws)
    bws = torch.empty(mra.bigbird_backward_workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, bb.block_size, r),
                      dtype=torch.uint8, device="cuda")
    grads = [torch.empty_like(q) for _ in range(3)]
    bwd = lambda: mra.bigbird_backward(q, k, v, out, g, fws, r, None, bb.block_size, *grads, bwd_workspace=bws)
    for _ in range(warmup):
        bwd()
    e0.record()
    for _ in range(steps):
        bwd()
    e1.record()
    torch.cuda.synchronize()
    ms_bwd = e0.elapsed_time(e1) / steps
    # attended 32-token cells: f x f per attended pattern cell
    nbb, f = w.N // bb.block_size, bb.block_size // 32
    cells = 0
    for b in range(w.B):
        for h in range(w.H):
            I = np.arange(nbb)[:, None]
            J = np.arange(nbb)[None, :]
            att = (np.abs(I - J) <= 1) | (I == 0) | (I == nbb - 1) | (J == 0) | (J == nbb - 1)
            for i in range(nbb):
                for x in bb.rand[b, h, i]:
                    if 0 <= x < nbb:
                        att[i, x] = True
            cells += int(att.sum()) * f * f
    nbytes = 4.0 * w.B * w.H * w.N * w.d * 2
    flops = 4.0 * 32 * 32 * w.d * cells
    return {"workload": w.name, "block_size": bb.block_size, "num_random_blocks": int(bb.rand.shape[3]),
            "ms_per_call": round(ms, 5), "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1),
            "attended_cells_32": cells, "algorithmic_bytes": int(nbytes),
            "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "backward_ms_per_call": round(ms_bwd, 5),
            "backward_tokens_per_s": round(w.B * w.N / (ms_bwd * 1e-3), 1)}


def bench_head128(mra, steps: int, warmup: int) -> dict:
    """The forward pass on 128-channel heads: bf16, B=2, H=12, N=4096,
    Q/K/V i.i.d. N(0,1)*0.5, block_per_row=4, full mode."""
    import numpy as np
    import torch

    import workloads

    w = workloads.iid("D128-bf16-N4096-full", 2, 12, 4096, d=128, dtype="bf16", seed=128, scale=0.5,
                      block_per_row=4, approx_mode="full")
    to_dev = lambda n: torch.from_numpy(w.raw(n).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_dev("q"), to_dev("k"), to_dev("v")
    kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode)
    call, out = mra.prepare(q, k, v, None, **kw)
    for _ in range(warmup):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # its backward pass on the selection that forward left
    ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, w.d, torch.bfloat16, w.block_per_row, w.approx_mode),
                     dtype=torch.uint8, device="cuda")
    out = mra.attention(q, k, v, None, workspace=ws, save_stats=True, **kw)
    g = torch.from_numpy(np.random.default_rng(3).standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16)
    run, _ = mra.prepare_backward(q, k, v, out, g.cuda(), ws, None, **kw)
    for _ in range(warmup):
        run()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_bwd = e0.elapsed_time(e1) / steps
    BH, K = w.B * w.H, mra.num_block(w.N, w.block_per_row)
    nbytes = 4.0 * BH * w.N * w.d * 2          # Q, K, V read and O written once, bf16
    flops = 4.0 * 32 * 32 * w.d * BH * K       # QK^T and PV on the selected blocks
    return {"workload": w.name, "head_dim": w.d, "ms_per_call": round(ms, 5),
            "backward_ms_per_call": round(ms_bwd, 5),
            "backward_tokens_per_s": round(w.B * w.N / (ms_bwd * 1e-3), 1),
            "tokens_per_s": round(w.B * w.N / (ms * 1e-3), 1), "algorithmic_bytes": int(nbytes),
            "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "mfma_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-bigbird", action="store_true")
    ap.add_argument("--no-head128", action="store_true")
    ap.add_argument("--no-regimes", action="store_true", help="skip the warm/cold per-call records")
    ap.add_argument("--calls", type=int, default=200, help="calls per regime record")
    ap.add_argument("--only-head128", action="store_true",
                    help="only time the forward pass on 128-channel heads (N=4096 bf16 full mode)")
    ap.add_argument("--only-bigbird", action="store_true",
                    help="only time BigBird block-sparse attention on its N=4096 workload")
    ap.add_argument("--only-backward", metavar="CFG", default=None,
                    help="only time the backward pass on workload CFG (C3 or C4) and print its record")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB fp32 copy (x * 1.0) 10 times, to calibrate HBM counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(10):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                          "launches": 10}))
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the MRA forward shards by (batch, head) with "
              "no exchange between shards); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_approximate_amd as mra
    import workloads

    if args.only_bigbird:
        torch.cuda.set_device(torch.device("cuda:0"))
        print(json.dumps({"bigbird": bench_bigbird(mra, args.steps, args.warmup)}), flush=True)
        return
    if args.only_head128:
        torch.cuda.set_device(torch.device("cuda:0"))
        print(json.dumps({"head128": bench_head128(mra, args.steps, args.warmup)}), flush=True)
        return
    if args.only_backward:
        torch.cuda.set_device(torch.device("cuda:0"))
        print(json.dumps({"backward": bench_backward(mra, args.steps, args.warmup, args.only_backward)}),
              flush=True)
        return

    w = workloads.get(args.config)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(name):
        x = w.raw(name)
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v = to_dev("q"), to_dev("k"), to_dev("v")
    mask = None if w.mask is None else torch.from_numpy(w.mask).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(mra.workspace_size(w.B, w.H, w.N, w.d, dt, w.block_per_row, w.approx_mode),
                     dtype=torch.uint8, device=dev)
    kw = dict(block_per_row=w.block_per_row, approx_mode=w.approx_mode,
              initial_prior_first_n_blocks=w.prior_first, initial_prior_diagonal_n_blocks=w.prior_diag,
              out=out, workspace=ws)

    step, _ = mra.prepare(q, k, v, mask, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = wall * 1e3 / args.steps

    # per-kernel durations: events around each launch, on the library's stream
    # (each call gets its own events, so the stream is never drained between calls)
    stages = list(mra.STAGES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * len(stages))] for _ in range(args.steps)]
    for ev in evs:
        for e in ev:
            e.record()
    torch.cuda.synchronize()
    tp0 = time.perf_counter()
    for ev in evs:
        mra.attention_profiled(q, k, v, ev, mask, **kw)
    torch.cuda.synchronize()
    prof_wall = (time.perf_counter() - tp0) * 1e3 / args.steps
    avg_ms = {s: sum(ev[2 * si].elapsed_time(ev[2 * si + 1]) for ev in evs) / args.steps
              for si, s in enumerate(stages)}
    if w.N // 32 in (64, 128):
        # one launch forms the logits and selects (its stage is the select one)
        avg_ms = {"pool": avg_ms["pool"], "logits+select": avg_ms["logits"] + avg_ms["select"],
                  "attn": avg_ms["attn"]}

    # attention alone: back-to-back relaunches on the workspace the last call
    # filled, one pair of events around them
    replay_ms = {}
    for si in (3,):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mra.debug_replay(q, k, v, si, 2, mask, **kw)
        r0.record()
        mra.debug_replay(q, k, v, si, args.steps, mask, **kw)
        r1.record()
        torch.cuda.synchronize()
        replay_ms[stages[si]] = r0.elapsed_time(r1) / args.steps

    sel_blocks = selected_valid_blocks(w)
    kernels = {}
    for s, t in avg_ms.items():
        amount, unit = algorithmic(w, s, sel_blocks)
        rate = amount / (replay_ms.get(s, t) * 1e-3)
        kernels[s] = {"avg_us": round(t * 1e3, 2), "gbs": round(rate / 1e9, 1),
                      "hbm_frac": round(rate / 1e9 / PEAK_HBM_GBS, 4)}
    for s, t in replay_ms.items():
        kernels[s]["replay_us"] = round(t * 1e3, 2)
    attn_flops = 4.0 * 32 * 32 * w.d * sel_blocks
    mfma_peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    attn_tflops = attn_flops / (replay_ms["attn"] * 1e-3) / 1e12
    kernels["attn"]["tflops"] = round(attn_tflops, 2)
    kernels["attn"]["mfma_frac"] = round(attn_tflops / mfma_peak, 4)
    dom = max(avg_ms, key=avg_ms.get)
    amount, unit = algorithmic(w, dom, sel_blocks)
    dom_s = replay_ms.get(dom, avg_ms[dom]) * 1e-3
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(amount / dom_s / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "duration_us": round(dom_s * 1e6, 2),
            "timing": "replay" if dom in replay_ms else "events"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["regime"] = ("warm: back-to-back relaunches on a workspace the previous call filled; inputs and "
                      "workspace resident in the 256 MB MALL" if dom in replay_ms else "warm: back-to-back calls")
    roof["traffic"] = load_traffic(dom, w.name)
    roof["algorithmic_bytes"] = int(amount)
    if dom == "attn":
        roof["mfma_tflops"] = kernels["attn"]["tflops"]
        roof["mfma_frac"] = kernels["attn"]["mfma_frac"]

    tokens = w.B * w.N
    rec = {
        "metric": METRIC,
        "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, see workloads.py)",
        "config": {"workload": w.name, "batch": w.B, "heads": w.H, "seq_len": w.N, "head_dim": w.d,
                   "block_per_row": w.block_per_row, "approx_mode": w.approx_mode,
                   "initial_prior_first_n_blocks": w.prior_first,
                   "initial_prior_diagonal_n_blocks": w.prior_diag, "parallelism": "single GPU"},
        "useful_tflops": round(attn_flops / (ms * 1e-3) / 1e12, 3),
        "attn_mfma_frac": kernels["attn"]["mfma_frac"],
        "kernels": kernels,
        "profiled_ms_per_step": round(prof_wall, 5),
        "roofline": roof,
    }
    if not args.no_regimes:
        cb = copy_bandwidth()
        rec["copy_bandwidth"] = cb
        roof["frac_of_measured_copy"] = round(roof["achieved"] / cb["GBs"], 4)
        rec.update(bench_regimes(mra, ("C3", "C4", "C5"), args.calls, cb["GBs"]))
    if not args.no_backward:
        rec["backward"] = [bench_backward(mra, args.steps, args.warmup, cfg) for cfg in ("C3", "C4")]
    if not args.no_bigbird:
        rec["bigbird"] = bench_bigbird(mra, args.steps, args.warmup)
    if not args.no_head128:
        rec["head128"] = bench_head128(mra, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
