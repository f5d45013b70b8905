#!/usr/bin/env python3
"""Benchmark of the HCA layer forward (pooling + attention) on one MI355X.

One step = one pass of the whole path over one batch of the workload:
  prefill workloads: hca_compress (K and V) then hca_attend_prefill;
  decode workload:   hca_attend_decode;
  mixed_1m:          pooling + prefill of the 32768-token chunk, then decode
                     of the 8 long-context sequences.
The default workload is prefill_128k (B=1, T=131072, Hq=64, Hkv=1, d=512,
W=128, 1024 compressed entries): the largest prefill and the one bound by
the matrix cores; `value` is its prefill throughput in tokens/s.  The same
run also times decode_64x128k (64 queries against 128K-token caches, under
"decode") and mixed_1m (8 decode queries at 256K-1M plus a 32768-token
chunk as one step, under "mixed"), and the measurement probes (a streaming
read and a matrix-core loop, under "measured_peaks").  Inputs are seeded
synthetic tensors resident in HBM before the timed region.

Per-kernel durations come from HIP events recorded on the stream the kernels
run on, around every launch of the timed steps (mean, median and min are
reported).  The roofline entries use algorithmic work: bytes (flops) the
method must move (compute), not what the implementation adds.  `traffic` is
filled from the counter summary in profiles/ when it was measured on the
current kernel source, else null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "HCA prefill tokens/s (%MFMA peak) + decode queries/s (%HBM peak), 1 GPU"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
WORKLOADS = ("prefill_8k", "prefill_128k", "decode_64x128k", "mixed_1m", "tiny_f32", "chunk_32k_at_224k",
             "dsa_decode_64x128k")
DSA_BATCH, DSA_LEN, DSA_TOPK, DSA_SEED = 64, 131072, 2048, 1011
EPILOGUE_RANK = 16  # head-mixing rank of the fused-epilogue measurement (the pages give none)
_CS = "compressed_kv_sparse_amd/csrc/"
KERNEL_SOURCES = {
    "prefill": (_CS + "prefill_bf16.hip", _CS + "bf16_tiles.h"),
    "prefill_gated_vha": (_CS + "prefill_bf16.hip", _CS + "bf16_tiles.h"),
    "decode": (_CS + "decode_bf16.hip", _CS + "bf16_tiles.h"),
    "decode_gated_vha": (_CS + "decode_bf16.hip", _CS + "bf16_tiles.h"),
    "compress": (_CS + "compress.hip",),
    "prefill_chunk": (_CS + "chunk.hip", _CS + "prefill_bf16.hip", _CS + "bf16_tiles.h"),
    "compress_chunk": (_CS + "compress.hip",),
    "ring_append": (_CS + "chunk.hip",),
    "decode_maintenance": (_CS + "compress.hip", _CS + "chunk.hip"),
    "backward": (_CS + "backward_bf16.hip", _CS + "bf16_tiles.h"),
    "dsa_decode": (_CS + "dsa.hip",),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def keys_visible(t, window, block=128):
    return (t + 1) // block + min(window, t + 1)


def prefill_work(c, lens, e):
    """(bytes, flops) of one hca_attend_prefill launch: Q read + O write,
    raw K+V read once, each compressed entry read once; 4*d*Hq flops per
    visible (query, key) pair."""
    ntok = sum(lens)
    nblk = sum(l // c.block for l in lens)
    byt = ntok * (2 * c.hq * c.d * e + 2 * c.hkv * c.d * e) + nblk * 2 * c.hkv * c.d * e
    pairs = 0
    for L in lens:
        n = L // c.block
        # sum over t of floor((t+1)/128): block j is seen by L - (128(j+1) - 1) tokens
        comp = sum(L - (c.block * (j + 1) - 1) for j in range(n))
        W = c.window
        raw = (min(W, L) * (min(W, L) + 1)) // 2 + max(0, L - W) * W
        pairs += comp + raw
    return byt, 4 * c.d * c.hq * pairs


def backward_work(c, lens, e):
    """(bytes, flops) of one hca_attend_prefill_backward call: q, o, dout
    read and dq written; raw K, V read and dK, dV written; the entries read;
    10*d*Hq flops per visible (query, key) pair (the scores S and dP, and
    the products for dQ, dK and dV, each 2*d per pair and head)."""
    pb, pf = prefill_work(c, lens, e)
    ntok = sum(lens)
    nblk = sum(l // c.block for l in lens)
    byt = ntok * (4 * c.hq * c.d * e + 4 * c.hkv * c.d * e + 4 * c.hq) + nblk * 2 * c.hkv * c.d * e
    return byt, pf // 4 * 10


def dsa_work(lens, topk, hq=64, d=256, di=128):
    """(bytes, flops) of one hca_dsa_decode call: every cached indexer key
    read once (di int8 bytes per position), the selected K and V rows read
    once, q read, o written, the selection written; 2*di integer ops per
    scored position and 4*d*Hq flops per selected key."""
    byt, flops = 0, 0
    for L in lens:
        n = min(L, topk)
        byt += L * di + n * 2 * d * 2 + 2 * hq * d * 2 + di + topk * 4
        flops += 2 * di * L + 4 * d * hq * n
    return byt, flops


def compress_work(c, lens, e):
    nblk = sum(l // c.block for l in lens)
    return nblk * c.hkv * (2 * c.block * c.d * e + 2 * c.d * e), nblk * c.hkv * 4 * c.block * c.d


def ntok_of(lens):
    return int(sum(lens))


def chunk_work(c, p0, n, e):
    """(bytes, flops) of one hca_attend_prefill_chunk call: Q read + O write,
    the chunk's raw K+V and the window-1 ring rows before it read once, every
    visible compressed entry read once; 4*d*Hq flops per visible (query, key)
    pair."""
    L = p0 + n
    byt = n * (2 * c.hq * c.d * e + 2 * c.hkv * c.d * e) + min(c.window - 1, p0) * 2 * c.hkv * c.d * e
    byt += (L // c.block) * 2 * c.hkv * c.d * e
    pairs = 0
    for t in range(p0, L):
        pairs += (t + 1) // c.block + min(c.window, t + 1)
    return byt, pairs * 4 * c.d * c.hq


def decode_work(c, lens, e):
    byt = 0
    flops = 0
    for L in lens:
        nk = L // c.block + min(c.window, L)
        byt += 2 * c.hq * c.d * e + 2 * c.hkv * c.d * e * nk
        flops += 4 * c.d * c.hq * nk
    return byt, flops


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------
class KernelClock:
    """HIP event pairs around launches on torch's current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        a = t.cuda.Event(enable_timing=True)
        b = t.cuda.Event(enable_timing=True)
        a.record()
        out = fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))
        return out

    def times_ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]

    def mean_ms(self, name):
        ts = self.times_ms(name)
        return sum(ts) / max(1, len(ts))

    def stats_ms(self, name):
        """(mean, median, min) over the recorded launches."""
        ts = sorted(self.times_ms(name))
        if not ts:
            return 0.0, 0.0, 0.0
        n = len(ts)
        med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
        return sum(ts) / n, med, ts[0]

    def reset(self):
        self.pairs = {}


def source_sha(rels):
    """SHA-256 (16 hex digits) over the kernel's source files, in order."""
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt if
    the counters were taken on the current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kernel not in KERNEL_SOURCES or kv.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MEASURED = {}  # ceilings the probes reached in this run: "hbm" (GB/s), "mfma" (TFLOP/s)


def roofline(kernel, workload, byt, flops, ms, bound, clock=None, name=None):
    """Roofline entry of one kernel: achieved = algorithmic work per launch /
    mean launch time (HIP events).  With the clock and the recorded name the
    median and min per launch are added; `frac_of_measured` reads the same
    achieved rate against the probe's ceiling of this run."""
    if bound == "hbm":
        ach = byt / (ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        ach = flops / (ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    out = {"kernel": kernel, "bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
           "frac": round(ach / peak, 4), "traffic": measured_traffic(kernel, workload),
           "algorithmic_bytes": int(byt), "algorithmic_flops": int(flops), "avg_ms": round(ms, 5)}
    if clock is not None and name is not None:
        _, med, mn = clock.stats_ms(name)
        out["median_ms"], out["min_ms"] = round(med, 5), round(mn, 5)
    if MEASURED.get(bound):
        out["frac_of_measured"] = round(ach / MEASURED[bound], 4)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------
def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # noqa: BLE001
        return 1


def oracle_sample_rows(T, window, n_blocks=16):
    """The query rows every prefill sample of the oracle includes: the
    key-set boundaries t in {0, W-1, W, 126, 127, 128, 255, 256, T-1}, and
    for n_blocks blocks spread over the sequence the rows 128j+126, 128j+127
    and 128j+128 (the last row before a block completes, the row that
    completes it, the first row of the next block)."""
    fixed = {0, window - 1, window, 126, 127, 128, 255, 256, T - 1}
    nb = T // 128
    for j in range(0, nb, max(1, nb // n_blocks)):
        fixed |= {128 * j + 126, 128 * j + 127, 128 * j + 128}
    return sorted(x for x in fixed if 0 <= x < T)


def cpu_baseline_prefill(c, inp, seconds, min_rows=0):
    """The oracle on the boundary rows plus seeded random query rows (at
    least min_rows in all, then as many as fit in `seconds`), and the pooling
    of every block; the attention time per row is extrapolated to all T
    rows (a uniform random sample gives an unbiased mean per row)."""
    import numpy as np
    import torch

    import oracle

    T = inp["lens"][0]
    cu = inp["cu_seqlens_host"]
    # the raw rows decoded (exactly) to float64 once, as the oracle would
    # decode them on every call
    k, v, w = inp["k"].cpu().double().numpy(), inp["v"].cpu().double().numpy(), inp["w"].cpu()
    t0 = time.perf_counter()
    kc = oracle.compress(k, w, cu)
    vc = oracle.compress(v, w, cu)
    t_pool = time.perf_counter() - t0
    fixed = oracle_sample_rows(T, c.window)
    fixed_set = set(fixed)
    rand = [int(x) for x in np.random.default_rng(5).permutation(T) if int(x) not in fixed_set]
    order = fixed + rand
    done = 0
    t_att = 0.0
    step = 16
    while done < T and (done < min_rows or t_att < seconds):
        rows = sorted(order[done:done + step])
        q_rows = inp["q"].index_select(0, torch.tensor(rows, device=inp["q"].device)).cpu()
        t1 = time.perf_counter()
        oracle.attend_prefill(q_rows, k, v, kc, vc, cu, c.window, rows=rows, q_holds_rows_only=True)
        t_att += time.perf_counter() - t1
        done += len(rows)
    per_tok = t_att / done + t_pool / T
    how = "all" if done >= T else "extrapolated from"
    return {"value": round(1.0 / per_tok, 3), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{done} of {T} query rows ({len(fixed)} block-boundary and window-edge rows, the rest "
                      f"seeded random) attended in {t_att:.1f} s, plus pooling of all {len(kc)} blocks in "
                      f"{t_pool:.1f} s; tokens/s {how} the sampled rows"}


def cpu_baseline_decode(c, inp, seconds):
    import oracle

    lens = inp["lens"]
    done = 0
    t_all = 0.0
    while t_all < seconds and done < len(lens):
        b = done
        t1 = time.perf_counter()
        nb = lens[b] // c.block
        cb = int(inp["cu_blocks_host"][b])
        oracle.attend_decode(inp["q"][b:b + 1].cpu(), inp["kc"][cb:cb + nb].cpu(),
                             inp["vc"][cb:cb + nb].cpu(), inp["kw"][b:b + 1].cpu(),
                             inp["vw"][b:b + 1].cpu(), [lens[b]], [0, nb], c.window)
        t_all += time.perf_counter() - t1
        done += 1
    return {"value": round(done / t_all, 3), "unit": "queries/s", "cores": blas_threads(),
            "kind": "oracle", "sample": f"{done} of {len(lens)} queries in {t_all:.1f} s"}


def warm_up(torch, step, warmup, min_s):
    """W untimed steps, continued until at least min_s seconds of GPU work have
    run: the clocks of an idle GPU take tens of milliseconds to ramp, and a
    few short steps would leave the timed region on cold clocks.  Returns the
    number of warmup steps run."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < min_s:
        step(n)
        n += 1
        if n >= warmup and n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
COLD_BYTES = 512 << 20  # overwritten between cold calls: twice the 256 MiB last-level cache


def run_prefill(torch, hca, c, steps, warmup, clock, min_warm_s, lens=None, extras=True):
    """The prefill step (pooling, then attention) timed `steps` times.  Then,
    apart from the step: the pooling alone with a 512 MiB scratch buffer
    overwritten before each call (so the last-level cache cannot serve its
    rows; recorded as compress_cold), and with `extras` the fused epilogue,
    the lse forward and the backward."""
    from hca_workloads import prefill_inputs

    inp = prefill_inputs(c, "cuda", lens=lens)
    dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    p = hca.make_params(c.hq, c.hkv, c.d, c.window, dt)
    kc = torch.empty((max(1, inp["total_blocks"]), c.hkv, c.d), dtype=dt, device="cuda")
    vc = torch.empty_like(kc)
    o = torch.empty_like(inp["q"])

    def compress():
        return hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"], inp["w"],
                                v=inp["v"], kc=kc, vc=vc)

    def step():
        clock.run("compress", compress)
        clock.run("prefill", lambda: hca.hca_attend_prefill(p, inp["cu_seqlens"], inp["cu_blocks"],
                                                            inp["max_seqlen"], inp["q"], inp["k"],
                                                            inp["v"], kc, vc, o=o))

    nwarm = warm_up(torch, lambda i: step(), warmup, min_warm_s)
    clock.reset()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    scratch = torch.empty(COLD_BYTES // 4, dtype=torch.int32, device="cuda")
    for i in range(steps):
        scratch.fill_(i)
        clock.run("compress_cold", compress)
    torch.cuda.synchronize()
    del scratch
    if c.dtype == "bf16" and extras:
        # the same attention with the fused epilogue (gate + rank-16 head
        # mixing), timed apart: its cost over the plain launch
        g = torch.Generator(device="cuda").manual_seed(c.seed + 29)
        gate = torch.randn((inp["q"].shape[0], c.hq), generator=g, device="cuda")
        u = torch.randn((c.hkv, c.hq // c.hkv, EPILOGUE_RANK), generator=g, device="cuda") * 0.1
        v = torch.randn_like(u) * 0.1
        # warmed like the step: the pooling's cold loop above leaves the
        # clocks low, and a few short launches would be timed before they ramp
        warm_up(torch, lambda i: hca.hca_attend_prefill_gated_vha(
            p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"], inp["k"], inp["v"], kc, vc,
            gate=gate, vha_u=u, vha_v=v, o=o), 3, min_warm_s)
        for _ in range(steps):
            clock.run("prefill_gated_vha", lambda: hca.hca_attend_prefill_gated_vha(
                p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"], inp["k"], inp["v"], kc, vc,
                gate=gate, vha_u=u, vha_v=v, o=o))
        torch.cuda.synchronize()
        # the backward: gradients of the pooling + attention for a synthetic
        # dL/dO, from the forward's o and lse
        dout = (torch.randn(inp["q"].shape, generator=g, device="cuda")).to(dt)
        o2, lse = hca.hca_attend_prefill_lse(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                             inp["k"], inp["v"], kc, vc)
        ntok = inp["q"].shape[0]
        ws = hca.new_backward_workspace(p, len(inp["lens"]), ntok, inp["total_blocks"], inp["max_seqlen"])
        dq, dk, dv = torch.empty_like(inp["q"]), torch.empty_like(inp["k"]), torch.empty_like(inp["v"])
        dw = torch.empty((c.hkv, c.block), dtype=torch.float32, device="cuda")

        def bwd():
            return hca.hca_attend_prefill_backward(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"],
                                                   inp["total_blocks"], inp["q"], inp["k"], inp["v"], inp["w"], kc,
                                                   vc, o2, lse, dout, workspace=ws, dq=dq, dk=dk, dv=dv, dw=dw)
        warm_up(torch, lambda i: bwd(), 2, min_warm_s)
        for _ in range(steps):
            clock.run("prefill_lse", lambda: hca.hca_attend_prefill_lse(
                p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"], inp["k"], inp["v"], kc, vc,
                o=o2, lse=lse))
            clock.run("backward", bwd)
        torch.cuda.synchronize()
        del dout, o2, lse, ws, dq, dk, dv, dw
    return inp, wall, nwarm


def run_chunk(torch, hca, c, steps, warmup, clock, min_warm_s):
    """A continuation chunk: the cache holds the entries of the blocks before
    pos0 and a ring of the raw rows before pos0.  One step = hca_compress_chunk
    (the 256 blocks the chunk completes) + hca_attend_prefill_chunk +
    hca_ring_append.  The append writes a second ring, so every step starts
    from the same cache state and repeats the same work."""
    from hca_workloads import chunk_inputs

    ci = chunk_inputs(c, "cuda")
    p0, n, R, L = ci["pos0"], ci["n"], c.ring, ci["length"]
    bf = torch.bfloat16
    p = hca.make_params(c.hq, c.hkv, c.d, c.window, bf)

    def i32(x):
        return torch.tensor(x, dtype=torch.int32, device="cuda")

    cap = L // c.block
    kc = torch.empty((cap, c.hkv, c.d), dtype=bf, device="cuda")
    vc = torch.empty_like(kc)
    nb0 = p0 // c.block
    hca.hca_compress(p, i32([0, p0]), i32([0, nb0]), nb0, ci["k"][:p0], ci["w"], v=ci["v"][:p0],
                     kc=kc[:nb0], vc=vc[:nb0])
    slots = torch.arange(p0 - R, p0, device="cuda") % R
    kwa = torch.zeros((1, R, c.hkv, c.d), dtype=bf, device="cuda")
    vwa = torch.zeros_like(kwa)
    kwa[0, slots] = ci["k"][p0 - R:p0]
    vwa[0, slots] = ci["v"][p0 - R:p0]
    kwb, vwb = torch.empty_like(kwa), torch.empty_like(vwa)
    kch, vch = ci["k"][p0:L].contiguous(), ci["v"][p0:L].contiguous()
    cu, pos0, cub = i32([0, n]), i32([p0]), i32([0, cap])
    ws = hca.new_prefill_chunk_workspace(p, 1, n)
    o = torch.empty_like(ci["q"])

    def step(i):
        clock.run("compress", lambda: hca.hca_compress_chunk(p, cu, pos0, cub, n, kch, ci["w"], kwa, kc, v=vch,
                                                             vw=vwa, vc=vc))
        clock.run("prefill", lambda: hca.hca_attend_prefill_chunk(p, cu, pos0, cub, n, ci["q"], kch, vch, kc, vc,
                                                                  kwa, vwa, workspace=ws, o=o))
        clock.run("ring_append", lambda: hca.hca_ring_append(p, cu, pos0, n, kch, kwb, v=vch, vw=vwb))

    nwarm = warm_up(torch, step, warmup, min_warm_s)
    clock.reset()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ci, wall, nwarm


def cpu_baseline_chunk(c, ci, seconds):
    """The oracle on seeded-random query rows of the chunk, plus the pooling
    of the 256 blocks the chunk completes, prorated per chunk token."""
    import numpy as np
    import torch

    import oracle

    p0, n, L = ci["pos0"], ci["n"], ci["length"]
    k, v, w = ci["k"].cpu(), ci["v"].cpu(), ci["w"].cpu()
    cu = [0, L]
    kc = oracle.compress(k, w, cu)  # all entries (the oracle's own pooling)
    vc = oracle.compress(v, w, cu)
    t0 = time.perf_counter()
    lo = p0 - p0 % c.block
    oracle.compress(k[lo:L], w, [0, L - lo])  # the blocks the chunk completes, timed
    oracle.compress(v[lo:L], w, [0, L - lo])
    t_pool = time.perf_counter() - t0
    order = np.random.default_rng(7).permutation(n)
    done, t_att, step = 0, 0.0, 16
    while t_att < seconds and done < n:
        rel = sorted(int(x) for x in order[done:done + step])
        q_rows = ci["q"].index_select(0, torch.tensor(rel, device=ci["q"].device)).cpu()
        t1 = time.perf_counter()
        oracle.attend_prefill(q_rows, k, v, kc, vc, cu, c.window, rows=[p0 + r for r in rel], q_holds_rows_only=True)
        t_att += time.perf_counter() - t1
        done += len(rel)
    per_tok = t_att / done + t_pool / n
    return {"value": round(1.0 / per_tok, 3), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {n} chunk query rows (seeded random) attended in {t_att:.1f} s plus pooling "
                      f"of the chunk's {L // c.block - p0 // c.block} blocks in {t_pool:.1f} s, prorated per token"}


def run_dsa(torch, hca, args, clock):
    """The sparse-attention decode step of the full-context layers: 64
    sequences of 131072 cached positions, k = 2048 (1.2 GB of HBM traffic
    per call, so the 256 MB last-level cache cannot serve repeats)."""
    from hca_workloads import dsa_inputs

    lens = [DSA_LEN] * DSA_BATCH
    inp = dsa_inputs(lens, DSA_SEED, "cuda")
    ws = torch.empty(hca.hca_dsa_decode_workspace_bytes(DSA_BATCH, DSA_LEN, DSA_TOPK), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(inp["q"])
    sel = torch.empty((DSA_BATCH, DSA_TOPK), dtype=torch.int32, device="cuda")

    def step(i=0):
        clock.run("dsa_decode", lambda: hca.hca_dsa_decode(inp["seqlens"], inp["cu_rows"], DSA_LEN, DSA_TOPK, inp["q"],
                                                           inp["qi"], inp["k"], inp["v"], inp["ki"], workspace=ws,
                                                           o=o, sel=sel))

    nwarm = warm_up(torch, step, args.warmup, args.min_warmup_s)
    clock.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return inp, wall, nwarm


def cpu_baseline_dsa(inp, seconds):
    """The oracle on as many of the sequences as fit in `seconds`."""
    import oracle

    t0 = time.perf_counter()
    done = 0
    while done < len(inp["lens"]) and (time.perf_counter() - t0 < seconds or done == 0):
        b = done
        oracle.dsa_decode(inp["q"][b:b + 1].cpu(), inp["qi"][b:b + 1].cpu(),
                          inp["k"][b * DSA_LEN:(b + 1) * DSA_LEN].cpu(), inp["v"][b * DSA_LEN:(b + 1) * DSA_LEN].cpu(),
                          inp["ki"][b * DSA_LEN:(b + 1) * DSA_LEN].cpu(), [DSA_LEN], [0], DSA_TOPK)
        done += 1
    el = time.perf_counter() - t0
    return {"value": round(done / el, 3), "unit": "queries/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{done} of {len(inp['lens'])} sequences (131072 positions, k = 2048) in {el:.1f} s"}


def run_decode(torch, hca, c, steps, warmup, clock, min_warm_s, n_sets=4, epilogue=True):
    """Rotates n_sets independent caches so repeats do not hit in the 256 MiB
    last-level cache (n_sets x the cache bytes must exceed 512 MiB).  With
    `epilogue` the same decode with the fused epilogue is timed apart."""
    from hca_workloads import decode_inputs

    # every set has the workload's context lengths (drawn once, from the
    # workload's seed) and its own cache contents; enough sets that together
    # they exceed 512 MiB
    first = decode_inputs(c, "cuda", seed=c.seed)
    lens = first["lens"]
    n_sets = max(n_sets, -(-COLD_BYTES // decode_work(c, lens, 2)[0]) + 1)
    sets = [first] + [decode_inputs(c, "cuda", lens=lens, seed=c.seed + 17 * i) for i in range(1, n_sets)]
    p = hca.make_params(c.hq, c.hkv, c.d, c.window, torch.bfloat16)
    ws = [hca.new_decode_workspace(p, len(s["lens"]), s["max_blocks"]) for s in sets]
    outs = [torch.empty_like(s["q"]) for s in sets]

    # Cache maintenance of the step (timed apart, not part of decode): the new
    # token's row goes through hca_compress_chunk (it completes a block when
    # L is a multiple of 128) and hca_ring_append.  The caches already hold
    # that token, so both rewrite what is there and every step is the same.
    upd = []
    for s in sets:
        b = len(s["lens"])
        pos = [L - 1 for L in s["lens"]]
        slot = torch.tensor([x % s["kw"].shape[1] for x in pos], dtype=torch.long, device="cuda")
        rows = torch.arange(b, device="cuda")
        upd.append({"cu": torch.arange(b + 1, dtype=torch.int32, device="cuda"),
                    "pos0": torch.tensor(pos, dtype=torch.int32, device="cuda"),
                    "k": s["kw"][rows, slot].contiguous(), "v": s["vw"][rows, slot].contiguous(),
                    "w": torch.randn((c.hkv, c.block), device="cuda") * c.w_std})

    def step(i):
        s, u = sets[i % n_sets], upd[i % n_sets]
        clock.run("decode_maintenance", lambda: (
            hca.hca_compress_chunk(p, u["cu"], u["pos0"], s["cu_blocks"], 1, u["k"], u["w"], s["kw"], s["kc"],
                                   v=u["v"], vw=s["vw"], vc=s["vc"]),
            hca.hca_ring_append(p, u["cu"], u["pos0"], 1, u["k"], s["kw"], v=u["v"], vw=s["vw"])))
        clock.run("decode", lambda: hca.hca_attend_decode(p, s["seqlens"], s["cu_blocks"],
                                                          s["max_blocks"], s["q"], s["kc"], s["vc"],
                                                          s["kw"], s["vw"], workspace=ws[i % n_sets],
                                                          o=outs[i % n_sets]))

    nwarm = warm_up(torch, step, warmup, min_warm_s)
    clock.reset()
    t0 = time.perf_counter()
    for i in range(steps):
        step(nwarm + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not epilogue:
        return sets[0], wall, nwarm
    # the same decode with the fused epilogue (gate + rank-16 head mixing in
    # the merge), timed apart
    g = torch.Generator(device="cuda").manual_seed(c.seed + 31)
    gates = [torch.randn((len(x["lens"]), c.hq), generator=g, device="cuda") for x in sets]
    u = torch.randn((c.hkv, c.hq // c.hkv, EPILOGUE_RANK), generator=g, device="cuda") * 0.1
    v = torch.randn_like(u) * 0.1

    def step_epi(i):
        s, k = sets[i % n_sets], i % n_sets
        clock.run("decode_gated_vha", lambda: hca.hca_attend_decode_gated_vha(
            p, s["seqlens"], s["cu_blocks"], s["max_blocks"], s["q"], s["kc"], s["vc"], s["kw"], s["vw"],
            gate=gates[k], vha_u=u, vha_v=v, workspace=ws[k], o=outs[k]))

    for i in range(n_sets):
        step_epi(i)
    clock.pairs.pop("decode_gated_vha", None)
    for i in range(steps):
        step_epi(i)
    torch.cuda.synchronize()
    return sets[0], wall, nwarm


def measure_peaks(torch, hca):
    """Ceilings this part reaches in this run: a streaming read of a 2 GiB
    buffer (HBM) into registers and through LDS with direct loads (the
    better one is the HBM ceiling), a loop of bf16 32x32x16 matrix-core
    products on register operands, one and two wavefronts per SIMD (the
    clock of the MFMA loop comes from the shader-clock and 100 MHz
    counters), and LDS reads.  Fills MEASURED."""
    dev = "cuda"
    nbytes = 2 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.empty(4 * 2048, dtype=torch.int32, device=dev)
    clock = KernelClock(torch)
    for i in range(8):
        clock.run("stream" if i >= 2 else "warm", lambda: hca.hca_probe_stream_read(buf, 2048, sink=sink))
    torch.cuda.synchronize()
    _, t_med, _ = clock.stats_ms("stream")
    hbm_vgpr = nbytes / (t_med * 1e-3) / 1e9
    # the same bytes through LDS with the attention kernels' direct loads
    # (one workgroup per CU); the buffer is rewritten between runs so that
    # no run starts from the last-level cache
    lds_bytes = nbytes // hca.PROBE_LDS_TILE * hca.PROBE_LDS_TILE
    for i in range(6):
        buf.fill_(i)
        clock.run("stream_lds" if i >= 1 else "warm", lambda: hca.hca_probe_stream_lds(buf, 256, sink=sink))
    torch.cuda.synchronize()
    _, t_med, _ = clock.stats_ms("stream_lds")
    hbm_lds = lds_bytes / (t_med * 1e-3) / 1e9
    hbm = max(hbm_vgpr, hbm_lds)
    del buf, sink
    out = {"hbm_stream_read_gbs": round(hbm_vgpr, 1), "hbm_stream_lds_gbs": round(hbm_lds, 1),
           "hbm_stream_bytes": nbytes, "hbm_gbs": round(hbm, 1)}
    best = 0.0
    for wps in (1, 2):
        grid = 256 * wps
        iters = 40000
        msink = torch.empty(4 + 4 * grid, dtype=torch.float32, device=dev)
        name = f"mfma{wps}"
        for i in range(6):
            clock.run(name if i >= 2 else "warm", lambda: hca.hca_probe_mfma_bf16(iters, grid, sink=msink))
        torch.cuda.synchronize()
        _, t_med, _ = clock.stats_ms(name)
        tf = grid * 4 * iters * 4 * 32768 / (t_med * 1e-3) / 1e12
        cyc, ticks = float(msink[0]), float(msink[1])
        ghz = cyc / (ticks / 100e6) / 1e9 if ticks > 0 else None
        out[f"mfma_bf16_tflops_{wps}wave_per_simd"] = round(tf, 1)
        out[f"mfma_loop_clock_ghz_{wps}wave_per_simd"] = round(ghz, 3) if ghz else None
        best = max(best, tf)
    out["mfma_bf16_tflops"] = round(best, 1)
    for mode, per in ((0, 1024), (1, 512)):
        grid, iters = 1024, 5000  # four workgroups (16 wavefronts) per CU keep enough reads in flight
        lsink = torch.empty(4 * grid, dtype=torch.int32, device=dev)
        name = f"lds{mode}"
        for i in range(5):
            clock.run(name if i >= 1 else "warm", lambda: hca.hca_probe_lds_read(mode, iters, grid, sink=lsink))
        torch.cuda.synchronize()
        _, t_med, _ = clock.stats_ms(name)
        byt = grid * 4 * iters * 8 * per
        out["lds_b128_read_tbs" if mode == 0 else "lds_tr16_read_tbs"] = round(byt / (t_med * 1e-3) / 1e12, 2)
    MEASURED["hbm"] = hbm
    MEASURED["mfma"] = best
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--min-warmup-s", type=float, default=0.3,
                    help="continue the warmup until this much GPU time has run (clock ramp)")
    ap.add_argument("--workload", default="prefill_128k", choices=WORKLOADS)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode_64x128k companion")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed_1m companion of prefill_128k")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fused-epilogue, lse and backward timings of the prefill workloads")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measurement probes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build runs the HCA forward on one GPU only; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_kv_sparse_amd as hca
    from hca_workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    hca.library()  # fails loudly if libhca.so is missing

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    clock = KernelClock(torch)
    if args.workload == "dsa_decode_64x128k":
        log(f"[bench] dsa_decode_64x128k: {DSA_BATCH} x {DSA_LEN} positions, k={DSA_TOPK}, steps={args.steps}")
        inp, wall, nwarm = run_dsa(torch, hca, args, clock)
        db, df = dsa_work(inp["lens"], DSA_TOPK)
        t = clock.mean_ms("dsa_decode")
        rl = roofline("dsa_decode", "dsa_decode_64x128k", db, df, t, "hbm")
        out = {"metric": METRIC, "value": round(DSA_BATCH / (t * 1e-3), 1), "unit": "queries/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (int8 indexer)",
               "data": "synthetic (seeded random tensors of the workload's shapes)",
               "config": {"workload": "dsa_decode_64x128k", "batch": DSA_BATCH, "context": DSA_LEN, "topk": DSA_TOPK,
                          "q_heads": 64, "head_dim": 256, "indexer_dim": 128, "parallelism": "none (1 GPU)"},
               "roofline": rl, "warmup_steps_run": nwarm, "kernels": {"dsa_decode": rl}}
        if not args.no_cpu_baseline:
            log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
            out["cpu_baseline"] = cpu_baseline_dsa(inp, args.cpu_seconds)
        print(json.dumps(out), flush=True)
        return
    if not args.no_peaks:
        log("[bench] measurement probes (stream read, matrix-core loop, LDS reads)")
        peaks = measure_peaks(torch, hca)
    c = CONFIGS[args.workload]
    e = 2 if c.dtype == "bf16" else 4
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": c.dtype, "data": "synthetic (seeded random tensors of the workload's shapes)"}
    kernels = {}

    if c.chunk_pos0:
        log(f"[bench] {c.name}: chunk of {c.prefill_lens[0]} tokens at position {c.chunk_pos0}, steps={args.steps}")
        ci, wall, nwarm = run_chunk(torch, hca, c, args.steps, args.warmup, clock, args.min_warmup_s)
        result["warmup_steps_run"] = nwarm
        p0, n = ci["pos0"], ci["n"]
        pb, pf = chunk_work(c, p0, n, e)
        nblk = (p0 + n) // c.block - p0 // c.block
        cb, cf = nblk * c.hkv * (2 * c.block * c.d * e + 2 * c.d * e), nblk * c.hkv * 4 * c.block * c.d
        rb = 2 * 2 * min(n, c.ring) * c.hkv * c.d * e  # K and V rows read and written
        t_pre, t_cmp, t_app = clock.mean_ms("prefill"), clock.mean_ms("compress"), clock.mean_ms("ring_append")
        ms_step = wall * 1e3 / args.steps
        bound = "hbm" if pf / pb < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"
        kernels["prefill"] = roofline("prefill_chunk", c.name, pb, pf, t_pre, bound, clock, "prefill")
        kernels["prefill"]["mfma_frac"] = round(pf / (t_pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        kernels["prefill"]["hbm_frac"] = round(pb / (t_pre * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        kernels["compress"] = roofline("compress_chunk", c.name, cb, cf, t_cmp, "hbm", clock, "compress")
        kernels["ring_append"] = roofline("ring_append", c.name, rb, 0, t_app, "hbm", clock, "ring_append")
        result.update({"value": round(n / (ms_step * 1e-3), 1), "unit": "tokens/s",
                       "ms_per_step": round(ms_step, 4)})
        result["config"] = {"workload": c.name, "batch": 1, "chunk_tokens": n, "pos0": p0, "seq_len": p0 + n,
                            "cache_entries_before": p0 // c.block, "ring": c.ring, "q_heads": c.hq,
                            "kv_heads": c.hkv, "head_dim": c.d, "window": c.window, "block": c.block,
                            "parallelism": "none (1 GPU)"}
        result["roofline"] = kernels["prefill"]
        if not args.no_cpu_baseline:
            log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
            result["cpu_baseline"] = cpu_baseline_chunk(c, ci, args.cpu_seconds)
        del ci
        torch.cuda.empty_cache()
    elif c.has_prefill:
        log(f"[bench] {c.name}: prefill lens={list(c.prefill_lens)} steps={args.steps}")
        fields, kern = prefill_section(torch, hca, c, args, clock, extras=not args.no_extras,
                                       cpu=not args.no_cpu_baseline)
        result.update(fields)
        kernels.update(kern)

    dcfg = None
    if c.name in ("decode_64x128k", "mixed_1m"):
        dcfg = c
    elif c.name in ("prefill_8k", "prefill_128k") and not args.no_decode:
        dcfg = CONFIGS["decode_64x128k"]
    if dcfg is not None:
        log(f"[bench] {dcfg.name}: decode steps={args.steps}")
        clock.reset()
        dec, kern = decode_section(torch, hca, dcfg, args, clock, epilogue=dcfg.name == "decode_64x128k",
                                   cpu=not args.no_cpu_baseline)
        kernels.update(kern)
        if c.has_prefill:
            result["decode"] = dec
            if c.name == "mixed_1m":
                # one step = chunk prefill (pooling + attention) + the decode batch
                ms_step = result["ms_per_step"] + dec["ms_per_call"]
                ntok = sum(c.prefill_lens) + dec["batch"]
                result["value"] = round(ntok / (ms_step * 1e-3), 1)
                result["ms_per_step"] = round(ms_step, 4)
                result["unit"] = "tokens/s"
        else:
            result.update({"value": dec["queries_per_s"], "unit": "queries/s",
                           "ms_per_step": dec["ms_per_step"]})
            result["config"] = dec["config"]
            result["roofline"] = kernels["decode"]
            if "cpu_baseline" in dec:
                result["cpu_baseline"] = dec["cpu_baseline"]
    if c.name == "prefill_128k" and not args.no_mixed:
        result["mixed"] = mixed_section(torch, hca, args)
    if not args.no_peaks:
        result["measured_peaks"] = peaks
    result["kernels"] = kernels
    order = ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
             "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"]
    out = {k: result[k] for k in order if k in result}
    out.update({k: v for k, v in result.items() if k not in out})
    print(json.dumps(out), flush=True)


def prefill_section(torch, hca, c, args, clock, extras=True, cpu=True, prefix=""):
    """Time the prefill step of workload c; returns (result fields, kernel
    roofline entries named prefix + kernel)."""
    e = 2 if c.dtype == "bf16" else 4
    inp, wall, nwarm = run_prefill(torch, hca, c, args.steps, args.warmup, clock, args.min_warmup_s, extras=extras)
    lens = inp["lens"]
    pb, pf = prefill_work(c, lens, e)
    cb, cf = compress_work(c, lens, e)
    t_pre, t_cmp = clock.mean_ms("prefill"), clock.mean_ms("compress_cold")
    ms_step = wall * 1e3 / args.steps
    ntok = sum(lens)
    bound = "hbm" if pf / pb < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"
    k = {}
    k["prefill"] = roofline("prefill", c.name, pb, pf, t_pre, bound, clock, "prefill")
    k["prefill"]["mfma_frac"] = round(pf / (t_pre * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
    k["prefill"]["hbm_frac"] = round(pb / (t_pre * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    # pooling with a cold last-level cache (its own loop); in-step time beside it
    k["compress"] = roofline("compress", c.name, cb, cf, t_cmp, "hbm", clock, "compress_cold")
    k["compress"]["in_step_avg_ms"] = round(clock.mean_ms("compress"), 5)
    if clock.pairs.get("prefill_gated_vha"):
        t_epi = clock.mean_ms("prefill_gated_vha")
        # + gate logits read; + 2 mixing products per (token, column): 4 * Hq * rank flops
        eb = pb + ntok_of(lens) * c.hq * 4
        ef = pf + ntok_of(lens) * c.d * 4 * c.hq * EPILOGUE_RANK
        k["prefill_gated_vha"] = roofline("prefill_gated_vha", c.name, eb, ef, t_epi, bound, clock,
                                          "prefill_gated_vha")
        k["prefill_gated_vha"]["overhead_vs_prefill"] = round(t_epi / t_pre - 1.0, 4)
    if clock.pairs.get("backward"):
        bb, bf = backward_work(c, lens, e)
        t_bwd, t_lse = clock.mean_ms("backward"), clock.mean_ms("prefill_lse")
        bbound = "hbm" if bf / bb < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) else "mfma"
        k["backward"] = roofline("backward", c.name, bb, bf, t_bwd, bbound, clock, "backward")
        k["backward"]["mfma_frac"] = round(bf / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        k["backward"]["hbm_frac"] = round(bb / (t_bwd * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        k["backward"]["ratio_to_forward"] = round(t_bwd / t_pre, 3)
        k["prefill_lse"] = roofline("prefill_lse", c.name, pb + ntok_of(lens) * c.hq * 4, pf, t_lse, bound,
                                    clock, "prefill_lse")
        k["prefill_lse"]["overhead_vs_prefill"] = round(t_lse / t_pre - 1.0, 4)
    fields = {"value": round(ntok / (ms_step * 1e-3), 1), "unit": "tokens/s", "ms_per_step": round(ms_step, 4),
              "warmup_steps_run": nwarm,
              "config": {"workload": c.name, "batch": len(lens), "seq_len": max(lens), "q_heads": c.hq,
                         "kv_heads": c.hkv, "head_dim": c.d, "window": c.window, "block": c.block,
                         "parallelism": "none (1 GPU)"},
              "roofline": k["prefill"]}
    if cpu:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        fields["cpu_baseline"] = cpu_baseline_prefill(c, inp, args.cpu_seconds,
                                                      min_rows=2048 if max(lens) > 65536 else 0)
    del inp
    torch.cuda.empty_cache()
    return fields, {prefix + n: v for n, v in k.items()}


def decode_section(torch, hca, dcfg, args, clock, epilogue=True, cpu=True, prefix=""):
    """Time hca_attend_decode on workload dcfg (rotating caches); returns
    (decode summary, kernel roofline entries named prefix + kernel)."""
    dinp, dwall, dwarm = run_decode(torch, hca, dcfg, args.steps, args.warmup, clock, args.min_warmup_s,
                                    epilogue=epilogue)
    db, df = decode_work(dcfg, dinp["lens"], 2)
    t_dec = clock.mean_ms("decode")
    k = {"decode": roofline("decode", dcfg.name, db, df, t_dec, "hbm", clock, "decode")}
    if clock.pairs.get("decode_gated_vha"):
        t_de = clock.mean_ms("decode_gated_vha")
        k["decode_gated_vha"] = roofline("decode_gated_vha", dcfg.name, db, df, t_de, "hbm", clock,
                                         "decode_gated_vha")
        k["decode_gated_vha"]["overhead_vs_decode"] = round(t_de / t_dec - 1.0, 4)
    # the step's cache maintenance (pool the completed block, append the new
    # row): one new K, V row in and 128 ring rows + the entry per sequence
    t_mnt = clock.mean_ms("decode_maintenance")
    mb = len(dinp["lens"]) * dcfg.hkv * dcfg.d * 2 * (2 * 128 + 2 + 2 + 2)
    k["decode_maintenance"] = roofline("decode_maintenance", dcfg.name, mb, 0, t_mnt, "hbm", clock,
                                       "decode_maintenance")
    dec = {"workload": dcfg.name, "queries_per_s": round(len(dinp["lens"]) / (t_dec * 1e-3), 1),
           "unit": "queries/s", "ms_per_call": round(t_dec, 5), "batch": len(dinp["lens"]),
           "context_lens": dinp["lens"] if len(dinp["lens"]) <= 8 else f"{dinp['lens'][0]} each",
           "warmup_steps_run": dwarm, "ms_per_step": round(dwall * 1e3 / args.steps, 4),
           "config": {"workload": dcfg.name, "batch": len(dinp["lens"]), "context": dinp["lens"][0],
                      "q_heads": dcfg.hq, "kv_heads": dcfg.hkv, "head_dim": dcfg.d, "window": dcfg.window,
                      "block": dcfg.block, "parallelism": "none (1 GPU)"},
           "roofline": k["decode"]}
    if cpu:
        dec["cpu_baseline"] = cpu_baseline_decode(dcfg, dinp, min(10.0, args.cpu_seconds))
    return dec, {prefix + n: v for n, v in k.items()}


def mixed_section(torch, hca, args):
    """mixed_1m as a companion of the default run: the 32768-token chunk
    (pooling + attention) and the decode of 8 sequences at 256K-1M, one step
    = both on one stream.  Oracle baselines are left to --workload mixed_1m."""
    from hca_workloads import CONFIGS

    c = CONFIGS["mixed_1m"]
    log(f"[bench] {c.name} (companion): chunk + decode, steps={args.steps}")
    clock = KernelClock(torch)
    fields, kern = prefill_section(torch, hca, c, args, clock, extras=False, cpu=False)
    clock.reset()
    dec, dk = decode_section(torch, hca, c, args, clock, epilogue=False, cpu=False)
    ms_step = fields["ms_per_step"] + dec["ms_per_call"]
    ntok = sum(c.prefill_lens) + dec["batch"]
    return {"workload": c.name, "value": round(ntok / (ms_step * 1e-3), 1), "unit": "tokens/s",
            "ms_per_step": round(ms_step, 4), "chunk_tokens": sum(c.prefill_lens),
            "decode_context_lens": dec["context_lens"], "chunk": kern["prefill"], "compress": kern["compress"],
            "decode": dk["decode"]}


if __name__ == "__main__":
    main()
