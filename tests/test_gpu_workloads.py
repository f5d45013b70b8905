"""Parity at the five named workloads' full sizes, in the launch
configuration the benchmark times.  Pooled entries and decode outputs are
compared in full; prefill outputs on sampled rows (every block and window
boundary plus seeded random rows) that the oracle computes one by one."""
import numpy as np
import pytest
import torch

import oracle
from hca_workloads import CONFIGS, decode_inputs, prefill_inputs
from parity_util import assert_close, params_for, run_decode, run_prefill, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _prefill_case(c, n_random):
    inp = prefill_inputs(c, DEV)
    p = params_for(c)
    kc, vc, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    T = inp["lens"][0]
    cu = inp["cu_seqlens_host"]
    w = inp["w"].cpu()
    k, v = inp["k"].cpu(), inp["v"].cpu()
    kc_ref = oracle.compress(k, w, cu)
    vc_ref = oracle.compress(v, w, cu)
    dt = o.dtype
    assert_close(kc, kc_ref, dt, f"{c.name} Kc")
    assert_close(vc, vc_ref, dt, f"{c.name} Vc")
    rows = sample_rows(T, c.window, n_random, seed=c.seed)
    idx = torch.tensor(rows, device=DEV)
    q_rows = inp["q"].index_select(0, idx).cpu()
    ref = oracle.attend_prefill(q_rows, k, v, kc_ref, vc_ref, cu, c.window, rows=rows,
                                q_holds_rows_only=True)
    assert_close(o.index_select(0, idx), ref, dt, f"{c.name} O ({len(rows)} sampled rows)")
    del inp, kc, vc, o
    torch.cuda.empty_cache()


def test_workload_tiny_f32():
    c = CONFIGS["tiny_f32"]
    inp = prefill_inputs(c, DEV)
    p = params_for(c)
    kc, vc, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens_host"]
    kc_ref = oracle.compress(inp["k"].cpu(), inp["w"].cpu(), cu)
    vc_ref = oracle.compress(inp["v"].cpu(), inp["w"].cpu(), cu)
    ref = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), kc_ref, vc_ref, cu,
                                c.window)
    assert_close(kc, kc_ref, torch.float32, "tiny_f32 Kc")
    assert_close(o, ref, torch.float32, "tiny_f32 O (all rows)")


def test_workload_prefill_8k():
    _prefill_case(CONFIGS["prefill_8k"], n_random=64)


def test_workload_prefill_128k():
    _prefill_case(CONFIGS["prefill_128k"], n_random=48)


def test_workload_decode_64x128k():
    c = CONFIGS["decode_64x128k"]
    inp = decode_inputs(c, DEV)
    p = params_for(c)
    o = run_decode(p, inp)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(),
                               inp["vw"].cpu(), inp["lens"], inp["cu_blocks_host"], c.window)
    assert_close(o, ref, torch.bfloat16, "decode_64x128k O (all 64 queries)")


def test_workload_mixed_1m():
    c = CONFIGS["mixed_1m"]
    dec = decode_inputs(c, DEV)
    assert all(262144 <= L <= 1048576 for L in dec["lens"])
    p = params_for(c)
    o = run_decode(p, dec)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(dec["q"].cpu(), dec["kc"].cpu(), dec["vc"].cpu(), dec["kw"].cpu(),
                               dec["vw"].cpu(), dec["lens"], dec["cu_blocks_host"], c.window)
    assert_close(o, ref, torch.bfloat16, f"mixed_1m decode O (lens={dec['lens']})")
    del dec, o
    _prefill_case(c, n_random=64)


def test_workload_chunk_32k_at_224k():
    """The continuation chunk of the serving path at its benchmark size: the
    cache holds the 1792 entries before the chunk and a 128-slot ring; the
    chunk pools 256 more blocks and attends over 1792..2047 entries plus the
    window.  Sampled rows against the oracle's prefill of the whole 256K
    sequence (every block boundary of the chunk's first window, its first
    and last rows, seeded random rows)."""
    import compressed_kv_sparse_amd as hca
    from hca_workloads import chunk_inputs

    c = CONFIGS["chunk_32k_at_224k"]
    ci = chunk_inputs(c, DEV)
    p0, n, L, R = ci["pos0"], ci["n"], ci["length"], c.ring
    p = params_for(c)
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)  # noqa: E731
    cap, nb0 = L // 128, p0 // 128
    kc = torch.full((cap, 1, c.d), 1000.0, dtype=torch.bfloat16, device=DEV)
    vc = kc.clone()
    hca.hca_compress(p, i32([0, p0]), i32([0, nb0]), nb0, ci["k"][:p0], ci["w"], v=ci["v"][:p0],
                     kc=kc[:nb0], vc=vc[:nb0])
    slots = torch.arange(p0 - R, p0, device=DEV) % R
    kw = torch.zeros((1, R, 1, c.d), dtype=torch.bfloat16, device=DEV)
    vw = torch.zeros_like(kw)
    kw[0, slots] = ci["k"][p0 - R:p0]
    vw[0, slots] = ci["v"][p0 - R:p0]
    kch, vch = ci["k"][p0:].contiguous(), ci["v"][p0:].contiguous()
    cu, pos0, cub = i32([0, n]), i32([p0]), i32([0, cap])
    hca.hca_compress_chunk(p, cu, pos0, cub, n, kch, ci["w"], kw, kc, v=vch, vw=vw, vc=vc)
    o = hca.hca_attend_prefill_chunk(p, cu, pos0, cub, n, ci["q"], kch, vch, kc, vc, kw, vw)
    torch.cuda.synchronize()
    k, v, w = ci["k"].cpu(), ci["v"].cpu(), ci["w"].cpu()
    kc_ref = oracle.compress(k, w, [0, L])
    vc_ref = oracle.compress(v, w, [0, L])
    assert_close(kc, kc_ref, torch.bfloat16, "chunk_32k_at_224k Kc (all 2048 entries)")
    assert_close(vc, vc_ref, torch.bfloat16, "chunk_32k_at_224k Vc (all 2048 entries)")
    rel = sorted(set([0, 1, 2, 126, 127, 128, 129, n - 2, n - 1] +
                     [int(x) for x in np.random.default_rng(c.seed).choice(n, 40, replace=False)]))
    idx = torch.tensor(rel, device=DEV)
    ref = oracle.attend_prefill(ci["q"].index_select(0, idx).cpu(), k, v, kc_ref, vc_ref, [0, L], c.window,
                                rows=[p0 + r for r in rel], q_holds_rows_only=True)
    assert_close(o.index_select(0, idx), ref, torch.bfloat16, f"chunk_32k_at_224k O ({len(rel)} sampled rows)")
