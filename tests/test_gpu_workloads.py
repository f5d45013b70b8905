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
