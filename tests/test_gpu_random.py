"""Seeded random sweep: many small shapes through every bf16 entry point
against the oracle.  Lengths, windows, KV head counts, chunk starts and
ring sizes are drawn from a fixed generator, so the sweep is the same on
every run; each case prints its draw before the GPU calls.

The early rows of random sequences see few keys and can have |O| > 4, where
a correctly rounded bf16 value is up to 0.0156 from the exact one: the
max-abs bound applies beyond half a bf16 ulp (rel-L2 stays literal)."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import CONFIGS, decode_inputs, prefill_inputs, ring_from_raw
from parity_util import assert_close, params_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_CASES = 8


def _draw(i):
    r = np.random.default_rng(7000 + i)
    nseq = int(r.integers(1, 4))
    lens = [int(x) for x in r.integers(1, 1400, size=nseq)]
    window = int(r.choice([1, 16, 64, 127, 128, 200]))
    hkv = int(r.choice([1, 1, 2]))
    return lens, window, hkv, r


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill_and_chunk(i):
    lens, window, hkv, r = _draw(i)
    print(f"case {i}: lens={lens} W={window} Hkv={hkv}", flush=True)
    c = dataclasses.replace(CONFIGS["prefill_8k"], window=window, hkv=hkv, hq=64 * hkv)
    inp = prefill_inputs(c, DEV, lens=lens, seed=7100 + i)
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"], inp["w"],
                              v=inp["v"])
    if kc.shape[0] == 0:
        kc = torch.zeros((1, hkv, c.d), dtype=torch.bfloat16, device=DEV)
        vc = kc.clone()
    o = hca.hca_attend_prefill(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"], inp["k"],
                               inp["v"], kc, vc)
    # one chunk per sequence, drawn inside it, over the cache of the whole sequence
    cu = inp["cu_seqlens_host"]
    chunks = []
    for L in lens:
        p0 = int(r.integers(0, L))
        chunks.append((p0, int(r.integers(1, L - p0 + 1))))
    ring = max(window, 128) + int(r.integers(0, 64))
    rows = [cu[b] + p0 + j for b, (p0, n) in enumerate(chunks) for j in range(n)]
    idx = torch.tensor(rows, dtype=torch.long, device=DEV)
    ccu = torch.tensor(np.concatenate([[0], np.cumsum([n for _, n in chunks])]), dtype=torch.int32, device=DEV)
    pos0 = torch.tensor([p0 for p0, _ in chunks], dtype=torch.int32, device=DEV)
    kw = torch.stack([ring_from_raw(inp["k"][cu[b]:cu[b + 1]], chunks[b][0], ring) for b in range(len(lens))])
    vw = torch.stack([ring_from_raw(inp["v"][cu[b]:cu[b + 1]], chunks[b][0], ring) for b in range(len(lens))])
    oc = hca.hca_attend_prefill_chunk(p, ccu, pos0, inp["cu_blocks"], max(n for _, n in chunks),
                                      inp["q"][idx].contiguous(), inp["k"][idx].contiguous(),
                                      inp["v"][idx].contiguous(), kc, vc, kw.contiguous(), vw.contiguous())
    torch.cuda.synchronize()
    w = inp["w"].cpu()
    kc_ref = oracle.compress(inp["k"].cpu(), w, cu)
    vc_ref = oracle.compress(inp["v"].cpu(), w, cu)
    ref = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), kc_ref, vc_ref, cu, window)
    assert_close(o, ref, torch.bfloat16, f"case {i} prefill", beyond_rounding=True)
    assert_close(oc, ref[rows], torch.bfloat16, f"case {i} chunk {chunks}", beyond_rounding=True)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(i):
    r = np.random.default_rng(7500 + i)
    b = int(r.integers(1, 10))
    lens = [int(x) for x in r.integers(1, 40000, size=b)]
    window = int(r.choice([1, 64, 128, 300]))
    ring = window + int(r.integers(0, 100))
    hkv = int(r.choice([1, 2]))
    print(f"case {i}: lens={lens} W={window} R={ring} Hkv={hkv}", flush=True)
    c = dataclasses.replace(CONFIGS["decode_64x128k"], window=window, ring=ring, hkv=hkv, hq=64 * hkv,
                            decode_batch=b)
    inp = decode_inputs(c, DEV, lens=lens, seed=7600 + i)
    p = params_for(c)
    ws = hca.new_decode_workspace(p, b, inp["max_blocks"])
    o = hca.hca_attend_decode(p, inp["seqlens"], inp["cu_blocks"], inp["max_blocks"], inp["q"], inp["kc"],
                              inp["vc"], inp["kw"], inp["vw"], workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(), inp["vw"].cpu(),
                               lens, inp["cu_blocks_host"], window)
    assert_close(o, ref, torch.bfloat16, f"case {i} decode", beyond_rounding=True)
