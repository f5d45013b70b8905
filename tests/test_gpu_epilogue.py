"""GPU parity of the fused attention epilogue (hca_attend_prefill_gated_vha):
a per-head sigmoid output gate and the cross-head low-rank mixing with
identity skip, against the oracle's attention followed by its
head_mix_and_gate."""
from __future__ import annotations

import dataclasses

import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import CONFIGS, decode_inputs, prefill_inputs, ring_from_raw
from parity_util import assert_close, params_for, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(lens, hkv, seed):
    c = dataclasses.replace(CONFIGS["prefill_8k"], hkv=hkv, hq=64 * hkv)
    inp = prefill_inputs(c, DEV, lens=lens, seed=seed)
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"], inp["w"],
                              v=inp["v"])
    return c, inp, p, kc, vc


def _factors(hkv, rank, seed, scale=0.1):
    g = torch.Generator(device=DEV).manual_seed(seed)
    u = torch.randn((hkv, 64, rank), generator=g, device=DEV) * scale
    v = torch.randn((hkv, 64, rank), generator=g, device=DEV) * scale
    return u, v


def _oracle(c, inp, u=None, v=None, gate=None):
    cu = inp["cu_seqlens_host"]
    w = inp["w"].cpu()
    o = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), oracle.compress(inp["k"].cpu(), w, cu),
                              oracle.compress(inp["v"].cpu(), w, cu), cu, c.window)
    return oracle.head_mix_and_gate(o, None if u is None else u.cpu(), None if v is None else v.cpu(),
                                    None if gate is None else gate.cpu())


@pytest.mark.parametrize("lens,hkv,rank,with_gate", [
    ([300, 1000], 1, 8, False),
    ([513], 1, 32, False),        # two rank steps
    ([700, 129], 1, 1, True),
    ([1000], 1, 16, True),
    ([400, 77], 2, 24, True),     # two KV heads: mixing stays inside each group
])
def test_gated_vha_bf16(lens, hkv, rank, with_gate):
    c, inp, p, kc, vc = _case(lens, hkv, seed=401)
    u, v = _factors(hkv, rank, seed=402)
    gate = None
    if with_gate:
        g = torch.Generator(device=DEV).manual_seed(403)
        gate = torch.randn((sum(lens), 64 * hkv), generator=g, device=DEV) * 2
    o = hca.hca_attend_prefill_gated_vha(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                         inp["k"], inp["v"], kc, vc, gate=gate, vha_u=u, vha_v=v)
    torch.cuda.synchronize()
    # the first rows of a sequence can have |O| > 4 (few visible keys), where
    # bf16 rounding alone reaches 0.0156
    assert_close(o, _oracle(c, inp, u, v, gate), torch.bfloat16,
                 f"gated VHA lens={lens} Hkv={hkv} rank={rank} gate={with_gate}", beyond_rounding=True)


def test_gate_only():
    c, inp, p, kc, vc = _case([900, 64], 1, seed=411)
    g = torch.Generator(device=DEV).manual_seed(412)
    gate = torch.randn((964, 64), generator=g, device=DEV) * 3
    o = hca.hca_attend_prefill_gated_vha(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                         inp["k"], inp["v"], kc, vc, gate=gate)
    torch.cuda.synchronize()
    assert_close(o, _oracle(c, inp, gate=gate), torch.bfloat16, "gate only", beyond_rounding=True)


def test_zero_mixing_is_plain_prefill():
    """U = 0: the epilogue adds exact zeros, so its separate store path must
    reproduce the plain kernel's output bit for bit."""
    c, inp, p, kc, vc = _case([777, 130], 1, seed=421)
    u, v = _factors(1, 8, seed=422)
    u.zero_()
    o_mix = hca.hca_attend_prefill_gated_vha(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                             inp["k"], inp["v"], kc, vc, vha_u=u, vha_v=v)
    o_plain = hca.hca_attend_prefill(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"], inp["k"],
                                     inp["v"], kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(o_mix.view(torch.int16), o_plain.view(torch.int16))


@pytest.mark.parametrize("name,n_random", [("prefill_8k", None), ("prefill_128k", 48)])
def test_gated_vha_workload(name, n_random):
    """The fused epilogue (gate + rank-16 mixing, gate logits N(0, 1), factors
    of standard deviation 0.1, as the benchmark times it) at the workload's
    full size and launch configuration: every row at 8K, sampled rows (the
    key-set boundaries plus seeded random rows) at 128K.  The mixing and the
    gate act within one row, so the oracle's prefill of the sampled rows
    followed by its mixing gives those rows' exact outputs."""
    c = CONFIGS[name]
    inp = prefill_inputs(c, DEV)
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"], inp["w"],
                              v=inp["v"])
    u, v = _factors(c.hkv, 16, seed=451)
    T = inp["lens"][0]
    g = torch.Generator(device=DEV).manual_seed(452)
    gate = torch.randn((T, c.hq), generator=g, device=DEV)
    o = hca.hca_attend_prefill_gated_vha(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                         inp["k"], inp["v"], kc, vc, gate=gate, vha_u=u, vha_v=v)
    torch.cuda.synchronize()
    cu = inp["cu_seqlens_host"]
    w = inp["w"].cpu()
    k, vv = inp["k"].cpu(), inp["v"].cpu()
    kc_ref, vc_ref = oracle.compress(k, w, cu), oracle.compress(vv, w, cu)
    if n_random is None:
        rows = list(range(T))
        ref = oracle.attend_prefill(inp["q"].cpu(), k, vv, kc_ref, vc_ref, cu, c.window)
    else:
        rows = sample_rows(T, c.window, n_random, seed=c.seed)
        q_rows = inp["q"].index_select(0, torch.tensor(rows, device=DEV)).cpu()
        ref = oracle.attend_prefill(q_rows, k, vv, kc_ref, vc_ref, cu, c.window, rows=rows, q_holds_rows_only=True)
    idx = torch.tensor(rows, device=DEV)
    ref = oracle.head_mix_and_gate(ref, u.cpu(), v.cpu(), gate.index_select(0, idx).cpu())
    assert_close(o.index_select(0, idx), ref, torch.bfloat16, f"{name} gated VHA rank 16 ({len(rows)} rows)",
                 beyond_rounding=True)
    del inp, o, gate
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens,rank,with_gate", [
    ([131072] * 4 + [1, 200, 5000], 16, True),    # several splits per sequence, short ones with one
    ([70000, 3000], 32, False),
    ([777], 1, True),
])
def test_decode_gated_vha(lens, rank, with_gate):
    c = dataclasses.replace(CONFIGS["decode_64x128k"], decode_batch=len(lens))
    inp = decode_inputs(c, DEV, lens=lens, seed=431)
    p = params_for(c)
    u, v = _factors(1, rank, seed=432)
    gate = None
    if with_gate:
        g = torch.Generator(device=DEV).manual_seed(433)
        gate = torch.randn((len(lens), 64), generator=g, device=DEV) * 2
    o = hca.hca_attend_decode_gated_vha(p, inp["seqlens"], inp["cu_blocks"], inp["max_blocks"], inp["q"], inp["kc"],
                                        inp["vc"], inp["kw"], inp["vw"], gate=gate, vha_u=u, vha_v=v)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(), inp["vw"].cpu(),
                               lens, inp["cu_blocks_host"], c.window)
    ref = oracle.head_mix_and_gate(ref, u.cpu(), v.cpu(), None if gate is None else gate.cpu())
    # a 1-token sequence's output is one value row, mixed: |O| passes 4, where
    # bf16 rounding alone reaches 0.0156
    assert_close(o, ref, torch.bfloat16, f"decode gated VHA lens={lens[:3]} rank={rank} gate={with_gate}",
                 beyond_rounding=True)


def test_chunk_gated_vha():
    """A chunk at position 1500 of a 2600-token sequence with the epilogue:
    rows 1500.. of the oracle's whole-sequence prefill, mixed and gated."""
    c, inp, p, kc, vc = _case([2600], 1, seed=441)
    p0, n, R = 1500, 1100, 128
    u, v = _factors(1, 16, seed=442)
    g = torch.Generator(device=DEV).manual_seed(443)
    gate = torch.randn((n, 64), generator=g, device=DEV) * 2
    kw = ring_from_raw(inp["k"], p0, R)[None].contiguous()
    vw = ring_from_raw(inp["v"], p0, R)[None].contiguous()
    i32 = lambda x: torch.tensor(x, dtype=torch.int32, device=DEV)  # noqa: E731
    sl = slice(p0, p0 + n)
    o = hca.hca_attend_prefill_chunk_gated_vha(p, i32([0, n]), i32([p0]), inp["cu_blocks"], n,
                                               inp["q"][sl].contiguous(), inp["k"][sl].contiguous(),
                                               inp["v"][sl].contiguous(), kc, vc, kw, vw, gate=gate, vha_u=u, vha_v=v)
    torch.cuda.synchronize()
    full = _oracle(c, inp)
    ref = oracle.head_mix_and_gate(full[p0:p0 + n], u.cpu(), v.cpu(), gate.cpu())
    assert_close(o, ref, torch.bfloat16, "chunk gated VHA")
