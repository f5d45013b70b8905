"""GPU parity: the HIP path through the C ABI against the float64 oracle,
element by element, at sizes the oracle finishes in seconds that still span
several key tiles and ragged tails, plus edge cases and invariants."""
import dataclasses

import numpy as np
import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import CONFIGS, decode_inputs, prefill_inputs, ring_from_raw
from parity_util import assert_close, params_for, run_decode, run_prefill, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16 = CONFIGS["prefill_8k"]


def cfg(base, **kw):
    return dataclasses.replace(base, **kw)


def oracle_prefill(inp, window, rows=None, kc=None, vc=None):
    cu = inp["cu_seqlens_host"]
    w = inp["w"].cpu()
    kc_ref = oracle.compress(inp["k"].cpu(), w, cu) if kc is None else kc
    vc_ref = oracle.compress(inp["v"].cpu(), w, cu) if vc is None else vc
    o = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), kc_ref, vc_ref, cu,
                              window, rows=rows)
    return kc_ref, vc_ref, o


# ---------------------------------------------------------------------------
# pooling
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,lens,hkv,d,dtype", [
    ("tiny_f32", [512], 1, 64, "f32"),
    ("f32_varlen_gqa", [300, 0, 129, 1000], 2, 64, "f32"),
    ("bf16_varlen", [700, 130, 5, 256, 0, 128], 1, 512, "bf16"),
    ("bf16_hkv2_d128", [1000, 383], 2, 128, "bf16"),
    ("bf16_d1024", [640], 1, 1024, "bf16"),
])
def test_compress(name, lens, hkv, d, dtype):
    c = cfg(BF16, dtype=dtype, hkv=hkv, hq=hkv, d=d, rms=(dtype == "bf16"))
    inp = prefill_inputs(c, DEV, lens=lens, seed=11)
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"],
                              inp["w"], v=inp["v"])
    torch.cuda.synchronize()
    cu = inp["cu_seqlens_host"]
    kc_ref = oracle.compress(inp["k"].cpu(), inp["w"].cpu(), cu)
    vc_ref = oracle.compress(inp["v"].cpu(), inp["w"].cpu(), cu)
    assert kc.shape == kc_ref.shape
    assert_close(kc, kc_ref, kc.dtype, f"{name} Kc")
    assert_close(vc, vc_ref, vc.dtype, f"{name} Vc")


def test_compress_keys_only_and_constant_blocks():
    """v = NULL pools K alone; rows constant within a block pool to that row
    exactly (the weights sum to one, so the bf16 value is reproduced)."""
    c = cfg(BF16, hkv=1, hq=64)
    inp = prefill_inputs(c, DEV, lens=[128 * 6], seed=12)
    base = torch.randn(6, 1, 512, device=DEV).to(torch.bfloat16)
    k = base.repeat_interleave(128, dim=0).contiguous()
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], 6, k, inp["w"] * 3)
    assert vc is None
    torch.cuda.synchronize()
    assert torch.equal(kc, base), (kc.float() - base.float()).abs().max()


# ---------------------------------------------------------------------------
# prefill attention
# ---------------------------------------------------------------------------
def test_prefill_tiny_f32_full():
    """Workload 'tiny_f32' in full (B=1, T=512, Hq=4, Hkv=1, d=64, W=64)."""
    c = CONFIGS["tiny_f32"]
    inp = prefill_inputs(c, DEV)
    p = params_for(c)
    kc, vc, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    kc_ref, vc_ref, o_ref = oracle_prefill(inp, c.window)
    assert_close(kc, kc_ref, torch.float32, "tiny Kc")
    assert_close(o, o_ref, torch.float32, "tiny O")


@pytest.mark.parametrize("lens,hq,hkv,d,window", [
    ([300, 0, 129, 1000], 4, 2, 64, 64),
    ([257, 31], 6, 3, 100, 300),
    ([200], 2, 1, 1024, 1),
])
def test_prefill_f32_shapes(lens, hq, hkv, d, window):
    c = cfg(CONFIGS["tiny_f32"], hq=hq, hkv=hkv, d=d, window=window)
    # pooling needs d % 64 == 0; otherwise the entries are drawn as inputs
    inp = prefill_inputs(c, DEV, lens=lens, seed=21, kc_random=bool(d % 64))
    p = params_for(c)
    if d % 64:
        _, _, o = run_prefill(p, inp, inp["kc"], inp["vc"])
        kc_ref, vc_ref = inp["kc"].cpu(), inp["vc"].cpu()
    else:
        _, _, o = run_prefill(p, inp)
        kc_ref = vc_ref = None
    torch.cuda.synchronize()
    _, _, o_ref = oracle_prefill(inp, window, kc=kc_ref, vc=vc_ref)
    assert_close(o, o_ref, torch.float32, f"f32 lens={lens} W={window}")


@pytest.mark.parametrize("lens,window,hkv", [
    ([700], 128, 1),                       # several tiles, odd length (lone last position)
    ([130, 5, 256, 1, 0, 383], 128, 1),    # varlen with empty and 1-token sequences
    ([600, 77], 64, 1),                    # W < 127: part of the current block is invisible
    ([520], 1, 1),                         # window of one token
    ([450], 300, 1),                       # window longer than a block
    ([300, 260], 128, 2),                  # two KV heads, 128 query heads
])
def test_prefill_bf16(lens, window, hkv):
    c = cfg(BF16, window=window, hkv=hkv, hq=64 * hkv)
    inp = prefill_inputs(c, DEV, lens=lens, seed=31)
    p = params_for(c)
    kc, vc, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    kc_ref, vc_ref, o_ref = oracle_prefill(inp, window)
    assert_close(kc, kc_ref, torch.bfloat16, f"lens={lens} Kc")
    # W=1: a row often follows its own raw token, |O| reaches 4 and more
    assert_close(o, o_ref, torch.bfloat16, f"lens={lens} W={window} O", beyond_rounding=window == 1)


def test_prefill_bf16_attention_only():
    """Attention alone, with compressed entries drawn as inputs."""
    c = cfg(BF16)
    inp = prefill_inputs(c, DEV, lens=[1100, 300], seed=41, kc_random=True)
    p = params_for(c)
    _, _, o = run_prefill(p, inp, inp["kc"], inp["vc"])
    torch.cuda.synchronize()
    _, _, o_ref = oracle_prefill(inp, c.window, kc=inp["kc"].cpu(), vc=inp["vc"].cpu())
    assert_close(o, o_ref, torch.bfloat16, "attention-only O")


def test_prefill_bf16_headroom_fallback():
    """Scores that climb steeply inside each 128-token run: for rows whose
    first key tile holds only low scores, later tiles exceed the row's
    reference max by far more than 32 (log2 units), which sends their
    workgroups through the exact two-pass schedule.  All rows must match."""
    c = cfg(BF16)
    T = 700
    inp = prefill_inputs(c, DEV, lens=[T], seed=51)
    u = inp["q"][0, 0].float()                      # one unit-RMS direction
    ramp = 0.015 * (torch.arange(T, device=DEV) % 128).float()
    inp["q"] = u.expand(T, 64, 512).to(torch.bfloat16).contiguous()
    inp["k"] = (ramp[:, None, None] * u).to(torch.bfloat16).contiguous()
    p = params_for(c)
    kc, vc, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    # rows 60..127: first tile max <= 0.47 * 32.65, their own key >= 0.9 * 32.65
    sc = (inp["k"][:, 0].float() @ u) / 512 ** 0.5 * 1.4427
    assert (sc[127] - sc[:32].max()).item() > 40
    _, _, o_ref = oracle_prefill(inp, c.window)
    assert_close(o, o_ref, torch.bfloat16, "fallback O")


def test_prefill_constant_values():
    """All visible values equal c: every output equals c (bf16 rounding)."""
    c = cfg(BF16)
    inp = prefill_inputs(c, DEV, lens=[513, 200], seed=61)
    cvec = torch.linspace(-2, 2, 512, device=DEV).to(torch.bfloat16)
    inp["v"] = cvec.expand_as(inp["v"]).contiguous()
    p = params_for(c)
    _, _, o = run_prefill(p, inp)
    torch.cuda.synchronize()
    err = (o.float() - cvec.float()).abs().max().item()
    ulp = cvec.float().abs().max().item() * 2 ** -7
    assert err <= ulp, (err, ulp)


def test_prefill_deterministic():
    c = cfg(BF16)
    inp = prefill_inputs(c, DEV, lens=[900, 131], seed=71)
    p = params_for(c)
    _, _, o1 = run_prefill(p, inp)
    _, _, o2 = run_prefill(p, inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("lens,window,ring,hkv", [
    ([1, 127, 128, 129, 1000, 4097], 128, 128, 1),
    ([5000, 300, 64], 64, 200, 1),          # ring longer than the window
    ([2000, 1], 300, 300, 2),               # window longer than a block, two KV heads
    ([70000], 128, 128, 1),                 # one long context: many splits
])
def test_decode_bf16(lens, window, ring, hkv):
    c = cfg(CONFIGS["decode_64x128k"], window=window, ring=ring, hkv=hkv, hq=64 * hkv)
    inp = decode_inputs(c, DEV, lens=lens, seed=81)
    p = params_for(c)
    o = run_decode(p, inp)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(),
                               inp["vw"].cpu(), lens, inp["cu_blocks_host"], window)
    assert_close(o, ref, torch.bfloat16, f"decode lens={lens}")


@pytest.mark.parametrize("lens,hq,hkv,d,window,ring", [
    ([1, 200, 5000], 4, 2, 64, 64, 64),
    ([333, 129], 8, 1, 256, 100, 128),
])
def test_decode_f32(lens, hq, hkv, d, window, ring):
    c = cfg(CONFIGS["tiny_f32"], hq=hq, hkv=hkv, d=d, window=window, ring=ring, decode_batch=len(lens))
    inp = decode_inputs(c, DEV, lens=lens, seed=91)
    p = params_for(c)
    o = run_decode(p, inp)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(),
                               inp["vw"].cpu(), lens, inp["cu_blocks_host"], window)
    assert_close(o, ref, torch.float32, f"f32 decode lens={lens}")


def test_decode_workspace_reuse_and_determinism():
    """One workspace serves many calls whatever it holds (it is filled with
    garbage first), and the split merge is bitwise repeatable."""
    c = CONFIGS["decode_64x128k"]
    inp = decode_inputs(c, DEV, lens=[3000, 9000, 20000], seed=101)
    p = params_for(c)
    ws = hca.new_decode_workspace(p, 3, inp["max_blocks"])
    ws.fill_(0x7f)
    o1 = run_decode(p, inp, ws).clone()
    o2 = run_decode(p, inp, ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(),
                               inp["vw"].cpu(), inp["lens"], inp["cu_blocks_host"], c.window)
    assert_close(o1, ref, torch.bfloat16, "decode with a reused, garbage-filled workspace")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_equals_last_prefill_row(dtype):
    """decode(L) == prefill row L-1 for a cache built from the same tokens."""
    if dtype == "bf16":
        c = cfg(BF16)
    else:
        c = cfg(CONFIGS["tiny_f32"], hq=4, hkv=2, d=64, window=64)
    lens = [1000, 128, 77]
    inp = prefill_inputs(c, DEV, lens=lens, seed=111)
    p = params_for(c)
    kc, vc, o_pre = run_prefill(p, inp)
    cu = inp["cu_seqlens_host"]
    ring = max(c.window, 128)
    kw = torch.stack([ring_from_raw(inp["k"][cu[b]:cu[b + 1]], lens[b], ring) for b in range(3)])
    vw = torch.stack([ring_from_raw(inp["v"][cu[b]:cu[b + 1]], lens[b], ring) for b in range(3)])
    rows = [int(cu[b + 1] - 1) for b in range(3)]
    dec = {"lens": lens, "seqlens": torch.tensor(lens, dtype=torch.int32, device=DEV),
           "cu_blocks": inp["cu_blocks"], "max_blocks": max(l // 128 for l in lens),
           "q": inp["q"][rows].contiguous(), "kc": kc, "vc": vc, "kw": kw.contiguous(),
           "vw": vw.contiguous()}
    o_dec = run_decode(p, dec)
    torch.cuda.synchronize()
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # both sides are rounded to bf16: they may differ by one bf16 step
    assert_close(o_dec, to_np(o_pre[rows]), dt, "decode vs prefill row (GPU)", beyond_rounding=True)
    _, _, o_ref = oracle_prefill(inp, c.window, rows=rows)
    assert_close(o_dec, o_ref, dt, "decode vs oracle prefill row")


def _decode_splits(p, batch, max_blocks):
    """Key splits per (sequence, KV head), read back from the workspace size
    the library asks for: two fp32 [splits, 64] arrays (m, l; each rounded
    up to 256 bytes) plus the bf16 partial outputs [splits, 64, 512] per
    unit.  The test needs it to place its score ramps inside each split."""
    ws = hca.hca_decode_workspace_bytes(p, batch, max_blocks)
    per_split = 2 * 64 * 4 + 64 * 512 * 2  # unit count * 64 * 4 is a multiple of 256 here
    assert ws % (batch * per_split) == 0, ws
    return ws // (batch * per_split)


@pytest.mark.parametrize("lens", [
    [131035] * 32 + [131072] * 32,   # 64 sequences, a few splits each; half the rings wrap
    [1048575],                       # one long context: many two-tile splits, a wrapped ring
], ids=["b64", "b1_1m"])
def test_decode_bf16_headroom_fallback(lens):
    """Scores that climb by more than 40 (log2 units) inside every key split
    of the decode kernel: each split's first tile holds only low scores, so
    its single-pass schedule is abandoned and the split reruns in the exact
    two-pass one (row max, then weights <= 1).  Every output must match."""
    c = cfg(CONFIGS["decode_64x128k"], decode_batch=len(lens))
    inp = decode_inputs(c, DEV, lens=lens, seed=131)
    p = params_for(c)
    B, R = len(lens), c.ring
    max_blocks = inp["max_blocks"]
    splits = _decode_splits(p, B, max_blocks)
    ntiles = (max_blocks + c.window + 31) // 32
    tps = -(-ntiles // splits)
    assert tps >= 2, (ntiles, splits)  # a one-tile split can never restart
    span = 32 * tps  # keys per split
    # slope per key so that a split's last tile max beats its first tile max
    # by 40 log2 units: k = a(slot) u, q = u, score = a 512 / sqrt(512) log2(e)
    lg = 512 ** 0.5 * 1.4426950408889634
    slope = 40.0 / (lg * (span - 32))
    u = inp["q"][0, 0].float()
    u = u / u.pow(2).mean().sqrt()
    inp["q"] = u.expand(B, 64, 512).to(torch.bfloat16).contiguous()
    cub = inp["cu_blocks_host"]
    kc = inp["kc"].clone()
    kw = inp["kw"].clone()
    for b, L in enumerate(lens):
        nc = L // 128
        lo = L - min(c.window, L)
        a_c = slope * (torch.arange(nc, device=DEV) % span).float()
        kc[int(cub[b]):int(cub[b]) + nc, 0] = (a_c[:, None] * u).to(torch.bfloat16)
        pos = torch.arange(lo, L, device=DEV)
        a_r = slope * ((nc + pos - lo) % span).float()
        kw[b, pos % R, 0] = (a_r[:, None] * u).to(torch.bfloat16)
    inp["kc"], inp["kw"] = kc.contiguous(), kw.contiguous()
    # the ramp as the kernel sees it (sequence 0, head 0): in every split some
    # later tile's max exceeds the first tile's max by more than 32
    L0, nc0 = lens[0], lens[0] // 128
    keys = torch.cat([kc[int(cub[0]):int(cub[0]) + nc0, 0].float(),
                      kw[0, torch.arange(L0 - min(c.window, L0), L0, device=DEV) % R, 0].float()])
    sc = (keys @ inp["q"][0, 0].float()) / 512 ** 0.5 * 1.4426950408889634
    nk = sc.shape[0]
    for s0 in range(0, nk, span):
        seg = sc[s0:min(nk, s0 + span)]
        if seg.shape[0] > 32:
            assert (seg[32:].max() - seg[:32].max()).item() > 32, s0
    o = run_decode(p, inp)
    torch.cuda.synchronize()
    ref = oracle.attend_decode(inp["q"].cpu(), inp["kc"].cpu(), inp["vc"].cpu(), inp["kw"].cpu(),
                               inp["vw"].cpu(), lens, cub, c.window)
    assert_close(o, ref, torch.bfloat16, f"decode fallback B={B} splits={splits} tiles/split={tps}")
