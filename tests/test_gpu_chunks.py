"""GPU parity of the serving path: chunks of new tokens over an existing cache
and decode steps with cache maintenance (hca_compress_chunk,
hca_attend_prefill_chunk, hca_ring_append).

The reference is always the whole sequence: a chunk's output must equal rows
pos0 .. pos0+n-1 of the oracle's prefill over the full sequence, the entries
pooled from a chunk must equal the oracle's pooling of the full sequence, and
the ring after an append must hold exactly the last ring_cap raw rows.
"""
from __future__ import annotations

import dataclasses

import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import CONFIGS, prefill_inputs, ring_from_raw
from parity_util import assert_close, params_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF16 = CONFIGS["prefill_8k"]
SENTINEL = 1000.0  # cache entries a call must not touch


def cfg(base, **kw):
    return dataclasses.replace(base, **kw)


def i32(x):
    return torch.tensor(list(x), dtype=torch.int32, device=DEV)


class Scenario:
    """Full sequences plus one chunk [pos0_b, pos0_b + n_b) of each, with the
    cache state a server holds when the chunk arrives: entries of the blocks
    completed before pos0_b and a ring of the raw rows before pos0_b."""

    def __init__(self, c, lens, chunks, seed, ring):
        self.c, self.lens, self.ring = c, list(lens), ring
        self.inp = prefill_inputs(c, DEV, lens=lens, seed=seed)
        self.p = params_for(c)
        cu = self.inp["cu_seqlens_host"]
        self.cu = cu
        self.pos0 = [p for p, _ in chunks]
        self.n = [n for _, n in chunks]
        assert all(p + n <= L for (p, n), L in zip(chunks, lens))
        self.rows = [cu[b] + self.pos0[b] + i for b in range(len(lens)) for i in range(self.n[b])]
        idx = torch.tensor(self.rows, dtype=torch.long, device=DEV)
        self.q = self.inp["q"][idx].contiguous()
        self.k = self.inp["k"][idx].contiguous()
        self.v = self.inp["v"][idx].contiguous()
        ccu = [0]
        for n in self.n:
            ccu.append(ccu[-1] + n)
        self.ccu = i32(ccu)
        self.dpos0 = i32(self.pos0)
        self.cub = self.inp["cu_blocks"]
        self.cub_host = self.inp["cu_blocks_host"]
        # full pooling on the GPU (the cache a server would hold after the whole sequence)
        self.kc_full, self.vc_full = hca.hca_compress(self.p, self.inp["cu_seqlens"], self.cub,
                                                      self.inp["total_blocks"], self.inp["k"], self.inp["w"],
                                                      v=self.inp["v"])
        if self.kc_full.shape[0] == 0:  # no complete block anywhere: keep one unused entry
            self.kc_full = torch.full((1, c.hkv, c.d), SENTINEL, dtype=self.kc_full.dtype, device=DEV)
            self.vc_full = self.kc_full.clone()
        # cache at chunk arrival: entries of blocks < floor(pos0/128) valid, the rest a sentinel
        self.kc = self.kc_full.clone()
        self.vc = self.vc_full.clone()
        for b in range(len(lens)):
            j0 = self.pos0[b] // 128
            self.kc[self.cub_host[b] + j0: self.cub_host[b + 1]] = SENTINEL
            self.vc[self.cub_host[b] + j0: self.cub_host[b + 1]] = SENTINEL
        self.kw = torch.stack([ring_from_raw(self.inp["k"][cu[b]:cu[b + 1]], self.pos0[b], ring)
                               for b in range(len(lens))]).contiguous()
        self.vw = torch.stack([ring_from_raw(self.inp["v"][cu[b]:cu[b + 1]], self.pos0[b], ring)
                               for b in range(len(lens))]).contiguous()

    def compress_chunk(self):
        hca.hca_compress_chunk(self.p, self.ccu, self.dpos0, self.cub, max(self.n), self.k, self.inp["w"],
                               self.kw, self.kc, v=self.v, vw=self.vw, vc=self.vc)

    def attend(self):
        return hca.hca_attend_prefill_chunk(self.p, self.ccu, self.dpos0, self.cub, max(self.n), self.q,
                                            self.k, self.v, self.kc, self.vc, self.kw, self.vw)

    def append(self):
        hca.hca_ring_append(self.p, self.ccu, self.dpos0, max(self.n), self.k, self.kw, v=self.v, vw=self.vw)

    def oracle_rows(self):
        cu = self.cu
        w = self.inp["w"].cpu()
        kc = oracle.compress(self.inp["k"].cpu(), w, cu)
        vc = oracle.compress(self.inp["v"].cpu(), w, cu)
        return oracle.attend_prefill(self.inp["q"].cpu(), self.inp["k"].cpu(), self.inp["v"].cpu(), kc, vc, cu,
                                     self.c.window, rows=self.rows)

    def completed(self, b):
        """Entry indices (global) pooled from sequence b's chunk."""
        lo = self.pos0[b] // 128
        hi = (self.pos0[b] + self.n[b]) // 128
        return range(self.cub_host[b] + lo, self.cub_host[b] + hi)


BF16_CASES = [
    # lens, chunks (pos0, n), window, ring
    ([300], [(0, 300)], 128, 128),                       # pos0 = 0: a plain prefill
    ([2], [(1, 1)], 128, 128),                           # second token alone
    ([400], [(5, 200)], 128, 128),                       # chunk inside the first window
    ([700], [(127, 300)], 128, 128),                     # starts on a block's last token
    ([700], [(128, 257)], 128, 200),                     # starts a block, ring longer than the window
    ([700], [(129, 1)], 128, 128),
    ([5000], [(4001, 777)], 128, 128),                   # odd start, chunk inside the sequence
    ([3000, 260, 1500], [(1024, 1976), (255, 5), (1, 1499)], 128, 128),  # ragged batch
    ([2600], [(2000, 600)], 64, 128),                    # window 64
    ([2600], [(1900, 700)], 300, 300),                   # window longer than a block
]


@pytest.mark.parametrize("lens,chunks,window,ring", BF16_CASES)
def test_chunk_bf16(lens, chunks, window, ring):
    c = cfg(BF16, window=window)
    sc = Scenario(c, lens, chunks, seed=301, ring=ring)
    ring0_k = sc.kw.clone()
    sc.compress_chunk()
    torch.cuda.synchronize()
    for b in range(len(lens)):
        got = list(sc.completed(b))
        if got:
            idx = torch.tensor(got, dtype=torch.long, device=DEV)
            # same pooling arithmetic, row order and column slices as hca_compress
            # (under 128 candidate blocks both use 64-column slices): identical bits
            assert torch.equal(sc.kc[idx].view(torch.int16), sc.kc_full[idx].view(torch.int16))
            assert torch.equal(sc.vc[idx].view(torch.int16), sc.vc_full[idx].view(torch.int16))
        after = torch.arange(sc.cub_host[b] + (sc.pos0[b] + sc.n[b]) // 128, sc.cub_host[b + 1], device=DEV)
        assert bool((sc.kc[after] == SENTINEL).all()), "entries past the chunk were written"
    o = sc.attend()
    torch.cuda.synchronize()
    assert torch.equal(sc.kw, ring0_k), "attention must not write the ring"
    assert_close(o, sc.oracle_rows(), torch.bfloat16, f"chunk lens={lens} chunks={chunks} W={window}")
    sc.append()
    torch.cuda.synchronize()
    for b in range(len(lens)):
        want = ring_from_raw(sc.inp["k"][sc.cu[b]:sc.cu[b + 1]], sc.pos0[b] + sc.n[b], ring)
        assert torch.equal(sc.kw[b], want), f"ring of sequence {b} after the append"
        want = ring_from_raw(sc.inp["v"][sc.cu[b]:sc.cu[b + 1]], sc.pos0[b] + sc.n[b], ring)
        assert torch.equal(sc.vw[b], want)


@pytest.mark.parametrize("lens,chunks,hq,hkv,d,window,ring", [
    ([600, 300], [(130, 400), (64, 1)], 4, 2, 64, 64, 128),
    ([900], [(255, 645)], 8, 1, 128, 200, 256),
])
def test_chunk_f32(lens, chunks, hq, hkv, d, window, ring):
    c = cfg(CONFIGS["tiny_f32"], hq=hq, hkv=hkv, d=d, window=window)
    sc = Scenario(c, lens, chunks, seed=303, ring=ring)
    sc.compress_chunk()
    o = sc.attend()
    sc.append()
    torch.cuda.synchronize()
    assert_close(o, sc.oracle_rows(), torch.float32, f"f32 chunk lens={lens} chunks={chunks}")
    for b in range(len(lens)):
        got = list(sc.completed(b))
        if got:
            idx = torch.tensor(got, dtype=torch.long, device=DEV)
            assert torch.equal(sc.kc[idx], sc.kc_full[idx])


def test_chunked_prefill_equals_whole():
    """One 2500-token sequence fed as chunks of 700, 800, 1 and 999 tokens:
    every row matches the oracle's prefill of the whole sequence, and the cache
    ends as the whole sequence's pooling plus its last raw rows."""
    c = cfg(BF16)
    L, ring = 2500, 128
    inp = prefill_inputs(c, DEV, lens=[L], seed=307)
    p = params_for(c)
    kc = torch.full((L // 128, 1, 512), SENTINEL, dtype=torch.bfloat16, device=DEV)
    vc = kc.clone()
    kw = torch.zeros((1, ring, 1, 512), dtype=torch.bfloat16, device=DEV)
    vw = kw.clone()
    cub = i32([0, L // 128])
    outs = []
    pos = 0
    for n in (700, 800, 1, 999):
        sl = slice(pos, pos + n)
        q, k, v = inp["q"][sl].contiguous(), inp["k"][sl].contiguous(), inp["v"][sl].contiguous()
        cu, p0 = i32([0, n]), i32([pos])
        hca.hca_compress_chunk(p, cu, p0, cub, n, k, inp["w"], kw, kc, v=v, vw=vw, vc=vc)
        outs.append(hca.hca_attend_prefill_chunk(p, cu, p0, cub, n, q, k, v, kc, vc, kw, vw))
        hca.hca_ring_append(p, cu, p0, n, k, kw, v=v, vw=vw)
        pos += n
    torch.cuda.synchronize()
    o = torch.cat(outs)
    kc_full, vc_full = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"],
                                        inp["w"], v=inp["v"])
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), kc_full.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc_full.view(torch.int16))
    assert torch.equal(kw[0], ring_from_raw(inp["k"], L, ring))
    w = inp["w"].cpu()
    cuh = inp["cu_seqlens_host"]
    ref = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), oracle.compress(inp["k"].cpu(), w, cuh),
                                oracle.compress(inp["v"].cpu(), w, cuh), cuh, c.window)
    # all 2500 rows, the first ones included: a row that sees a few raw keys
    # can have |O| > 4, where bf16 rounding alone reaches 0.0156
    assert_close(o, ref, torch.bfloat16, "chunked prefill of 2500 tokens", beyond_rounding=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_steps_with_cache_maintenance(dtype):
    """A serving loop: three sequences at lengths 250, 1000 and 60 take 12
    decode steps each (pooling the block a new token completes, appending it
    to the ring, attending).  Sequences 0 and 1 cross block ends (positions
    255 and 1023).  Every step matches the oracle's prefill row of the whole
    sequence."""
    if dtype == "bf16":
        c = cfg(BF16)
    else:
        c = cfg(CONFIGS["tiny_f32"], hq=4, hkv=1, d=64, window=100)
    steps, L0, ring = 12, [250, 1000, 60], 128
    lens = [l + steps for l in L0]
    inp = prefill_inputs(c, DEV, lens=lens, seed=311)
    p = params_for(c)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cu = inp["cu_seqlens_host"]
    cub, cubh = inp["cu_blocks"], inp["cu_blocks_host"]
    kc_full, vc_full = hca.hca_compress(p, inp["cu_seqlens"], cub, inp["total_blocks"], inp["k"], inp["w"],
                                        v=inp["v"])
    kc, vc = kc_full.clone(), vc_full.clone()
    for b in range(3):  # blocks completed at or after L0 are not pooled yet
        kc[cubh[b] + L0[b] // 128: cubh[b + 1]] = SENTINEL
        vc[cubh[b] + L0[b] // 128: cubh[b + 1]] = SENTINEL
    kw = torch.stack([ring_from_raw(inp["k"][cu[b]:cu[b + 1]], L0[b], ring) for b in range(3)]).contiguous()
    vw = torch.stack([ring_from_raw(inp["v"][cu[b]:cu[b + 1]], L0[b], ring) for b in range(3)]).contiguous()
    one = i32([0, 1, 2, 3])
    got, rows = [], []
    for s in range(steps):
        pos = [L0[b] + s for b in range(3)]
        idx = torch.tensor([cu[b] + pos[b] for b in range(3)], dtype=torch.long, device=DEV)
        q, k, v = inp["q"][idx].contiguous(), inp["k"][idx].contiguous(), inp["v"][idx].contiguous()
        p0 = i32(pos)
        hca.hca_compress_chunk(p, one, p0, cub, 1, k, inp["w"], kw, kc, v=v, vw=vw, vc=vc)
        hca.hca_ring_append(p, one, p0, 1, k, kw, v=v, vw=vw)
        seqlens = i32([x + 1 for x in pos])
        ws = hca.new_decode_workspace(p, 3, max((x + 1) // 128 for x in pos))
        got.append(hca.hca_attend_decode(p, seqlens, cub, max((x + 1) // 128 for x in pos), q, kc, vc, kw, vw,
                                         workspace=ws).clone())
        rows += idx.tolist()
    torch.cuda.synchronize()
    for b in range(3):  # every block completed during the loop was pooled exactly as in one pass
        done = torch.arange(cubh[b] + L0[b] // 128, cubh[b] + lens[b] // 128, device=DEV)
        assert torch.equal(kc[done], kc_full[done]) and torch.equal(vc[done], vc_full[done])
    w = inp["w"].cpu()
    ref = oracle.attend_prefill(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), oracle.compress(inp["k"].cpu(), w, cu),
                                oracle.compress(inp["v"].cpu(), w, cu), cu, c.window, rows=rows)
    assert_close(torch.cat(got), ref, dt, f"{steps} decode steps with cache maintenance ({dtype})")
