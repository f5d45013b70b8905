"""Pins for the CPU oracle, written against things other than the oracle.

Each pin takes the oracle module as an argument and raises AssertionError on
a mismatch, so tests/test_oracle_mutants.py can run the same pins against
copies of the oracle with planted mistakes and check that each is caught.

The pins use independent formulations: a dense masked attention over an
explicit [T, n_blocks + T] mask with a pooling matrix (brute force), torch's
scaled_dot_product_attention (library routine), torch's avg_pool1d (library
routine), closed forms (constant rows, zero queries, dominant logits) and
invariants (row sums, permutations, coverage).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


# --------------------------------------------------------------------------
# brute force: dense pooling matrix + dense boolean mask, float64
# --------------------------------------------------------------------------
def brute_force(q, k, v, w, lens, window, block, scale=None):
    """Dense formulation of the whole layer for packed sequences.

    For each sequence: a pooling matrix P[h, j, s] = softmax(w_h)[s - block*j]
    for s in block j (scipy softmax), compressed keys P @ K, a key matrix of
    all compressed entries followed by every raw row, and an explicit boolean
    mask mask[t, j] = block*(j+1) <= t+1, mask[t, nb+s] = t-W+1 <= s <= t.
    Returns (out [N, Hq, d], kc [total_blocks, Hkv, d], vc).
    """
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    p = scipy.special.softmax(np.asarray(w, np.float64), axis=-1)  # [Hkv, block]
    cu = _cu(lens)
    out = np.zeros((n, hq, d))
    kcs, vcs = [], []
    for b, T in enumerate(lens):
        s, e = cu[b], cu[b + 1]
        nb = T // block
        P = np.zeros((hkv, nb, T))
        for j in range(nb):
            P[:, j, block * j: block * (j + 1)] = p
        kc = np.einsum("hjs,shd->jhd", P, k[s:e])
        vc = np.einsum("hjs,shd->jhd", P, v[s:e])
        kcs.append(kc)
        vcs.append(vc)
        keys = np.concatenate([kc, k[s:e]], axis=0)  # [nb+T, Hkv, d]
        vals = np.concatenate([vc, v[s:e]], axis=0)
        tt = np.arange(T)[:, None]
        mask = np.zeros((T, nb + T), dtype=bool)
        jj = np.arange(nb)[None, :]
        mask[:, :nb] = block * (jj + 1) <= tt + 1
        ss = np.arange(T)[None, :]
        mask[:, nb:] = (ss <= tt) & (ss >= tt - window + 1)
        for hh in range(hq):
            kvh = hh // g
            sc = q[s:e, hh] @ keys[:, kvh].T * scale  # [T, nb+T]
            sc = np.where(mask, sc, -np.inf)
            pr = scipy.special.softmax(sc, axis=1)
            out[s:e, hh] = pr @ vals[:, kvh]
    d_ = k.shape[2]
    kc_all = np.concatenate(kcs) if kcs else np.zeros((0, hkv, d_))
    vc_all = np.concatenate(vcs) if vcs else np.zeros((0, hkv, d_))
    return out, kc_all, vc_all


def _rand_case(seed, lens, hq, hkv, d, block):
    r = _rng(seed)
    n = int(sum(lens))
    q = r.standard_normal((n, hq, d))
    k = r.standard_normal((n, hkv, d))
    v = r.standard_normal((n, hkv, d))
    w = r.standard_normal((hkv, block)) * 1.5
    return q, k, v, w


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_brute_force(orc):
    """Oracle == dense brute force on varlen batches, several windows, GQA."""
    cases = [
        # (lens, hq, hkv, d, block, window)
        ([300, 130, 7], 4, 2, 16, 128, 64),
        ([512], 4, 1, 8, 128, 128),
        ([260], 2, 2, 8, 128, 127),
        ([400, 129], 4, 2, 8, 128, 1),
        ([390], 4, 1, 8, 128, 300),
        ([33, 20, 41], 6, 3, 4, 8, 5),   # small block: many entries per sequence
    ]
    for i, (lens, hq, hkv, d, block, win) in enumerate(cases):
        q, k, v, w = _rand_case(100 + i, lens, hq, hkv, d, block)
        ref, kc_ref, vc_ref = brute_force(q, k, v, w, lens, win, block)
        cu = _cu(lens)
        kc = orc.compress(k, w, cu, block=block)
        vc = orc.compress(v, w, cu, block=block)
        assert kc.shape == kc_ref.shape, (i, kc.shape, kc_ref.shape)
        assert np.allclose(kc, kc_ref, rtol=1e-12, atol=1e-12), (i, "kc")
        assert np.allclose(vc, vc_ref, rtol=1e-12, atol=1e-12), (i, "vc")
        out = orc.attend_prefill(q, k, v, kc, vc, cu, win, block=block)
        assert _rel(out, ref) <= 1e-12, (i, _rel(out, ref))


def pin_causal_sdpa(orc):
    """T <= min(W, block-1): no block is complete and the window holds the
    whole prefix, so the layer is ordinary causal attention."""
    for i, (T, win, hq, hkv, d) in enumerate([(100, 128, 4, 2, 16), (60, 64, 4, 1, 32),
                                              (127, 127, 2, 1, 8), (1, 1, 4, 4, 8),
                                              (127, 200, 4, 2, 8)]):
        q, k, v, w = _rand_case(200 + i, [T], hq, hkv, d, 128)
        cu = _cu([T])
        kc = orc.compress(k, w, cu)
        vc = orc.compress(v, w, cu)
        assert kc.shape[0] == 0
        out = orc.attend_prefill(q, k, v, kc, vc, cu, win)
        g = hq // hkv
        tq = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1, Hq, T, d]
        tk = torch.from_numpy(k).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
        tv = torch.from_numpy(v).repeat_interleave(g, dim=1).permute(1, 0, 2)[None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert _rel(out, ref) <= 1e-12, (i, _rel(out, ref))


def pin_constant_blocks(orc):
    """Rows constant within each block compress to that constant (the pooling
    weights sum to one)."""
    r = _rng(3)
    lens = [128 * 3 + 50, 256]
    hkv, d = 2, 8
    per_block = r.standard_normal((10, hkv, d))
    x = np.zeros((sum(lens), hkv, d))
    cu = _cu(lens)
    expect = []
    bi = 0
    for b, T in enumerate(lens):
        for j in range(T // 128):
            x[cu[b] + 128 * j: cu[b] + 128 * (j + 1)] = per_block[bi]
            expect.append(per_block[bi])
            bi += 1
        tail = T - 128 * (T // 128)
        if tail:
            x[cu[b + 1] - tail: cu[b + 1]] = 99.0  # partial block: never pooled
    w = r.standard_normal((hkv, 128)) * 3
    kc = orc.compress(x, w, cu)
    assert kc.shape == (len(expect), hkv, d)
    assert np.allclose(kc, np.stack(expect), rtol=1e-13, atol=1e-13)


def pin_uniform_logits_avg_pool(orc):
    """Equal logits give the block mean = torch avg_pool1d(kernel=stride=128)."""
    r = _rng(4)
    T, hkv, d = 128 * 5 + 17, 2, 6
    x = r.standard_normal((T, hkv, d))
    w = np.full((hkv, 128), 0.37)
    kc = orc.compress(x, w, _cu([T]))
    ref = torch.nn.functional.avg_pool1d(torch.from_numpy(x).permute(1, 2, 0),
                                         kernel_size=128, stride=128)  # [Hkv, d, nb]
    ref = ref.permute(2, 0, 1).numpy()
    assert kc.shape == ref.shape
    assert np.allclose(kc, ref, rtol=1e-12, atol=1e-12)


def pin_dominant_logit(orc):
    """w = 60 e_r (one large logit) selects row r of every block: the other
    weights are e^-60 / (1 + 127 e^-60) < 1e-25."""
    r = _rng(5)
    T, hkv, d = 128 * 4, 2, 5
    x = r.standard_normal((T, hkv, d))
    sel = [17, 101]
    w = np.zeros((hkv, 128))
    for h in range(hkv):
        w[h, sel[h]] = 60.0
    kc = orc.compress(x, w, _cu([T]))
    for j in range(4):
        for h in range(hkv):
            assert np.allclose(kc[j, h], x[128 * j + sel[h], h], rtol=0, atol=1e-20)


def pin_permutation(orc):
    """Permuting the 128 rows of every block together with the logits leaves
    the entries unchanged; the result is linear in the rows."""
    r = _rng(6)
    T, hkv, d = 128 * 3, 1, 4
    x = r.standard_normal((T, hkv, d))
    y = r.standard_normal((T, hkv, d))
    w = r.standard_normal((hkv, 128))
    perm = r.permutation(128)
    xp = x.reshape(3, 128, hkv, d)[:, perm].reshape(T, hkv, d)
    cu = _cu([T])
    a = orc.compress(x, w, cu)
    b = orc.compress(xp, w[:, perm], cu)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
    lin = orc.compress(2.0 * x - 3.0 * y, w, cu)
    assert np.allclose(lin, 2.0 * a - 3.0 * orc.compress(y, w, cu), rtol=1e-12, atol=1e-12)


def pin_row_sums(orc):
    """Each probability row sums to one and has the visible-key count as its
    length: floor((t+1)/128) entries plus min(W, t+1) raw rows."""
    lens = [300, 140]
    q, k, v, w = _rand_case(7, lens, 4, 2, 8, 128)
    cu = _cu(lens)
    kc, vc = orc.compress(k, w, cu), orc.compress(v, w, cu)
    win = 40
    _, probs = orc.attend_prefill(q, k, v, kc, vc, cu, win, return_probs=True)
    for (tok, h), pr in probs.items():
        b = int(np.searchsorted(cu, tok, side="right") - 1)
        t = tok - cu[b]
        assert pr.shape[1] == (t + 1) // 128 + min(win, t + 1), (tok, pr.shape)
        assert np.allclose(pr.sum(axis=1), 1.0, atol=1e-12)


def pin_zero_query_mean(orc):
    """Q = 0: every score is zero, so each output is the plain average of the
    visible values (computed here from running sums)."""
    lens = [300, 129]
    _, k, v, w = _rand_case(8, lens, 4, 2, 8, 128)
    q = np.zeros((sum(lens), 4, 8))
    cu = _cu(lens)
    kc, vc = orc.compress(k, w, cu), orc.compress(v, w, cu)
    win = 50
    out = orc.attend_prefill(q, k, v, kc, vc, cu, win)
    cb = 0
    for b, T in enumerate(lens):
        vs = v[cu[b]:cu[b + 1]]
        csum = np.concatenate([np.zeros((1,) + vs.shape[1:]), np.cumsum(vs, axis=0)])
        vcs = vc[cb: cb + T // 128]
        ccum = np.concatenate([np.zeros((1,) + vs.shape[1:]), np.cumsum(vcs, axis=0)])
        for t in range(T):
            nvis = (t + 1) // 128
            lo = max(0, t - win + 1)
            tot = ccum[nvis] + (csum[t + 1] - csum[lo])
            mean = tot / (nvis + t + 1 - lo)  # [Hkv, d]
            expect = np.repeat(mean, 2, axis=0)  # heads 2h, 2h+1 read KV head h
            assert np.allclose(out[cu[b] + t], expect, rtol=1e-12, atol=1e-12), (b, t)
        cb += T // 128


def pin_constant_values(orc):
    """All visible values equal c: the output is c whatever Q and K are."""
    lens = [260]
    q, k, _, w = _rand_case(9, lens, 2, 1, 8, 128)
    c = np.linspace(-2, 3, 8)
    v = np.broadcast_to(c, (260, 1, 8)).copy()
    cu = _cu(lens)
    kc, vc = orc.compress(k, w, cu), orc.compress(v, w, cu)
    out = orc.attend_prefill(q * 4, k, v, kc, vc, cu, 100)
    assert np.allclose(out, c, rtol=1e-12, atol=1e-12)


def pin_coverage(orc):
    """W >= block-1: every position <= t reaches row t, raw or through its
    complete block; W < block-1 leaves a gap of block-1-W positions at most."""
    for win in (127, 128, 300):
        for t in range(0, 2000):
            n, s0 = orc.visible_sets(t, win)
            assert s0 <= 128 * n, (win, t)
    gaps = [max(0, orc.visible_sets(t, 64)[1] - 128 * orc.visible_sets(t, 64)[0])
            for t in range(2000)]
    assert max(gaps) == 127 - 64


def pin_decode_is_last_prefill_row(orc):
    """decode(L) == prefill row L-1 when the cache holds the same tokens."""
    hq, hkv, d, win, ring = 4, 2, 8, 60, 64
    lens = [300, 128, 61, 1]
    q, k, v, w = _rand_case(10, lens, hq, hkv, d, 128)
    cu = _cu(lens)
    kc, vc = orc.compress(k, w, cu), orc.compress(v, w, cu)
    cub = orc.cu_blocks_from_cu_seqlens(cu)
    rows = [int(cu[b + 1] - 1) for b in range(len(lens))]
    ref = orc.attend_prefill(q, k, v, kc, vc, cu, win, rows=rows)
    kw = np.zeros((len(lens), ring, hkv, d))
    vw = np.zeros((len(lens), ring, hkv, d))
    for b, L in enumerate(lens):
        for s in range(max(0, L - ring), L):
            kw[b, s % ring] = k[cu[b] + s]
            vw[b, s % ring] = v[cu[b] + s]
    out = orc.attend_decode(q[rows], kc, vc, kw, vw, np.array(lens), cub, win)
    assert _rel(out, ref) <= 1e-13


def pin_hand_example(orc):
    """Values worked out by hand (tests/golden/hand_example.json)."""
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    blk = g["block"]
    k = np.array(g["k"], dtype=np.float64)[:, None, :]
    v = np.array(g["v"], dtype=np.float64)[:, None, :]
    q = np.array(g["q"], dtype=np.float64)[:, None, :]
    w = np.array([g["w"]], dtype=np.float64)
    cu = _cu([k.shape[0]])
    kc = orc.compress(k, w, cu, block=blk)
    vc = orc.compress(v, w, cu, block=blk)
    assert np.allclose(kc[:, 0], np.array(g["expect_kc"]), rtol=0, atol=1e-14)
    assert np.allclose(vc[:, 0], np.array(g["expect_vc"]), rtol=0, atol=1e-14)
    out = orc.attend_prefill(q, k, v, kc, vc, cu, g["window"], scale=g["scale"], block=blk)
    assert np.allclose(out[:, 0], np.array(g["expect_out"]), rtol=0, atol=1e-14)


def pin_page_entry_counts(orc):
    """The pages' structural numbers (tests/golden/page_structure.json)."""
    with open(os.path.join(GOLDEN, "page_structure.json")) as f:
        g = json.load(f)
    assert orc.BLOCK == g["tokens_per_entry"]
    for ctx, entries in g["compressed_entries_at_context"].items():
        L = int(ctx)
        assert int(orc.blocks_per_sequence([L])[0]) == entries
        # compressed part alone: exactly tokens_per_entry times fewer entries
        assert L // entries == g["tokens_per_entry"]
    for ctx, n in g["cache_entries_with_window_128"].items():
        assert orc.cache_entries(int(ctx), 128) == n


def pin_head_mix_dense(orc):
    """R7 against a dense formulation: per token, the [Hq, Hq] block-diagonal
    matrix I + U V^T (one block per KV head) applied with torch, then the
    gate.  Non-symmetric U, V and varying gates catch an exchanged U / V,
    a transposed product and the gate applied before the mixing."""
    r = _rng(61)
    n, hkv, g, rank, d = 5, 2, 6, 3, 7
    o = r.standard_normal((n, hkv * g, d))
    u = r.standard_normal((hkv, g, rank))
    v = r.standard_normal((hkv, g, rank)) * 0.5
    gate = r.standard_normal((n, hkv * g)) * 2
    m = torch.zeros((hkv * g, hkv * g), dtype=torch.float64)
    for h in range(hkv):
        m[h * g:(h + 1) * g, h * g:(h + 1) * g] = torch.eye(g, dtype=torch.float64) + \
            torch.from_numpy(u[h]) @ torch.from_numpy(v[h]).T
    ref = torch.einsum("ij,njd->nid", m, torch.from_numpy(o)) * torch.sigmoid(torch.from_numpy(gate))[:, :, None]
    got = orc.head_mix_and_gate(o, u, v, gate)
    assert _rel(got, ref.numpy()) < 1e-12, _rel(got, ref.numpy())


def pin_head_mix_special_cases(orc):
    """Closed forms: no mixing and no gate is the identity; U = 0 is the
    identity; a rank-1 mix with U = e_a, V = e_b adds head b to head a only;
    a zero gate logit halves the output and a large one keeps it."""
    r = _rng(62)
    o = r.standard_normal((3, 4, 5))
    assert np.array_equal(orc.head_mix_and_gate(o), o)
    z = np.zeros((1, 4, 2))
    assert np.allclose(orc.head_mix_and_gate(o, z, r.standard_normal((1, 4, 2))), o, rtol=0, atol=0)
    u = np.zeros((1, 4, 1))
    v = np.zeros((1, 4, 1))
    u[0, 1, 0] = 1.0
    v[0, 3, 0] = 1.0
    want = o.copy()
    want[:, 1] += o[:, 3]
    assert np.allclose(orc.head_mix_and_gate(o, u, v), want, rtol=0, atol=1e-15)
    assert np.allclose(orc.head_mix_and_gate(o, gate=np.zeros((3, 4))), 0.5 * o, rtol=0, atol=1e-15)
    assert np.allclose(orc.head_mix_and_gate(o, gate=np.full((3, 4), 60.0)), o, rtol=1e-15, atol=0)


ALL_PINS = [
    pin_brute_force, pin_causal_sdpa, pin_constant_blocks, pin_uniform_logits_avg_pool,
    pin_dominant_logit, pin_permutation, pin_row_sums, pin_zero_query_mean,
    pin_constant_values, pin_coverage, pin_decode_is_last_prefill_row, pin_hand_example,
    pin_page_entry_counts, pin_head_mix_dense, pin_head_mix_special_cases,
]
