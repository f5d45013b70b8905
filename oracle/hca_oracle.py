"""Plain CPU oracle for the Heavily Compressed Attention (HCA) layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code, constant table or helper with the HIP
library; the two meet only through the seeded synthetic inputs.

What the method computes (sources, by page title and section):

* "ERNIE 5.5 Flash Base" release blog, section 2.1 (hybrid sparse attention),
  HCA paragraph: every HCA layer turns each run of 128 tokens into one cached
  entry and then attends to all of these entries together with a short window
  of recent tokens that were not compressed; the layer therefore still sees
  the whole sequence while caching a fraction of a full layer's keys/values.
* Zhidx article "280B total parameters, 14B activated ...", section
  "1. Latent-Gated Sparse Attention": attention runs only over the compressed
  entries and a window made of a small number of recent uncompressed tokens.
* Model card "ERNIE 5.5 Flash Base" (nlp.com.ai), architecture paragraph:
  the HCA layers keep a single cached entry for each 128-token block, and
  their attention heads are 512 wide.

Readings taken where the pages leave a step open (each is restated where it is
used below):

R1  compressor: entry j of KV head h is the softmax(w_h)-weighted sum of the
    128 raw rows of block j, w_h a learned length-128 logit vector per KV head;
    the same weights pool K and V.
R2  blocks are the non-overlapping runs [128j, 128j+127] counted from the start
    of each sequence; a trailing partial block is not compressed.
R3  query t sees compressed entry j iff the block is complete at t, i.e.
    128(j+1) <= t+1, and raw positions max(0, t-W+1) .. t.
R4  the two key sets are concatenated (no de-duplication) under one softmax
    with scale 1/sqrt(d); values use the same selection.
R5  query head h reads KV head h // (Hq / Hkv).
R6  decode: a sequence of length L has its query at position L-1; raw
    position s lives in ring slot s mod R.
R7  attention epilogue (release blog, section 2.1, last paragraph; Zhidx
    article, Low-Rank Gated Attention and Virtual Head Attention
    paragraphs): the pages give an output gate computed from the query
    latent and a cross-head low-rank mixing with an identity skip, applied
    after attention; they fix no rank and no gate granularity.  Here the
    mixing acts among the G heads that share a KV head, O' = O + U (V^T O)
    with U, V [G, r] per KV head, and the gate is one logit per (token,
    head) taken through a sigmoid after the mixing: y = sigmoid(g) O'.
    The gate projection itself runs upstream (its logits are an input).

Arithmetic is float64 throughout; inputs are decoded exactly (bf16 -> f64 is
exact).  Matrix products and reductions are numpy library calls; nothing is
blocked, fused or reordered beyond the definitions above.

Pins (tests/test_oracle.py): brute-force dense masked attention in float64;
reduction to ordinary causal attention (torch SDPA) when T <= min(W, 127);
constant-within-block rows compress to themselves; uniform logits give the
block mean (avg_pool1d); a dominant logit selects one row; Q = 0 gives the
unweighted mean of the visible values; constant values give that constant;
probability rows sum to one; decode(L) equals prefill row L-1; the page's
128-tokens-per-entry count.  Every function below is covered by at least one
of them; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# Tokens per compressed entry: an HCA layer keeps one cached entry for each
# run of 128 tokens (release blog, section 2.1, HCA paragraph).
BLOCK = 128


def _f64(x) -> np.ndarray:
    """Decode any array-like (numpy, or torch CPU tensor of any float dtype)
    exactly into float64."""
    if hasattr(x, "detach"):  # torch tensor: widen on the torch side, exact
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def pooling_weights(w) -> np.ndarray:
    """R1: p_h = softmax(w_h) over the 128 positions of a block.

    w: [Hkv, block] logits.  Returns [Hkv, block] float64, rows summing to 1.
    The maximum is subtracted before exponentiating (softmax is invariant to
    it) so large logits do not overflow.
    """
    w = _f64(w)
    z = w - w.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def blocks_per_sequence(lengths, block: int = BLOCK) -> np.ndarray:
    """R2: number of complete blocks floor(len / block) of each sequence."""
    return _ints(lengths) // block


def cu_blocks_from_cu_seqlens(cu_seqlens, block: int = BLOCK) -> np.ndarray:
    """Prefix sum of complete-block counts: entry range of sequence b in the
    packed compressed cache is [cu_blocks[b], cu_blocks[b+1])."""
    cu = _ints(cu_seqlens)
    nb = blocks_per_sequence(cu[1:] - cu[:-1], block)
    return np.concatenate([[0], np.cumsum(nb)]).astype(np.int64)


def compress(x, w, cu_seqlens, block: int = BLOCK) -> np.ndarray:
    """R1/R2: pool every complete block of raw rows into one cached entry.

    x: [N_tok, Hkv, d] raw keys (or values), sequences packed by cu_seqlens.
    w: [Hkv, block] pooling logits.
    Returns [total_blocks, Hkv, d] float64 with entry cu_blocks[b] + j equal
    to sum_i p[h, i] * x[cu_seqlens[b] + block*j + i, h, :].
    """
    x = _f64(x)
    p = pooling_weights(w)  # [Hkv, block]
    cu = _ints(cu_seqlens)
    hkv, d = x.shape[1], x.shape[2]
    assert p.shape == (hkv, block)
    out = []
    for b in range(len(cu) - 1):
        start, end = int(cu[b]), int(cu[b + 1])
        for j in range((end - start) // block):
            rows = x[start + block * j: start + block * (j + 1)]  # [block, Hkv, d]
            # weight row i of KV head h by p[h, i], then sum over the block
            out.append((p.T[:, :, None] * rows).sum(axis=0))
    if not out:
        return np.zeros((0, hkv, d))
    return np.stack(out)


def visible_sets(t: int, window: int, block: int = BLOCK):
    """R3 for query position t (0-based within its sequence).

    Returns (n, s0): compressed entries 0..n-1 and raw positions s0..t are
    visible, with n = floor((t+1)/block) (block j complete iff
    block*(j+1) <= t+1) and s0 = max(0, t-window+1).
    """
    return (t + 1) // block, max(0, t - window + 1)


def _attend_rows(qh, keys, vals, scale):
    """One softmax over the concatenated key set (R4).

    qh: [G, d] query rows sharing one KV head; keys, vals: [nk, d].
    Returns (out [G, d], probs [G, nk]).
    """
    z = (qh @ keys.T) * scale  # [G, nk] scaled scores
    a = np.exp(z - z.max(axis=1, keepdims=True))
    probs = a / a.sum(axis=1, keepdims=True)
    return probs @ vals, probs


def attend_prefill(q, k, v, kc, vc, cu_seqlens, window: int, scale=None,
                   block: int = BLOCK, rows=None, return_probs: bool = False,
                   q_holds_rows_only: bool = False):
    """R3-R5: causal HCA attention for every token of packed sequences.

    q: [N_tok, Hq, d]; k, v: [N_tok, Hkv, d] raw; kc, vc: [total_blocks, Hkv, d]
    compressed entries packed by cu_blocks (derived from cu_seqlens).
    rows: optional iterable of global token indices; when given only those
    rows are computed and the result is [len(rows), Hq, d].  With
    q_holds_rows_only, q is [len(rows), Hq, d] and q[i] is the query of token
    rows[i] (so a sample of a very long prefill needs only its own queries).
    Returns float64 output (and, with return_probs, a dict mapping
    (token, kv_head) -> probability matrix [G, n + t - s0 + 1], compressed
    keys first, raw keys in position order).
    """
    k, v, kc, vc = _f64(k), _f64(v), _f64(kc), _f64(vc)
    cu = _ints(cu_seqlens)
    cub = cu_blocks_from_cu_seqlens(cu, block)
    ntok = int(cu[-1])
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    assert hq % hkv == 0
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if rows is None:
        rows = range(ntok)
    rows = [int(r) for r in rows]
    assert not q_holds_rows_only or len(rows) == q.shape[0]
    seq_of = np.searchsorted(cu, np.asarray(rows, dtype=np.int64), side="right") - 1
    out = np.zeros((len(rows), hq, d))
    probs = {}
    for i, (tok, b) in enumerate(zip(rows, seq_of)):
        start = int(cu[b])
        t = tok - start
        n, s0 = visible_sets(t, window, block)
        assert cub[b] + n <= cub[b + 1]
        qt = _f64(q[i] if q_holds_rows_only else q[tok])  # [Hq, d]
        for h in range(hkv):
            keys = np.concatenate([kc[cub[b]: cub[b] + n, h], k[start + s0: tok + 1, h]])
            vals = np.concatenate([vc[cub[b]: cub[b] + n, h], v[start + s0: tok + 1, h]])
            o, p = _attend_rows(qt[h * g:(h + 1) * g], keys, vals, scale)
            out[i, h * g:(h + 1) * g] = o
            if return_probs:
                probs[(tok, h)] = p
    if return_probs:
        return out, probs
    return out


def attend_decode(q, kc, vc, kw, vw, seqlens, cu_blocks, window: int,
                  scale=None, block: int = BLOCK):
    """R3-R6 for one new query per sequence.

    q: [B, Hq, d] queries at positions L_b - 1; kc, vc: [total, Hkv, d] packed
    by cu_blocks (sequence b owns at least floor(L_b/block) entries from
    cu_blocks[b]); kw, vw: [B, R, Hkv, d] rings holding raw position s in slot
    s mod R.  Returns [B, Hq, d] float64.
    """
    q, kc, vc, kw, vw = _f64(q), _f64(kc), _f64(vc), _f64(kw), _f64(vw)
    lens = _ints(seqlens)
    cub = _ints(cu_blocks)
    nb, hq, d = q.shape
    ring = kw.shape[1]
    hkv = kc.shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((nb, hq, d))
    for b in range(nb):
        t = int(lens[b]) - 1
        n, s0 = visible_sets(t, window, block)
        assert cub[b] + n <= cub[b + 1]
        assert ring >= t - s0 + 1
        slots = [s % ring for s in range(s0, t + 1)]
        for h in range(hkv):
            keys = np.concatenate([kc[cub[b]: cub[b] + n, h], kw[b, slots, h]])
            vals = np.concatenate([vc[cub[b]: cub[b] + n, h], vw[b, slots, h]])
            out[b, h * g:(h + 1) * g], _ = _attend_rows(q[b, h * g:(h + 1) * g], keys, vals, scale)
    return out


def cache_entries(length: int, window: int, block: int = BLOCK) -> int:
    """Entries an HCA layer keeps for a sequence of `length` tokens: one per
    complete block plus the raw window (release blog, section 2.1: a fraction
    of a full layer's cache)."""
    return length // block + min(window, length)


def head_mix_and_gate(o, mix_u=None, mix_v=None, gate=None):
    """R7: y[t, h] = sigmoid(gate[t, h]) * (o[t, h] + sum_r U[h, r] sum_h' V[h', r] o[t, h'])
    within each KV head's group of G query heads.

    o: [N, Hq, d]; mix_u, mix_v: [Hkv, G, r] (None: no mixing); gate:
    [N, Hq] logits (None: no gate).  Returns float64 [N, Hq, d].
    """
    o = _f64(o)
    out = o.copy()
    if mix_u is not None:
        u, v = _f64(mix_u), _f64(mix_v)
        hkv, g, _ = u.shape
        for h in range(hkv):
            grp = o[:, h * g:(h + 1) * g, :]              # [N, G, d]
            z = np.einsum("ngd,gr->nrd", grp, v[h])       # V^T O   [N, r, d]
            out[:, h * g:(h + 1) * g, :] = grp + np.einsum("gr,nrd->ngd", u[h], z)
    if gate is not None:
        out = out * (1.0 / (1.0 + np.exp(-_f64(gate))))[:, :, None]
    return out
