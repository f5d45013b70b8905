"""Plain CPU oracle for the gradient of the HCA layer forward (prefill).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code, constant table or helper with the HIP
library.

The forward is the one in hca_oracle (readings R1-R5 there): the pages train
the model at long context (release blog "ERNIE 5.5 Flash Base", section 2.1;
the model card gives the 128K training context) but print no backward, so the
gradient is the plain derivative of that forward, written out with the chain
rule in the forward's order:

  forward   p = softmax(w_h);  Kc_j = sum_i p_i K_{128j+i},  Vc likewise;
            per query row (t, head): keys X = [Kc_0..Kc_{n-1}; K_{s0..t}],
            values Y likewise, z = scale X q, a = softmax(z), O = a Y.
  backward  for a loss L with dL/dO = dO:
            dY_j += a_j dO                       (each key's value)
            dP_j  = dO . Y_j,  D = sum_j a_j dP_j  (= dO . O)
            dz_j  = a_j (dP_j - D)               (softmax Jacobian)
            dq    = scale sum_j dz_j X_j
            dX_j += scale dz_j q
            then the keys and values scatter back: a raw key row to dK / dV
            of its position, a compressed entry to dKc / dVc; the pooling
            sends dK_{128j+i} += p_i dKc_j (dV likewise) and
            g_i = sum_j (dKc_j . K_{128j+i} + dVc_j . V_{128j+i}),
            dw = p * (g - sum_k p_k g_k)         (softmax Jacobian again).

Arithmetic is float64; matrix products are numpy calls, nothing is blocked or
fused.  Pins (tests/test_oracle_backward.py): central finite differences of
the forward oracle's loss sum(dO * O) along random directions of q, k, v and
w; reduction to ordinary causal attention (torch autograd through SDPA in
float64) when no block is complete and the window covers the sequence; the
pooling gradient dw sums to zero over each block position set; zero dO gives
zero gradients.  None of the functions here is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

from .hca_oracle import BLOCK, _f64, _ints, attend_prefill, compress, cu_blocks_from_cu_seqlens, \
    pooling_weights, visible_sets


def attend_prefill_backward(q, k, v, w, dout, cu_seqlens, window: int, scale=None, block: int = BLOCK,
                            return_stats: bool = False, rows=None, q_holds_rows_only: bool = False):
    """Gradients of sum(dout * O) for O = the HCA prefill forward of q, k, v, w.

    q, dout: [N_tok, Hq, d]; k, v: [N_tok, Hkv, d] raw rows; w: [Hkv, block]
    pooling logits; sequences packed by cu_seqlens.  Returns float64
    (dq [N_tok, Hq, d], dk, dv [N_tok, Hkv, d], dw [Hkv, block]); with
    return_stats also a dict holding the per-row log-sum-exp of the scaled
    scores ('lse', [N_tok, Hq], natural log) and D = dO . O ('delta').

    rows: optional global token indices.  Only those query rows are taken
    through the chain rule: dq, lse and delta are [len(rows), ...] in that
    order, and dk, dv, dw hold the contributions of those rows alone (the
    exact gradient of sum over the selected rows of dout . O).  A raw row r
    whose every reader is selected (the rows r .. r+W-1 of its window, and
    every row that sees r's compressed entry) therefore gets its exact dk and
    dv.  With q_holds_rows_only, q and dout are [len(rows), Hq, d] and hold
    the rows of those tokens, so a sample of a very long sequence needs only
    its own queries.
    """
    k, v = _f64(k), _f64(v)
    cu = _ints(cu_seqlens)
    cub = cu_blocks_from_cu_seqlens(cu, block)
    ntok = int(cu[-1])
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    p = pooling_weights(w)  # [Hkv, block]
    kc, vc = compress(k, w, cu, block), compress(v, w, cu, block)
    if rows is None:
        rows = range(ntok)
    rows = [int(r) for r in rows]
    assert not q_holds_rows_only or (len(rows) == q.shape[0] and len(rows) == dout.shape[0])
    seq_of = np.searchsorted(cu, np.asarray(rows, dtype=np.int64), side="right") - 1

    dq = np.zeros((len(rows), hq, d))
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    dkc, dvc = np.zeros_like(kc), np.zeros_like(vc)
    lse = np.zeros((len(rows), hq))
    delta = np.zeros((len(rows), hq))
    for i, (tok, b) in enumerate(zip(rows, seq_of)):
        start = int(cu[b])
        t = tok - start
        n, s0 = visible_sets(t, window, block)
        qt = _f64(q[i] if q_holds_rows_only else q[tok])  # [Hq, d]
        dot = _f64(dout[i] if q_holds_rows_only else dout[tok])
        for h in range(hkv):
            hs = slice(h * g, (h + 1) * g)
            keys = np.concatenate([kc[cub[b]: cub[b] + n, h], k[start + s0: tok + 1, h]])  # [nk, d]
            vals = np.concatenate([vc[cub[b]: cub[b] + n, h], v[start + s0: tok + 1, h]])
            qh, doh = qt[hs], dot[hs]  # [G, d]
            z = (qh @ keys.T) * scale  # [G, nk]
            zmax = z.max(axis=1, keepdims=True)
            e = np.exp(z - zmax)
            a = e / e.sum(axis=1, keepdims=True)  # probabilities
            o = a @ vals
            dp = doh @ vals.T  # [G, nk]
            dd = (doh * o).sum(axis=1)  # D = dO . O per row
            dz = a * (dp - dd[:, None])
            dq[i, hs] = scale * (dz @ keys)
            dkeys = scale * (dz.T @ qh)  # [nk, d]
            dvals = a.T @ doh
            dkc[cub[b]: cub[b] + n, h] += dkeys[:n]
            dvc[cub[b]: cub[b] + n, h] += dvals[:n]
            dk[start + s0: tok + 1, h] += dkeys[n:]
            dv[start + s0: tok + 1, h] += dvals[n:]
            lse[i, hs] = zmax[:, 0] + np.log(e.sum(axis=1))
            delta[i, hs] = dd
    dk_raw_only, dv_raw_only = dk.copy(), dv.copy()
    # pooling: entry j of sequence b is sum_i p_i x_{128j+i}
    gsum = np.zeros((hkv, block))
    for b in range(len(cu) - 1):
        start = int(cu[b])
        for j in range(int(cub[b + 1] - cub[b])):
            e = int(cub[b]) + j
            blk = slice(start + block * j, start + block * (j + 1))
            for h in range(hkv):
                dk[blk, h] += p[h][:, None] * dkc[e, h][None, :]
                dv[blk, h] += p[h][:, None] * dvc[e, h][None, :]
                gsum[h] += k[blk, h] @ dkc[e, h] + v[blk, h] @ dvc[e, h]
    dw = p * (gsum - (p * gsum).sum(axis=1, keepdims=True))
    if return_stats:
        return dq, dk, dv, dw, {"lse": lse, "delta": delta, "dkc": dkc, "dvc": dvc,
                                "dk_raw": dk_raw_only, "dv_raw": dv_raw_only}
    return dq, dk, dv, dw


def loss_for_gradcheck(q, k, v, w, dout, cu_seqlens, window: int, scale=None, block: int = BLOCK) -> float:
    """sum(dout * O) through the forward oracle: the scalar whose gradient
    attend_prefill_backward returns (used by the finite-difference pins)."""
    kc = compress(k, w, cu_seqlens, block)
    vc = compress(v, w, cu_seqlens, block)
    o = attend_prefill(q, k, v, kc, vc, cu_seqlens, window, scale=scale, block=block)
    return float((_f64(dout) * o).sum())
