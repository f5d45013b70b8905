"""Plain CPU oracle for the sparse-attention decode step of the full-context
(MLA) layers: indexer scores, top-k selection, attention over the selected
positions.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What the pages say (release blog "ERNIE 5.5 Flash Base", section 2.1; Zhidx
article, section "1. Latent-Gated Sparse Attention"; model card): the few
full-context MLA layers use DeepSeek-style sparse attention: a lightweight
indexer scores the past positions of each query, and core attention runs only
over the top-k highest-scoring positions, so its per-query cost stays
constant as the context grows; these layers use 256-dim query/key/value
heads.

Readings where the pages leave steps open (restated where used):

D1  indexer: one head of width 128 in int8; the score of past position s for
    the query is the exact integer dot product qi . ki[s].
D2  selection: the k positions with the highest score among 0 .. t (the query
    sits at t = L - 1 and sees itself); equal scores go to the smaller
    position; with L <= k every position is selected.  The result is the
    selected positions in increasing order.
D3  core attention: 64 query heads of width 256 over one shared key/value
    head of width 256 (as in the HCA layers, Hkv = 1), one softmax with scale
    1/sqrt(256) over the selected positions only.

Arithmetic: integers for D1/D2 (exact), float64 for D3.  Pins
(tests/test_dsa_oracle.py): selection against a brute-force rank count
(a position is selected iff fewer than k positions beat it); attention
against torch SDPA over the gathered rows and, with k >= L, against
ordinary full attention; invariance of the output
to the order of the selected list; closed forms (constant values, a dominant
score).  None of the functions is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


def _i64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x).astype(np.int64)


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def index_scores(qi, ki_rows) -> np.ndarray:
    """D1: exact integer scores qi . ki[s] for every row s of ki_rows.

    qi: [d_i] int8; ki_rows: [L, d_i] int8.  Returns [L] int64."""
    return _i64(ki_rows) @ _i64(qi)


def select_topk(scores, k: int) -> np.ndarray:
    """D2: positions of the k highest scores (ties: smaller position first),
    returned in increasing position order.  scores: [L] integers."""
    s = _i64(scores)
    n = s.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    # rank by (score descending, position ascending): lexsort's last key is
    # the primary one
    order = np.lexsort((np.arange(n), -s))
    return np.sort(order[:k]).astype(np.int64)


def attend_selected(q, k_rows, v_rows, scale=None) -> np.ndarray:
    """D3: q [H, d] attends to the selected key/value rows [n, d] under one
    softmax.  Returns [H, d] float64."""
    q, kr, vr = _f64(q), _f64(k_rows), _f64(v_rows)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    z = (q @ kr.T) * scale
    a = np.exp(z - z.max(axis=1, keepdims=True))
    return (a / a.sum(axis=1, keepdims=True)) @ vr


def dsa_decode(q, qi, k, v, ki, seqlens, cu_rows, topk: int, scale=None):
    """One decode step for a batch: sequence b has L = seqlens[b] cached rows
    (rows cu_rows[b] .. cu_rows[b] + L - 1 of k, v [rows, d] and ki [rows,
    d_i]); its query q[b] [H, d] with indexer query qi[b] [d_i] sits at
    position L - 1.  Returns (o [B, H, d] float64, list of selected positions
    per sequence)."""
    lens, cu = _i64(seqlens), _i64(cu_rows)
    kk, vv, kki = _f64(k), _f64(v), _i64(ki)
    out, sel = [], []
    for b in range(lens.shape[0]):
        L, r0 = int(lens[b]), int(cu[b])
        pos = select_topk(index_scores(_i64(qi[b]), kki[r0:r0 + L]), topk)
        sel.append(pos)
        out.append(attend_selected(_f64(q[b]), kk[r0 + pos], vv[r0 + pos], scale))
    return np.stack(out), sel
