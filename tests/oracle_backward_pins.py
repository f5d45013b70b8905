"""Pins for the backward oracle, written against things other than it.

Each pin takes (forward oracle module, backward oracle module) and raises
AssertionError on a mismatch, so tests/test_oracle_backward.py can also run
them against copies of the backward oracle with planted mistakes.

Independent references: central finite differences of the forward oracle's
loss sum(dO * O) (the forward is pinned on its own, tests/oracle_pins.py),
torch autograd through scaled_dot_product_attention in float64 (library
routine) where the layer reduces to causal attention, scipy's logsumexp, and
invariants of the softmax Jacobian.
"""
from __future__ import annotations

import math

import numpy as np
import scipy.special
import torch


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _case(seed, lens, hq, hkv, d, block, w_scale=1.0):
    r = np.random.default_rng(seed)
    n = int(sum(lens))
    q = r.standard_normal((n, hq, d))
    k = r.standard_normal((n, hkv, d))
    v = r.standard_normal((n, hkv, d))
    w = r.standard_normal((hkv, block)) * w_scale
    dout = r.standard_normal((n, hq, d))
    return q, k, v, w, dout


def _rel(a, b):
    return float(np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300))


def _fd_check(fwd, bwd, lens, hq, hkv, d, block, window, seed):
    q, k, v, w, dout = _case(seed, lens, hq, hkv, d, block)
    cu = _cu(lens)
    dq, dk, dv, dw = bwd.attend_prefill_backward(q, k, v, w, dout, cu, window, block=block)
    r = np.random.default_rng(seed + 1)
    eps = 1e-5

    def loss(q_, k_, v_, w_):
        kc = fwd.compress(k_, w_, cu, block)
        vc = fwd.compress(v_, w_, cu, block)
        return float((dout * fwd.attend_prefill(q_, k_, v_, kc, vc, cu, window, block=block)).sum())

    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("w", dw)):
        args = {"q": q, "k": k, "v": v, "w": w}
        delta = r.standard_normal(args[name].shape)
        hi = dict(args)
        lo = dict(args)
        hi[name] = args[name] + eps * delta
        lo[name] = args[name] - eps * delta
        fd = (loss(**{x + "_": y for x, y in hi.items()}) - loss(**{x + "_": y for x, y in lo.items()})) / (2 * eps)
        an = float((grad * delta).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(fd), 1.0), f"d{name}: finite difference {fd} vs gradient {an}"


def pin_bwd_finite_differences_small_blocks(fwd, bwd):
    """Many compressed entries at a small block size (16), two sequences,
    grouped heads: every gradient against central differences."""
    _fd_check(fwd, bwd, lens=[70, 45], hq=4, hkv=2, d=8, block=16, window=10, seed=11)


def pin_bwd_finite_differences_block128(fwd, bwd):
    """The layer's own block of 128 with a window of 20 over 300 tokens."""
    _fd_check(fwd, bwd, lens=[300], hq=2, hkv=1, d=4, block=128, window=20, seed=12)


def pin_bwd_causal_sdpa_autograd(fwd, bwd):
    """No complete block and a window that covers the sequence: ordinary
    causal attention, whose gradients torch autograd gives through SDPA
    (float64); the pooling logits get no gradient at all."""
    lens, hq, hkv, d, block = [50], 4, 2, 16, 128
    q, k, v, w, dout = _case(21, lens, hq, hkv, d, block)
    dq, dk, dv, dw = bwd.attend_prefill_backward(q, k, v, w, dout, _cu(lens), window=64, block=block)
    tq = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2).requires_grad_(True)  # [Hq, T, d]
    tk = torch.tensor(k, dtype=torch.float64).permute(1, 0, 2).requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(1, 0, 2).requires_grad_(True)
    g = hq // hkv
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=0), tv.repeat_interleave(g, dim=0), is_causal=True)
    (o * torch.tensor(dout, dtype=torch.float64).permute(1, 0, 2)).sum().backward()
    assert _rel(dq, tq.grad.permute(1, 0, 2).numpy()) < 1e-10
    assert _rel(dk, tk.grad.permute(1, 0, 2).numpy()) < 1e-10
    assert _rel(dv, tv.grad.permute(1, 0, 2).numpy()) < 1e-10
    assert np.all(dw == 0.0)


def pin_bwd_dw_sums_to_zero(fwd, bwd):
    """softmax is invariant to adding a constant to all logits, so the
    gradient of the pooling logits of each KV head sums to zero."""
    lens, block = [300, 260], 128
    q, k, v, w, dout = _case(31, lens, 4, 2, 8, block)
    dw = bwd.attend_prefill_backward(q, k, v, w, dout, _cu(lens), 16, block=block)[3]
    assert np.abs(dw).max() > 1e-6
    assert np.abs(dw.sum(axis=1)).max() < 1e-12 * np.abs(dw).sum()


def pin_bwd_zero_dout(fwd, bwd):
    """dL/dO = 0 gives zero gradients everywhere."""
    lens, block = [140], 128
    q, k, v, w, dout = _case(41, lens, 2, 1, 8, block)
    for gr in bwd.attend_prefill_backward(q, k, v, w, 0 * dout, _cu(lens), 8, block=block):
        assert np.all(gr == 0.0)


def pin_bwd_row_statistics(fwd, bwd):
    """The saved per-row statistics: lse is scipy's logsumexp of the scaled
    scores over the visible keys (built here from the forward's pooled
    entries), and delta = dO . O with O from the forward oracle."""
    lens, hq, hkv, d, block, window = [200], 4, 2, 8, 16, 12
    q, k, v, w, dout = _case(51, lens, hq, hkv, d, block)
    cu = _cu(lens)
    *_, st = bwd.attend_prefill_backward(q, k, v, w, dout, cu, window, block=block, return_stats=True)
    kc = fwd.compress(k, w, cu, block)
    vc = fwd.compress(v, w, cu, block)
    o = fwd.attend_prefill(q, k, v, kc, vc, cu, window, block=block)
    assert _rel(st["delta"], (dout * o).sum(axis=2)) < 1e-12
    g = hq // hkv
    for t in (0, 15, 16, 31, 100, 199):
        n, s0 = (t + 1) // block, max(0, t - window + 1)
        for head in range(hq):
            h = head // g
            keys = np.concatenate([kc[:n, h], k[s0:t + 1, h]])
            z = keys @ q[t, head] / math.sqrt(d)
            assert abs(st["lse"][t, head] - scipy.special.logsumexp(z)) < 1e-12


def pin_bwd_row_subset_finite_differences(fwd, bwd):
    """The rows= filter: with a subset of query rows (given as their own q
    and dout rows), the gradients are those of sum over the subset of
    dout . O, checked by central differences of the forward oracle on that
    restricted loss; dq comes back for the subset only."""
    lens, hq, hkv, d, block, window = [90, 60], 4, 2, 8, 16, 12
    q, k, v, w, dout = _case(61, lens, hq, hkv, d, block)
    cu = _cu(lens)
    rows = [3, 15, 16, 47, 89, 90, 105, 149]
    dq, dk, dv, dw = bwd.attend_prefill_backward(q[rows], k, v, w, dout[rows], cu, window, block=block, rows=rows,
                                                 q_holds_rows_only=True)
    assert dq.shape == (len(rows), hq, d)
    r = np.random.default_rng(62)
    eps = 1e-5

    def loss(q_, k_, v_, w_):
        kc = fwd.compress(k_, w_, cu, block)
        vc = fwd.compress(v_, w_, cu, block)
        o = fwd.attend_prefill(q_, k_, v_, kc, vc, cu, window, block=block, rows=rows, q_holds_rows_only=True)
        return float((dout[rows] * o).sum())

    args = {"q": q[rows], "k": k, "v": v, "w": w}
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("w", dw)):
        delta = r.standard_normal(args[name].shape)
        hi, lo = dict(args), dict(args)
        hi[name] = args[name] + eps * delta
        lo[name] = args[name] - eps * delta
        fd = (loss(**{x + "_": y for x, y in hi.items()}) - loss(**{x + "_": y for x, y in lo.items()})) / (2 * eps)
        an = float((grad * delta).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(fd), 1.0), f"d{name} (row subset): finite difference {fd} vs {an}"


BACKWARD_PINS = [
    pin_bwd_finite_differences_small_blocks,
    pin_bwd_finite_differences_block128,
    pin_bwd_causal_sdpa_autograd,
    pin_bwd_dw_sums_to_zero,
    pin_bwd_zero_dout,
    pin_bwd_row_statistics,
    pin_bwd_row_subset_finite_differences,
]
