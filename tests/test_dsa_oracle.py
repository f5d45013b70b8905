"""Pins of the sparse-attention (DSA) decode oracle against brute force,
library routines and closed forms, and planted mistakes it must catch."""
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.dsa_oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dsa_oracle.py")


def _brute_select(scores, k):
    """A position is selected iff fewer than k positions beat it (a higher
    score, or the same score at a smaller position)."""
    n = len(scores)
    out = []
    for p in range(n):
        beat = sum(1 for r in range(n) if scores[r] > scores[p] or (scores[r] == scores[p] and r < p))
        if beat < k:
            out.append(p)
    return np.asarray(out, dtype=np.int64)


def pin_select_brute_force(m):
    r = np.random.default_rng(1)
    for n, k, hi in [(40, 7, 5), (60, 60, 100), (33, 40, 3), (50, 1, 2), (64, 16, 1000)]:
        s = r.integers(-hi, hi + 1, size=n)  # small ranges: many ties
        assert np.array_equal(m.select_topk(s, k), _brute_select(list(s), k)), (n, k)


def pin_scores_exact(m):
    r = np.random.default_rng(2)
    qi = r.integers(-128, 128, size=128).astype(np.int8)
    ki = r.integers(-128, 128, size=(50, 128)).astype(np.int8)
    ref = np.array([sum(int(qi[j]) * int(ki[s, j]) for j in range(128)) for s in range(50)])
    assert np.array_equal(m.index_scores(qi, ki), ref)
    # the extreme: every product -128 * -128
    assert m.index_scores(np.full(128, -128, np.int8), np.full((1, 128), -128, np.int8))[0] == 128 * 128 * 128


def pin_attend_sdpa(m):
    r = np.random.default_rng(3)
    q, kr, vr = r.standard_normal((8, 32)), r.standard_normal((20, 32)), r.standard_normal((20, 32))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[:, None], torch.tensor(kr)[None],
                                                           torch.tensor(vr)[None])[:, 0].numpy()
    assert np.abs(m.attend_selected(q, kr, vr) - ref).max() < 1e-12


def pin_closed_forms(m):
    r = np.random.default_rng(4)
    q, kr = r.standard_normal((4, 16)), r.standard_normal((9, 16))
    v = np.tile(r.standard_normal(16), (9, 1))  # constant values
    assert np.abs(m.attend_selected(q, kr, v) - v[0]).max() < 1e-12
    kd = np.zeros((9, 16))
    kd[5] = 400.0 * q[0] / np.linalg.norm(q[0])  # one dominant key for head 0
    o = m.attend_selected(q[:1], kd, r.standard_normal((9, 16)))
    vv = r.standard_normal((9, 16))
    assert np.abs(m.attend_selected(q[:1], kd, vv) - vv[5]).max() < 1e-9
    del o


def pin_decode_dense_and_order(m):
    """k >= L: ordinary attention over all cached rows; the selected list is
    increasing; permuting the selection does not change the output."""
    r = np.random.default_rng(5)
    lens, H, d = [1, 7, 30], 4, 16
    cu = np.concatenate([[0], np.cumsum(lens)])
    n = int(cu[-1])
    q = r.standard_normal((3, H, d))
    k, v = r.standard_normal((n, d)), r.standard_normal((n, d))
    qi = r.integers(-5, 6, size=(3, 128)).astype(np.int8)
    ki = r.integers(-5, 6, size=(n, 128)).astype(np.int8)
    o, sel = m.dsa_decode(q, qi, k, v, ki, lens, cu, topk=64)
    for b, L in enumerate(lens):
        assert np.array_equal(sel[b], np.arange(L))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q[b])[:, None], torch.tensor(k[cu[b]:cu[b] + L])[None], torch.tensor(v[cu[b]:cu[b] + L])[None])
        assert np.abs(o[b] - ref[:, 0].numpy()).max() < 1e-12
    o2, sel2 = m.dsa_decode(q, qi, k, v, ki, lens, cu, topk=5)
    for b, L in enumerate(lens):
        s = sel2[b]
        assert len(s) == min(5, L) and np.all(np.diff(s) > 0)
        perm = s[::-1]
        assert np.abs(m.attend_selected(q[b], k[cu[b] + perm], v[cu[b] + perm]) - o2[b]).max() < 1e-12
    # the scale is 1/sqrt(d)
    qq = r.standard_normal((1, d))
    z = (qq @ k[:4].T) / math.sqrt(d)
    a = np.exp(z - z.max())
    assert np.abs(m.attend_selected(qq, k[:4], v[:4]) - (a / a.sum()) @ v[:4]).max() < 1e-12


PINS = [pin_select_brute_force, pin_scores_exact, pin_attend_sdpa, pin_closed_forms, pin_decode_dense_and_order]

MUTANTS = [
    ("ties to the larger position", "order = np.lexsort((np.arange(n), -s))", "order = np.lexsort((-np.arange(n), -s))"),
    ("lowest scores selected", "order = np.lexsort((np.arange(n), -s))", "order = np.lexsort((np.arange(n), s))"),
    ("one position short", "return np.sort(order[:k]).astype(np.int64)", "return np.sort(order[:k - 1]).astype(np.int64)"),
    ("selection unsorted", "return np.sort(order[:k]).astype(np.int64)", "return order[:k].astype(np.int64)"),
    ("no softmax scale", "scale = 1.0 / math.sqrt(q.shape[-1])", "scale = 1.0"),
    ("values read from keys", "return (a / a.sum(axis=1, keepdims=True)) @ vr", "return (a / a.sum(axis=1, keepdims=True)) @ kr"),
    ("query excludes its own position", "pos = select_topk(index_scores(_i64(qi[b]), kki[r0:r0 + L]), topk)",
     "pos = select_topk(index_scores(_i64(qi[b]), kki[r0:r0 + L - 1]), topk)"),
    ("scores wrap in int8", "return _i64(ki_rows) @ _i64(qi)", "return (_i64(ki_rows) @ _i64(qi)).astype(np.int8).astype(np.int64)"),
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_dsa_oracle_pin(pin):
    pin(oracle.dsa_oracle)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_dsa_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert old in src, name
    mod = types.ModuleType("dsa_mutant")
    exec(compile(src.replace(old, new, 1), "dsa_mutant.py", "exec"), mod.__dict__)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant '{name}' passed every pin"
