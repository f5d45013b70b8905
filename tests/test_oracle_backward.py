"""The backward oracle against its pins (finite differences of the pinned
forward, SDPA autograd, invariants), and planted mistakes in a copy of it
that the pins must catch."""
import os
import types

import pytest

import oracle
import oracle.hca_backward
from oracle_backward_pins import BACKWARD_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "hca_backward.py")

# (name, original text, mutated text)
MUTANTS = [
    ("softmax Jacobian without the -D term", "dz = a * (dp - dd[:, None])", "dz = a * dp"),
    ("dq without the score scale", "dq[i, hs] = scale * (dz @ keys)", "dq[i, hs] = dz @ keys"),
    ("value gradient through dz", "dvals = a.T @ doh", "dvals = dz.T @ doh"),
    ("key gradient from dO instead of q", "dkeys = scale * (dz.T @ qh)", "dkeys = scale * (dz.T @ doh)"),
    ("compressed keys get no gradient", "dkc[cub[b]: cub[b] + n, h] += dkeys[:n]",
     "dkc[cub[b]: cub[b] + n, h] += 0 * dkeys[:n]"),
    ("window gradient to reversed positions", "dk[start + s0: tok + 1, h] += dkeys[n:]",
     "dk[start + s0: tok + 1, h] += dkeys[n:][::-1]"),
    ("pooling scatter with reversed weights", "dk[blk, h] += p[h][:, None] * dkc[e, h][None, :]",
     "dk[blk, h] += p[h][::-1, None] * dkc[e, h][None, :]"),
    ("dw without the V path", "gsum[h] += k[blk, h] @ dkc[e, h] + v[blk, h] @ dvc[e, h]",
     "gsum[h] += k[blk, h] @ dkc[e, h]"),
    ("dw without centring", "dw = p * (gsum - (p * gsum).sum(axis=1, keepdims=True))", "dw = p * gsum"),
    ("lse without the max", "lse[i, hs] = zmax[:, 0] + np.log(e.sum(axis=1))", "lse[i, hs] = np.log(e.sum(axis=1))"),
]


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=[p.__name__ for p in BACKWARD_PINS])
def test_backward_oracle_pin(pin):
    pin(oracle, oracle.hca_backward)


def _load(src):
    mod = types.ModuleType("hca_backward_mutant")
    src = src.replace("from .hca_oracle import", "from oracle.hca_oracle import")
    exec(compile(src, "hca_backward_mutant.py", "exec"), mod.__dict__)
    return mod


def test_backward_mutation_sites_exist():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert old in src, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert old in src
    mod = _load(src.replace(old, new, 1))
    caught = []
    for pin in BACKWARD_PINS:
        try:
            pin(oracle, mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant '{name}' passed every pin"
