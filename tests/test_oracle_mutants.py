"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them."""
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "hca_oracle.py")

# (name, original text, mutated text)
MUTANTS = [
    ("block visible one token late", "return (t + 1) // block, max(0, t - window + 1)",
     "return t // block, max(0, t - window + 1)"),
    ("window one token short", "return (t + 1) // block, max(0, t - window + 1)",
     "return (t + 1) // block, max(0, t - window + 2)"),
    ("window one token long", "return (t + 1) // block, max(0, t - window + 1)",
     "return (t + 1) // block, max(0, t - window)"),
    ("no softmax scale", "scale = 1.0 / math.sqrt(d)\n    if rows", "scale = 1.0\n    if rows"),
    ("scale 1/d", "scale = 1.0 / math.sqrt(d)\n    if rows", "scale = 1.0 / d\n    if rows"),
    ("pooling ignores logits", "out.append((p.T[:, :, None] * rows).sum(axis=0))",
     "out.append(rows.mean(axis=0))"),
    ("pooling weights reversed", "out.append((p.T[:, :, None] * rows).sum(axis=0))",
     "out.append((p.T[::-1, :, None] * rows).sum(axis=0))"),
    ("softmax over the wrong axis of w", "return e / e.sum(axis=-1, keepdims=True)",
     "return e / e.sum(axis=0, keepdims=True)"),
    ("values read from keys",
     "vals = np.concatenate([vc[cub[b]: cub[b] + n, h], v[start + s0: tok + 1, h]])",
     "vals = np.concatenate([kc[cub[b]: cub[b] + n, h], v[start + s0: tok + 1, h]])"),
    ("compressed entries of sequence 0 for every sequence",
     "keys = np.concatenate([kc[cub[b]: cub[b] + n, h], k[start + s0: tok + 1, h]])",
     "keys = np.concatenate([kc[0: n, h], k[start + s0: tok + 1, h]])"),
    ("raw window excludes the query's own token",
     "keys = np.concatenate([kc[cub[b]: cub[b] + n, h], k[start + s0: tok + 1, h]])",
     "keys = np.concatenate([kc[cub[b]: cub[b] + n, h], k[start + s0 - 1: tok, h]])"),
    ("probabilities normalised over queries", "probs = a / a.sum(axis=1, keepdims=True)",
     "probs = a / a.sum(axis=0, keepdims=True)"),
    ("scores transposed operand", "z = (qh @ keys.T) * scale",
     "z = (qh @ keys[:, ::-1].T) * scale"),
    ("GQA: every query head reads KV head 0",
     "o, p = _attend_rows(qt[h * g:(h + 1) * g], keys, vals, scale)",
     "o, p = _attend_rows(qt[h * g:(h + 1) * g], keys if h == 0 else keys * 0 + keys[::-1], vals, scale)"),
    ("decode ring slot off by one", "slots = [s % ring for s in range(s0, t + 1)]",
     "slots = [(s + 1) % ring for s in range(s0, t + 1)]"),
    ("decode query one position late", "t = int(lens[b]) - 1", "t = int(lens[b])"),
    ("de-duplicated window", "n, s0 = visible_sets(t, window, block)\n        assert cub[b] + n <= cub[b + 1]\n        qt",
     "n, s0 = visible_sets(t, window, block)\n        s0 = max(s0, block * n)\n        assert cub[b] + n <= cub[b + 1]\n        qt"),
    ("partial trailing block pooled", "for j in range((end - start) // block):",
     "for j in range(-(-(end - start) // block)):"),
    ("cache entry count ignores the window", "return length // block + min(window, length)",
     "return length // block"),
    ("head mix with U and V exchanged", 'out[:, h * g:(h + 1) * g, :] = grp + np.einsum("gr,nrd->ngd", u[h], z)',
     'out[:, h * g:(h + 1) * g, :] = grp + np.einsum("gr,nrd->ngd", v[h], np.einsum("ngd,gr->nrd", grp, u[h]))'),
    ("head mix without the identity skip", 'out[:, h * g:(h + 1) * g, :] = grp + np.einsum("gr,nrd->ngd", u[h], z)',
     'out[:, h * g:(h + 1) * g, :] = np.einsum("gr,nrd->ngd", u[h], z)'),
    ("gate through exp instead of sigmoid", "out = out * (1.0 / (1.0 + np.exp(-_f64(gate))))[:, :, None]",
     "out = out * np.exp(_f64(gate))[:, :, None]"),
    ("gate applied before the mixing", "    out = o.copy()\n    if mix_u is not None:",
     "    if gate is not None:\n        o = o * (1.0 / (1.0 + np.exp(-_f64(gate))))[:, :, None]\n        gate = None\n    out = o.copy()\n    if mix_u is not None:"),
]


def _load(src):
    mod = types.ModuleType("hca_oracle_mutant")
    exec(compile(src, "hca_oracle_mutant.py", "exec"), mod.__dict__)
    return mod


def test_mutation_sites_exist():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert old in src, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC).read()
    assert old in src
    mod = _load(src.replace(old, new, 1))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant '{name}' passed every pin"
