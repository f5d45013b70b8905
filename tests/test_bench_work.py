"""The algorithmic work bench.py divides by (roofline 'achieved'), checked
against brute-force counts: the visible (query, key) pairs come from the
oracle's visibility rule summed row by row, the bytes from the tensor
shapes each launch must touch once."""
import dataclasses

import pytest

import bench
import oracle
from hca_workloads import CONFIGS


def _pairs(lens, window, p0=0):
    total = 0
    for L in lens:
        for t in range(p0, L):
            n, s0 = oracle.visible_sets(t, window)
            total += n + (t - s0 + 1)
    return total


@pytest.mark.parametrize("lens,window", [([8192], 128), ([1, 127, 128, 129, 3000], 64), ([700], 300), ([50], 1)])
def test_prefill_work(lens, window):
    c = dataclasses.replace(CONFIGS["prefill_8k"], window=window)
    byt, flops = bench.prefill_work(c, lens, 2)
    assert flops == 4 * c.d * c.hq * _pairs(lens, window)
    ntok = sum(lens)
    entries = sum(L // 128 for L in lens)
    # per token: Q read + O written (Hq rows of d bf16), raw K and V read (Hkv
    # rows); per complete block: its Kc and Vc entries read
    assert byt == ntok * (2 * c.hq * c.d * 2 + 2 * c.hkv * c.d * 2) + entries * 2 * c.hkv * c.d * 2


def test_chunk_work():
    c = CONFIGS["chunk_32k_at_224k"]
    p0, n = 5000, 900
    byt, flops = bench.chunk_work(c, p0, n, 2)
    pairs = 0
    for t in range(p0, p0 + n):
        nc, s0 = oracle.visible_sets(t, c.window)
        pairs += nc + (t - s0 + 1)
    assert flops == 4 * c.d * c.hq * pairs
    halo = min(c.window - 1, p0)
    assert byt == n * (2 * c.hq * c.d * 2 + 2 * c.hkv * c.d * 2) + halo * 2 * c.hkv * c.d * 2 + \
        ((p0 + n) // 128) * 2 * c.hkv * c.d * 2


def test_decode_and_compress_work():
    c = CONFIGS["decode_64x128k"]
    lens = [1, 128, 131072]
    byt, flops = bench.decode_work(c, lens, 2)
    keys = [L // 128 + min(c.window, L) for L in lens]
    assert flops == sum(4 * c.d * c.hq * k for k in keys)
    assert byt == sum(2 * c.hq * c.d * 2 + 2 * c.hkv * c.d * 2 * k for k in keys)
    c8 = CONFIGS["prefill_8k"]
    cb, cf = bench.compress_work(c8, [8192, 300], 2)
    nblk = 64 + 2
    assert cb == nblk * c8.hkv * (2 * 128 * c8.d * 2 + 2 * c8.d * 2)  # K, V rows read; Kc, Vc written
    assert cf == nblk * c8.hkv * 4 * 128 * c8.d


@pytest.mark.parametrize("lens,window", [([8192], 128), ([1, 127, 129, 3000], 64)])
def test_backward_work(lens, window):
    c = dataclasses.replace(CONFIGS["prefill_8k"], window=window)
    byt, flops = bench.backward_work(c, lens, 2)
    # scores S and dP, and the products for dQ, dK and dV: 2*d flops each per
    # visible (query row, key) pair
    assert flops == 5 * 2 * c.d * c.hq * _pairs(lens, window)
    ntok = sum(lens)
    entries = sum(L // 128 for L in lens)
    # q, o, dout read and dq written (Hq rows); k, v read and dk, dv written
    # (Hkv rows); the fp32 lse read; the entries read
    assert byt == ntok * (4 * c.hq * c.d * 2 + 4 * c.hkv * c.d * 2 + 4 * c.hq) + entries * 2 * c.hkv * c.d * 2


def test_dsa_work():
    lens, k = [1, 2048, 131072], 2048
    byt, flops = bench.dsa_work(lens, k)
    sel = [min(L, k) for L in lens]
    # indexer keys (128 int8 per position), selected K and V rows (256 bf16
    # each), q and o (64 x 256 bf16), the indexer query, the selection
    assert byt == sum(L * 128 + n * 2 * 256 * 2 + 2 * 64 * 256 * 2 + 128 + k * 4 for L, n in zip(lens, sel))
    assert flops == sum(2 * 128 * L + 4 * 256 * 64 * n for L, n in zip(lens, sel))
