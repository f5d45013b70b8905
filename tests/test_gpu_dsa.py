"""GPU parity of the sparse-attention decode of the full-context layers
(hca_dsa_decode) against the oracle: the selected positions bit for bit
(integer scores decide them on both sides), the output within the bf16 bound
(max-abs <= 1e-2, rel-L2 <= 5e-3)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import dsa_inputs
from parity_util import assert_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(lens, topk, seed, ties=False):
    print(f"case lens={lens[:6]} k={topk} ties={ties}", flush=True)
    inp = dsa_inputs(lens, seed, DEV, ties=ties)
    o, sel = hca.hca_dsa_decode(inp["seqlens"], inp["cu_rows"], inp["max_seqlen"], topk, inp["q"], inp["qi"],
                                inp["k"], inp["v"], inp["ki"])
    torch.cuda.synchronize()
    ref, rsel = oracle.dsa_decode(inp["q"].cpu(), inp["qi"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["ki"].cpu(),
                                  lens, inp["cu_rows_host"], topk)
    got = sel.cpu().numpy()
    for b, L in enumerate(lens):
        n = min(L, topk)
        assert np.array_equal(got[b, :n], rsel[b]), f"selection of sequence {b} (L={L})"
        assert np.all(got[b, n:] == -1)
    assert_close(o, torch.tensor(ref), torch.bfloat16, f"dsa lens={lens[:4]} k={topk}")


@pytest.mark.parametrize("lens,topk", [
    ([1, 100, 2047, 2048, 2049, 5000], 2048),   # around k: all selected, exactly k, one dropped
    ([3000, 17, 9000], 64),
    ([4000], 1),
    ([513, 257], 3),
])
def test_dsa_decode(lens, topk):
    _check(lens, topk, seed=601)


def test_dsa_decode_ties():
    """Indexer values in {-1, 0, 1}: most scores are shared, so the tie rule
    (smaller position first) decides most of the selection."""
    _check([3000, 700], 64, seed=611, ties=True)
    _check([5000], 2048, seed=612, ties=True)


def test_dsa_decode_128k():
    """One sequence at the workload's context length (131072) and k = 2048."""
    _check([131072, 5], 2048, seed=621)


@pytest.mark.parametrize("lens,topk", [
    ([256, 4096, 4097, 8192], 2048),   # chunk and row-padding boundaries
    ([1, 1, 1], 2048),                 # single-token sequences: the query sees only itself
    ([2049, 4095], 2048),
])
def test_dsa_decode_boundaries(lens, topk):
    _check(lens, topk, seed=631)


def test_dsa_decode_rows_with_gaps():
    """cu_rows is each sequence's first cache row, not a prefix sum: rows of
    other data (here, random rows) may sit between the sequences."""
    lens, gap, topk = [3000, 700, 5000], 37, 512
    inp = dsa_inputs([L + gap for L in lens], 641, DEV)
    starts = [int(c) + gap for c in inp["cu_rows_host"]]
    cu = torch.tensor(starts, dtype=torch.int32, device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, sel = hca.hca_dsa_decode(sl, cu, max(lens), topk, inp["q"], inp["qi"], inp["k"], inp["v"], inp["ki"])
    torch.cuda.synchronize()
    ref, rsel = oracle.dsa_decode(inp["q"].cpu(), inp["qi"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["ki"].cpu(),
                                  lens, starts, topk)
    for b in range(len(lens)):
        assert np.array_equal(sel.cpu().numpy()[b, :min(lens[b], topk)], rsel[b])
    assert_close(o, torch.tensor(ref), torch.bfloat16, "dsa rows with gaps")


def test_dsa_decode_bench_workload():
    """The benchmarked workload at full size, in the launch configuration
    bench.py times (64 sequences of 131072 positions, k = 2048, workspace,
    o and sel passed in): every sequence's selection bit for bit, and the
    output of 8 seeded-random sequences against the oracle, one sequence at
    a time."""
    import bench

    B, L, K = bench.DSA_BATCH, bench.DSA_LEN, bench.DSA_TOPK
    print(f"case bench workload B={B} L={L} k={K}", flush=True)
    inp = dsa_inputs([L] * B, bench.DSA_SEED, DEV)
    ws = torch.empty(hca.hca_dsa_decode_workspace_bytes(B, L, K), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(inp["q"])
    sel = torch.empty((B, K), dtype=torch.int32, device=DEV)
    for _ in range(2):  # a second call on the same workspace gives the same result
        hca.hca_dsa_decode(inp["seqlens"], inp["cu_rows"], L, K, inp["q"], inp["qi"], inp["k"], inp["v"], inp["ki"],
                           workspace=ws, o=o, sel=sel)
        torch.cuda.synchronize()
        got = sel.cpu().numpy()
        ki = inp["ki"].cpu()
        qi = inp["qi"].cpu()
        for b in range(B):
            r0 = inp["cu_rows_host"][b]
            ref = oracle.select_topk(oracle.index_scores(qi[b], ki[r0:r0 + L]), K)
            assert np.array_equal(got[b], ref), f"selection of sequence {b}"
    rng = np.random.default_rng(17)
    for b in sorted(rng.choice(B, size=8, replace=False).tolist()):
        r0 = inp["cu_rows_host"][b]
        rows = slice(r0, r0 + L)
        ref, _ = oracle.dsa_decode(inp["q"][b:b + 1].cpu(), inp["qi"][b:b + 1].cpu(), inp["k"][rows].cpu(),
                                   inp["v"][rows].cpu(), inp["ki"][rows].cpu(), [L], [0], K)
        assert_close(o[b:b + 1], torch.tensor(ref), torch.bfloat16, f"dsa bench workload sequence {b}")
