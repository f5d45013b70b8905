"""GPU parity of the backward (hca_attend_prefill_backward) and of the saved
log-sum-exp (hca_attend_prefill_lse) against the float64 backward oracle.

Tolerance.  The kernels recompute P = exp(scale q.k - lse) in fp32 and feed P
and dS = P (dP - D) to the matrix cores in bf16 (relative rounding <= 2^-9
per element, like P in the forward's P.V), accumulate in fp32 and round dq,
dk, dv to bf16 once.  Each gradient is a sum of many such terms with random
signs, so the rounding errors add in quadrature; D = dO.O also uses the
forward's bf16 O.  Against the exact gradient this gives a relative L2 error
of 1.7e-3 .. 2.6e-3 (the output rounding alone is ~1.1e-3); the bound is the
forward's bf16 one, rel-L2 <= 5e-3 for dq, dk, dv and dw, with max-abs
<= 1e-2 * max|ref| per tensor (gradients are not O(1): the bound follows the
tensor's scale).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import compressed_kv_sparse_amd as hca
import oracle
from hca_workloads import CONFIGS, backward_inputs
from parity_util import params_for

pytestmark = pytest.mark.gpu
DEV = "cuda"
REL_L2 = 5e-3
MAX_REL = 1e-2


def _run(lens, hkv=1, window=128, seed=501):
    c = dataclasses.replace(CONFIGS["prefill_8k"], hkv=hkv, hq=64 * hkv, window=window)
    inp = backward_inputs(c, DEV, lens=lens, seed=seed)
    p = params_for(c)
    kc, vc = hca.hca_compress(p, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"], inp["k"], inp["w"],
                              v=inp["v"])
    if kc.shape[0] == 0:
        kc = torch.zeros((1, hkv, c.d), dtype=torch.bfloat16, device=DEV)
        vc = kc.clone()
    o, lse = hca.hca_attend_prefill_lse(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"], inp["q"],
                                        inp["k"], inp["v"], kc, vc)
    grads = hca.hca_attend_prefill_backward(p, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"],
                                            inp["total_blocks"], inp["q"], inp["k"], inp["v"], inp["w"], kc, vc, o,
                                            lse, inp["dout"])
    torch.cuda.synchronize()
    return c, inp, kc, vc, o, lse, grads


def _oracle(c, inp):
    return oracle.attend_prefill_backward(inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), inp["w"].cpu(),
                                          inp["dout"].cpu(), inp["cu_seqlens_host"], c.window, return_stats=True)


def _check(name, gpu, ref):
    g = gpu.detach().double().cpu().numpy()
    ref = np.asarray(ref, dtype=np.float64)
    scale = max(np.abs(ref).max(), 1e-30)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30))
    mx = float(np.abs(g - ref).max() / scale)
    msg = f"{name}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e} |ref|max={scale:.3g}"
    print(msg, flush=True)
    assert rel <= REL_L2 and mx <= MAX_REL, msg


@pytest.mark.parametrize("lens,hkv,window", [
    ([300, 1000], 1, 128),    # ragged, trailing partial blocks, windows over entries
    ([700, 129], 2, 128),     # two KV heads; a sequence with one block and one extra row
    ([1100], 1, 64),          # narrower window
    ([600], 1, 300),          # window wider than a block
])
def test_backward_bf16(lens, hkv, window):
    print(f"case lens={lens} Hkv={hkv} W={window}", flush=True)
    c, inp, kc, vc, o, lse, (dq, dk, dv, dw) = _run(lens, hkv, window)
    rdq, rdk, rdv, rdw, st = _oracle(c, inp)
    _check("dq", dq, rdq)
    _check("dk", dk, rdk)
    _check("dv", dv, rdv)
    _check("dw", dw, rdw)


def test_backward_no_complete_block():
    """Sequences shorter than a block: ordinary windowed attention; dw = 0."""
    c, inp, kc, vc, o, lse, (dq, dk, dv, dw) = _run([100, 37], 1, 64, seed=511)
    rdq, rdk, rdv, rdw, st = _oracle(c, inp)
    _check("dq", dq, rdq)
    _check("dk", dk, rdk)
    _check("dv", dv, rdv)
    assert torch.count_nonzero(dw).item() == 0


def test_forward_lse():
    """The saved lse matches the oracle's; o is the plain forward's, bit for bit."""
    c, inp, kc, vc, o, lse, _ = _run([500, 260], 1, 128, seed=521)
    o_plain = hca.hca_attend_prefill(params_for(c), inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"],
                                     inp["q"], inp["k"], inp["v"], kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_plain.view(torch.int16))
    *_, st = _oracle(c, inp)
    err = float(np.abs(lse.double().cpu().numpy() - st["lse"]).max())
    print(f"lse max abs error {err:.3e}", flush=True)
    # the forward's row sum adds the bf16-rounded weights: relative 2^-9 at most
    assert err <= 4e-3


def test_backward_prefill_8k_full():
    """The benchmarked workload at full size (one 8192-token sequence, Hq 64,
    d 512, W 128), in the launch configuration bench.py times: every row of
    dq, dk, dv and all of dw against the oracle (about 15 s of CPU)."""
    c0 = CONFIGS["prefill_8k"]
    c, inp, kc, vc, o, lse, (dq, dk, dv, dw) = _run(list(c0.prefill_lens), c0.hkv, c0.window, seed=c0.seed)
    rdq, rdk, rdv, rdw, st = _oracle(c, inp)
    _check("dq", dq, rdq)
    _check("dk", dk, rdk)
    _check("dv", dv, rdv)
    _check("dw", dw, rdw)


def test_backward_long_run_split_full():
    """16640 tokens: 130 complete blocks, so the compressed keys span three
    64-entry tiles, and the positions that see a compressed tile are split
    into uneven runs of 65 (the long-context work split; at 8192 tokens and
    below every run has 64 positions and only the first tile exists).  Every
    row of dq, dk, dv and all of dw against the oracle."""
    c, inp, kc, vc, o, lse, (dq, dk, dv, dw) = _run([16640], 1, 128, seed=531)
    rdq, rdk, rdv, rdw, st = _oracle(c, inp)
    _check("dq", dq, rdq)
    _check("dk", dk, rdk)
    _check("dv", dv, rdv)
    _check("dw", dw, rdw)


def test_backward_prefill_128k_sampled():
    """The 128K training context (one 131072-token sequence, Hq 64, d 512,
    W 128) in the launch configuration bench.py times: dq on sampled rows
    (every key-set boundary plus seeded random rows), and dk, dv in full for
    the last block.  Those rows are read only by the last 128 query rows
    (their windows, and entry 1023, which only the last row sees), so the
    oracle run over those query rows gives their exact gradients.  dw needs
    every row of the sequence and is checked in full at 16640 tokens."""
    from parity_util import sample_rows

    c0 = CONFIGS["prefill_128k"]
    T = c0.prefill_lens[0]
    c, inp, kc, vc, o, lse, (dq, dk, dv, dw) = _run([T], c0.hkv, c0.window, seed=c0.seed)
    last = list(range(T - 128, T))
    rows = sorted(set(sample_rows(T, c.window, 40, seed=541)) | set(last))
    idx = torch.tensor(rows, device=DEV)
    q_rows, do_rows = inp["q"].index_select(0, idx).cpu(), inp["dout"].index_select(0, idx).cpu()
    dq_rows = dq.index_select(0, idx)
    del inp["q"], inp["dout"], o, dq
    torch.cuda.empty_cache()
    print(f"oracle over {len(rows)} query rows", flush=True)
    rdq, rdk, rdv, _ = oracle.attend_prefill_backward(q_rows, inp["k"].cpu(), inp["v"].cpu(), inp["w"].cpu(),
                                                      do_rows, inp["cu_seqlens_host"], c.window, rows=rows,
                                                      q_holds_rows_only=True)
    _check("dq (sampled rows)", dq_rows, rdq)
    _check("dk (last block)", dk[T - 128:], rdk[T - 128:])
    _check("dv (last block)", dv[T - 128:], rdv[T - 128:])
    assert torch.isfinite(dw).all() and abs(float(dw.sum())) <= 1e-3 * float(dw.abs().sum())
