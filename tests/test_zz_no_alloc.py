"""The allocation-free decode entry point (hca_attend_decode_noalloc) against
the workspace one (hca_attend_decode): same kernels, so the outputs must be
bit-identical.  Two calls in a row on the library's static scratch, the
second with a smaller batch and shorter contexts than the first (the scratch
still holds the first call's partials), and a batch too large for the
scratch, which is refused on the host."""
from __future__ import annotations

import pytest
import torch

import compressed_kv_sparse_amd as hca
from hca_workloads import CONFIGS, decode_inputs
from parity_util import params_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(p, inp):
    ws = hca.new_decode_workspace(p, len(inp["lens"]), inp["max_blocks"], device=DEV)
    ref = hca.hca_attend_decode(p, inp["seqlens"], inp["cu_blocks"], inp["max_blocks"], inp["q"], inp["kc"],
                                inp["vc"], inp["kw"], inp["vw"], workspace=ws)
    out = torch.full_like(inp["q"], float("nan"))
    hca.hca_attend_decode_noalloc(p, inp["seqlens"], inp["cu_blocks"], inp["max_blocks"], inp["q"], inp["kc"],
                                  inp["vc"], inp["kw"], inp["vw"], out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_decode_matches_workspace_decode_twice():
    c = CONFIGS["decode_64x128k"]
    p = params_for(c)
    # first call: the benchmarked batch (64 x 131072, 16.9 MB of partials)
    big = decode_inputs(c, DEV, seed=141)
    assert hca.hca_decode_workspace_bytes(p, 64, big["max_blocks"]) <= hca.DECODE_NOALLOC_SCRATCH_BYTES
    ref, out = _both(p, big)
    print(f"call 1: B={len(big['lens'])} L={big['lens'][0]}", flush=True)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    # second call, smaller: stale partials of the first call stay in the scratch
    small = decode_inputs(c, DEV, lens=[1, 129, 700, 5000, 131071], seed=142)
    ref2, out2 = _both(p, small)
    print(f"call 2: B={len(small['lens'])} lens={small['lens']}", flush=True)
    assert torch.equal(out2.view(torch.int16), ref2.view(torch.int16))


def test_noalloc_decode_refuses_too_large_a_batch():
    c = CONFIGS["decode_64x128k"]
    p = params_for(c)
    # the plan gives every sequence one split or more, so 1024 sequences need
    # 1024 partial blocks of 66 KB: twice what the scratch holds
    B, mb = 1024, 1024
    assert hca.hca_decode_workspace_bytes(p, B, mb) > hca.DECODE_NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.int32, device=DEV)
    st = hca.library().hca_attend_decode_noalloc(p, B, mb, *([dummy.data_ptr()] * 7), 128, dummy.data_ptr(), None)
    assert st == 4  # HCA_ERR_WORKSPACE, returned before anything is launched
