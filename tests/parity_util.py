"""Shared helpers for the GPU parity tests: tolerances and the HIP-path runner.

Tolerances (written here, used by every parity test):
  bf16 tensors: max |gpu - oracle| <= 1e-2 and ||gpu - oracle|| / ||oracle|| <= 5e-3
  fp32 tensors: ||gpu - oracle|| / ||oracle|| <= 1e-5 and max |gpu - oracle| <= 1e-5 * max |oracle|
The oracle computes in float64 from the same input bits.

Edge-case tests may pass `beyond_rounding=True`: the bf16 max-abs bound then
applies to |gpu - oracle| minus half a bf16 ulp of the oracle value, i.e. to
the error beyond the output format's own rounding.  A correctly rounded bf16
result of a value with |x| >= 4 is already up to 2^-6 = 0.0156 away from the
float64 value, so inputs whose outputs reach that size (one visible raw key
dominating, for instance) cannot meet a literal 1e-2 bound with any kernel.
The five named workloads are held to the literal bound.
"""
from __future__ import annotations

import numpy as np
import torch

import compressed_kv_sparse_amd as hca

BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
F32_REL = 1e-5


def to_np(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def half_ulp_bf16(r: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 numbers (8 significant bits) around |r|."""
    a = np.abs(r)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def errors(gpu, ref):
    g = to_np(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    assert np.isfinite(g).all(), "non-finite values in the GPU result"
    diff = np.abs(g - r)
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    beyond = float(np.maximum(diff - half_ulp_bf16(r), 0.0).max())
    return float(diff.max()), rel, float(np.abs(r).max()), beyond


def assert_close(gpu, ref, dtype, what="", beyond_rounding=False):
    max_abs, rel, ref_max, beyond = errors(gpu, ref)
    if dtype == torch.bfloat16:
        checked = beyond if beyond_rounding else max_abs
        ok = checked <= BF16_MAX_ABS and rel <= BF16_REL_L2
        bound = (f"{'max_abs beyond bf16 rounding' if beyond_rounding else 'max_abs'}<={BF16_MAX_ABS}, "
                 f"rel_l2<={BF16_REL_L2}")
    else:
        ok = rel <= F32_REL and max_abs <= F32_REL * ref_max
        bound = f"rel_l2<={F32_REL}, max_abs<={F32_REL}*{ref_max:.3g}"
    msg = (f"{what}: max_abs={max_abs:.3e} beyond_rounding={beyond:.3e} rel_l2={rel:.3e} "
           f"|ref|max={ref_max:.3g} ({bound})")
    print(msg, flush=True)
    assert ok, msg
    return max_abs, rel


def params_for(cfg_like, window=None, dtype=None):
    dt = dtype or (torch.bfloat16 if cfg_like.dtype == "bf16" else torch.float32)
    return hca.make_params(cfg_like.hq, cfg_like.hkv, cfg_like.d,
                           cfg_like.window if window is None else window, dt)


def run_prefill(params, inp, kc=None, vc=None):
    """hca_compress (unless kc/vc are given) then hca_attend_prefill."""
    if kc is None:
        kc, vc = hca.hca_compress(params, inp["cu_seqlens"], inp["cu_blocks"], inp["total_blocks"],
                                  inp["k"], inp["w"], v=inp["v"])
    o = hca.hca_attend_prefill(params, inp["cu_seqlens"], inp["cu_blocks"], inp["max_seqlen"],
                               inp["q"], inp["k"], inp["v"], kc, vc)
    return kc, vc, o


def run_decode(params, inp, workspace=None):
    if workspace is None:
        workspace = hca.new_decode_workspace(params, len(inp["lens"]), inp["max_blocks"])
    return hca.hca_attend_decode(params, inp["seqlens"], inp["cu_blocks"], inp["max_blocks"],
                                 inp["q"], inp["kc"], inp["vc"], inp["kw"], inp["vw"],
                                 workspace=workspace)


def sample_rows(T: int, window: int, n_random: int, seed: int):
    """Token positions that exercise every boundary of the key-set rules,
    plus seeded random positions."""
    fixed = {0, 1, window - 2, window - 1, window, window + 1, 126, 127, 128, 129, 254, 255, 256,
             T - 2, T - 1}
    for base in (128 * 5, T // 2 - T // 2 % 128, T - T % 128 - 128):
        for off in (-2, -1, 0, 1):
            fixed.add(base + off)
    rng = np.random.default_rng(seed)
    fixed |= set(int(x) for x in rng.integers(0, T, size=n_random))
    return sorted(x for x in fixed if 0 <= x < T)
