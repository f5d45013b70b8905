"""Seeded input generators (torch on any device, numpy for host metadata)."""
from __future__ import annotations

import numpy as np
import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _DT[name]


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, g, device, rms: bool, dtype: torch.dtype, chunk_rows: int = 4096):
    """N(0,1) fp32 draw, optionally RMS-normalised per trailing [d] vector,
    cast to `dtype`.  Drawn in row chunks so huge tensors never need a full
    fp32 temporary."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32)
        if rms:
            x = x / torch.sqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
        flat[r0:r1] = x.reshape(r1 - r0, -1).to(dtype)
    return out


def cu_from_lengths(lengths):
    """Exclusive prefix sum [0, l0, l0+l1, ...] as a host int64 array."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int64)


def draw_lengths(lo: int, hi: int, n: int, seed: int):
    """n integers uniform on [lo, hi] inclusive (host RNG, device independent)."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in rng.integers(lo, hi + 1, size=n)]


def prefill_inputs(cfg, device="cpu", lens=None, seed=None, kc_random: bool = False):
    """Q, K, V and pooling logits w for a packed prefill batch.

    lens overrides cfg.prefill_lens (sizes for small parity cases).  With
    kc_random the compressed caches are drawn too (N(0, 1/16)), so that the
    attention step can be checked apart from the pooling step.
    Returns a dict of tensors on `device` plus host metadata.
    """
    lens = list(cfg.prefill_lens if lens is None else lens)
    seed = cfg.seed if seed is None else seed
    dt = _DT[cfg.dtype]
    g = _gen(seed, device)
    ntok = int(sum(lens))
    cu = cu_from_lengths(lens)
    nblk = [l // cfg.block for l in lens]
    cub = cu_from_lengths(nblk)
    d = {
        "lens": lens,
        "cu_seqlens_host": cu,
        "cu_blocks_host": cub,
        "total_blocks": int(cub[-1]),
        "max_seqlen": int(max(lens)) if lens else 0,
        "q": _normal((ntok, cfg.hq, cfg.d), g, device, cfg.rms, dt),
        "k": _normal((ntok, cfg.hkv, cfg.d), g, device, cfg.rms, dt),
        "v": _normal((ntok, cfg.hkv, cfg.d), g, device, cfg.rms, dt),
        "w": torch.randn((cfg.hkv, cfg.block), generator=g, device=device,
                         dtype=torch.float32) * cfg.w_std,
        "cu_seqlens": torch.tensor(cu, dtype=torch.int32, device=device),
        "cu_blocks": torch.tensor(cub, dtype=torch.int32, device=device),
    }
    if kc_random:
        nb = max(1, d["total_blocks"])
        d["kc"] = (torch.randn((nb, cfg.hkv, cfg.d), generator=g, device=device) * 0.25).to(dt)
        d["vc"] = (torch.randn((nb, cfg.hkv, cfg.d), generator=g, device=device) * 0.25).to(dt)
    return d


def backward_inputs(cfg, device="cpu", lens=None, seed=None):
    """prefill_inputs plus the output gradient dout [N_tok, Hq, d], drawn
    like the queries (a synthetic dL/dO of the layer's output)."""
    seed = cfg.seed if seed is None else seed
    d = prefill_inputs(cfg, device, lens=lens, seed=seed)
    g = _gen(seed + 7919, device)
    ntok = d["q"].shape[0]
    d["dout"] = _normal((ntok, cfg.hq, cfg.d), g, device, cfg.rms, _DT[cfg.dtype])
    return d


def dsa_inputs(lens, seed, device="cpu", ties: bool = False, hq: int = 64, d: int = 256, di: int = 128):
    """Sparse-attention decode batch of the full-context layers: sequence b
    has lens[b] cached rows (packed, first row cu_rows[b]) and one query at
    its last position.  q, k, v: RMS-normalised N(0, 1) in bf16; qi, ki:
    uniform int8 in [-127, 127] (ties: in {-1, 0, 1}, so many scores are
    equal)."""
    g = _gen(seed, device)
    lens = [int(x) for x in lens]
    rows = int(sum(lens))
    cu = cu_from_lengths(lens)
    lo, hi = (-1, 2) if ties else (-127, 128)
    return {
        "lens": lens,
        "cu_rows_host": cu[:-1],
        "max_seqlen": max(lens),
        "seqlens": torch.tensor(lens, dtype=torch.int32, device=device),
        "cu_rows": torch.tensor(cu[:-1], dtype=torch.int32, device=device),
        "q": _normal((len(lens), hq, d), g, device, True, torch.bfloat16),
        "k": _normal((rows, d), g, device, True, torch.bfloat16),
        "v": _normal((rows, d), g, device, True, torch.bfloat16),
        "qi": torch.randint(lo, hi, (len(lens), di), generator=g, device=device, dtype=torch.int8),
        "ki": torch.randint(lo, hi, (rows, di), generator=g, device=device, dtype=torch.int8),
    }


def decode_inputs(cfg, device="cpu", lens=None, seed=None, ring=None):
    """Decode batch: one query per sequence plus a filled cache.

    Sequence b has context L_b (its query sits at position L_b - 1); its
    compressed cache holds floor(L_b/128) entries packed by cu_blocks and its
    ring holds R raw rows.  All cache values are N(0,1).  Only the slots the
    query can see matter; the rest are still drawn so every byte is defined.
    """
    seed = cfg.seed if seed is None else seed
    if lens is None:
        if cfg.decode_len_range:
            lens = draw_lengths(cfg.decode_len_range[0], cfg.decode_len_range[1],
                                cfg.decode_batch, seed + 7)
        else:
            lens = [cfg.decode_len] * cfg.decode_batch
    lens = [int(x) for x in lens]
    ring = int(cfg.ring if ring is None else ring)
    dt = _DT[cfg.dtype]
    g = _gen(seed, device)
    nblk = [l // cfg.block for l in lens]
    cub = cu_from_lengths(nblk)
    total = max(1, int(cub[-1]))
    b = len(lens)
    return {
        "lens": lens,
        "cu_blocks_host": cub,
        "max_blocks": int(max(nblk)) if nblk else 0,
        "ring": ring,
        "q": _normal((b, cfg.hq, cfg.d), g, device, False, dt),
        "kc": _normal((total, cfg.hkv, cfg.d), g, device, False, dt),
        "vc": _normal((total, cfg.hkv, cfg.d), g, device, False, dt),
        "kw": _normal((b, ring, cfg.hkv, cfg.d), g, device, False, dt),
        "vw": _normal((b, ring, cfg.hkv, cfg.d), g, device, False, dt),
        "seqlens": torch.tensor(lens, dtype=torch.int32, device=device),
        "cu_blocks": torch.tensor(cub, dtype=torch.int32, device=device),
    }


def ring_from_raw(raw, length: int, ring: int):
    """Lay the last min(ring, length) raw rows of one sequence ([L, Hkv, d])
    into a ring buffer [ring, Hkv, d], position s in slot s mod ring; slots
    never written stay zero.  This is cache layout, not arithmetic."""
    out = torch.zeros((ring,) + tuple(raw.shape[1:]), dtype=raw.dtype, device=raw.device)
    for s in range(max(0, length - ring), length):
        out[s % ring] = raw[s]
    return out


def chunk_inputs(cfg, device="cpu", seed=None):
    """A continuation chunk: raw K, V [L, Hkv, d] and pooling logits of a whole
    sequence of L = chunk_pos0 + n tokens, and the queries [n, Hq, d] of its
    last n positions (the chunk).  Distributions as for prefill_inputs."""
    seed = cfg.seed if seed is None else seed
    dt = _DT[cfg.dtype]
    g = _gen(seed, device)
    n = int(cfg.prefill_lens[0])
    L = int(cfg.chunk_pos0) + n
    return {
        "pos0": int(cfg.chunk_pos0),
        "n": n,
        "length": L,
        "q": _normal((n, cfg.hq, cfg.d), g, device, cfg.rms, dt),
        "k": _normal((L, cfg.hkv, cfg.d), g, device, cfg.rms, dt),
        "v": _normal((L, cfg.hkv, cfg.d), g, device, cfg.rms, dt),
        "w": torch.randn((cfg.hkv, cfg.block), generator=g, device=device,
                         dtype=torch.float32) * cfg.w_std,
    }
