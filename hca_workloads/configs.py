"""The five named HCA workloads, plus a continuation chunk of the serving path.

Each entry fixes shapes, dtype, window and value distributions.  Seeds are
1000 + index.  "rms" means every [d] head vector of Q/K/V is drawn N(0,1) in
fp32, divided by sqrt(mean(x^2) + 1e-6) and then cast (round to nearest even)
to the workload dtype; otherwise the draw is plain N(0,1).  Pooling logits w
are drawn N(0, w_std^2) in fp32.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class HcaConfig:
    index: int
    name: str
    dtype: str                 # "f32" or "bf16"
    hq: int
    hkv: int
    d: int
    window: int
    block: int = 128
    # prefill part: sequence lengths of the packed batch (empty: none)
    prefill_lens: tuple = ()
    rms: bool = False
    w_std: float = 1.0
    # decode part: number of sequences and their context lengths; when
    # decode_len_range is set the lengths are drawn uniformly (inclusive)
    decode_batch: int = 0
    decode_len: int = 0
    decode_len_range: tuple = ()
    ring: int = 0
    # continuation chunk: the prefill part is one chunk whose first token sits
    # at this position of a longer sequence (0: a fresh sequence)
    chunk_pos0: int = 0
    notes: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 1000 + self.index

    @property
    def has_prefill(self) -> bool:
        return len(self.prefill_lens) > 0

    @property
    def has_decode(self) -> bool:
        return self.decode_batch > 0


CONFIGS = {
    "tiny_f32": HcaConfig(
        index=1, name="tiny_f32", dtype="f32", hq=4, hkv=1, d=64, window=64,
        prefill_lens=(512,), rms=False, w_std=1.0,
        notes="B=1, T=512, Hq=4, Hkv=1, d=64, W=64; N(0,1) Q/K/V and w"),
    "prefill_8k": HcaConfig(
        index=2, name="prefill_8k", dtype="bf16", hq=64, hkv=1, d=512, window=128,
        prefill_lens=(8192,), rms=True, w_std=0.5,
        notes="B=1, T=8192, Hq=64, Hkv=1, d=512, W=128; 64 compressed entries"),
    "prefill_128k": HcaConfig(
        index=3, name="prefill_128k", dtype="bf16", hq=64, hkv=1, d=512, window=128,
        prefill_lens=(131072,), rms=True, w_std=0.5,
        notes="B=1, T=131072; 1024 compressed entries"),
    "decode_64x128k": HcaConfig(
        index=4, name="decode_64x128k", dtype="bf16", hq=64, hkv=1, d=512, window=128,
        decode_batch=64, decode_len=131072, ring=128,
        notes="64 sequences x 1 query, context 131072: 1024 entries + 128-token ring"),
    "mixed_1m": HcaConfig(
        index=5, name="mixed_1m", dtype="bf16", hq=64, hkv=1, d=512, window=128,
        prefill_lens=(32768,), rms=True, w_std=0.5,
        decode_batch=8, decode_len_range=(262144, 1048576), ring=128,
        notes="decode B=8, contexts U[262144, 1048576] + one 32768-token prefill chunk"),
    "chunk_32k_at_224k": HcaConfig(
        index=6, name="chunk_32k_at_224k", dtype="bf16", hq=64, hkv=1, d=512, window=128,
        prefill_lens=(32768,), rms=True, w_std=0.5, ring=128, chunk_pos0=229376,
        notes="one 32768-token chunk at positions 229376..262143 over a cache of 1792 entries "
              "+ a 128-slot ring; the chunk completes 256 more blocks"),
}


def get_config(name: str) -> HcaConfig:
    return CONFIGS[name]
