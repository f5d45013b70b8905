"""HCA (Heavily Compressed Attention) layer forward and backward for AMD MI355X.

The computation lives in libhca.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/hca.h); this package is its Python binding.  Build the
library with `python -m compressed_kv_sparse_amd.build`.
"""
from .hca import (  # noqa: F401
    DECODE_NOALLOC_SCRATCH_BYTES,
    EXPORTS,
    HCA_BF16,
    HCA_F32,
    HcaError,
    HcaLibraryMissing,
    HcaParams,
    hca_attend_decode,
    hca_attend_decode_noalloc,
    hca_attend_decode_gated_vha,
    hca_attend_prefill,
    hca_attend_prefill_backward,
    hca_attend_prefill_backward_workspace_bytes,
    hca_attend_prefill_gated_vha,
    hca_attend_prefill_lse,
    hca_attend_prefill_chunk,
    hca_attend_prefill_chunk_gated_vha,
    hca_compress,
    hca_compress_chunk,
    hca_decode_workspace_bytes,
    hca_dsa_decode,
    hca_dsa_decode_workspace_bytes,
    hca_prefill_chunk_workspace_bytes,
    hca_probe_lds_read,
    hca_probe_mfma_bf16,
    hca_probe_stream_read,
    hca_probe_stream_lds,
    PROBE_LDS_TILE,
    hca_ring_append,
    hca_status_string,
    hca_version,
    library,
    make_params,
    new_backward_workspace,
    new_decode_workspace,
    new_prefill_chunk_workspace,
)
