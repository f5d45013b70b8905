"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/hca.h declares, and rejects invalid arguments on the host before
anything is launched (these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

import compressed_kv_sparse_amd as hca
from compressed_kv_sparse_amd import hca as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hca.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"HCA_API\s+[\w\s\*]+?\b(hca_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return hca.library()


def test_header_declares_the_binding_names():
    assert declared_symbols() == sorted(hca.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    assert hca.hca_version().count(".") == 2
    for s in range(6):
        assert hca.hca_status_string(s).startswith("HCA_")
    assert hca.hca_status_string(99) == "HCA_ERR_UNKNOWN"


def _p(**kw):
    base = dict(num_q_heads=64, num_kv_heads=1, head_dim=512, window=128, dtype=hca.HCA_BF16)
    base.update(kw)
    return hca.make_params(**base)


NULL = None
DUMMY = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _compress(lib, params, batch=1, total_blocks=1, cu=DUMMY, cub=DUMMY, k=DUMMY, v=DUMMY,
              w=DUMMY, kc=DUMMY, vc=DUMMY):
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_compress(pp, batch, total_blocks, cu, cub, k, v, w, kc, vc, None)


def _prefill(lib, params, batch=1, max_seqlen=256, ptrs=None):
    p = [DUMMY] * 8 if ptrs is None else ptrs
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_attend_prefill(pp, batch, max_seqlen, *p, None)


def _decode(lib, params, batch=1, max_blocks=4, ring=128, ws=DUMMY, ws_bytes=1 << 40, ptrs=None):
    p = [DUMMY] * 7 if ptrs is None else ptrs
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_attend_decode(pp, batch, max_blocks, p[0], p[1], p[2], p[3], p[4], p[5], p[6],
                                 ring, DUMMY, ws, ws_bytes, None)


def test_compress_validation(lib):
    assert _compress(lib, None) == ERR_NULL
    assert _compress(lib, _p(block=64)) == ERR_UNSUPPORTED
    assert _compress(lib, _p(head_dim=500)) == ERR_UNSUPPORTED
    assert _compress(lib, _p(head_dim=2048)) == ERR_UNSUPPORTED
    assert _compress(lib, _p(num_q_heads=3, num_kv_heads=2)) == ERR_SHAPE
    assert _compress(lib, _p(window=0)) == ERR_SHAPE
    assert _compress(lib, _p(dtype=7)) == ERR_UNSUPPORTED
    assert _compress(lib, _p(), batch=-1) == ERR_SHAPE
    assert _compress(lib, _p(), total_blocks=-1) == ERR_SHAPE
    assert _compress(lib, _p(), v=NULL) == ERR_NULL          # v and vc must both be given or both NULL
    assert _compress(lib, _p(), k=NULL) == ERR_NULL
    assert _compress(lib, _p(), w=NULL) == ERR_NULL
    assert _compress(lib, _p(), batch=0) == ERR_SHAPE        # entries without sequences
    assert _compress(lib, _p(), total_blocks=0) == OK        # nothing to do: no launch
    # sequences shorter than one block: empty outputs may come as NULL
    assert _compress(lib, _p(), total_blocks=0, kc=NULL, vc=NULL) == OK
    assert _compress(lib, _p(), batch=0, total_blocks=0, cu=NULL, cub=NULL) == OK


def test_prefill_validation(lib):
    assert _prefill(lib, None) == ERR_NULL
    assert _prefill(lib, _p(head_dim=256)) == ERR_UNSUPPORTED   # bf16 path: d == 512 only
    assert _prefill(lib, _p(num_q_heads=32)) == ERR_UNSUPPORTED  # bf16 path: 64 heads per KV head
    assert _prefill(lib, _p(), batch=-1) == ERR_SHAPE
    assert _prefill(lib, _p(), batch=70000) == ERR_SHAPE
    assert _prefill(lib, _p(), max_seqlen=-5) == ERR_SHAPE
    assert _prefill(lib, _p(), batch=0) == OK
    assert _prefill(lib, _p(), max_seqlen=0) == OK
    ptrs = [DUMMY] * 8
    ptrs[2] = NULL  # q
    assert _prefill(lib, _p(), ptrs=ptrs) == ERR_NULL
    ptrs = [DUMMY] * 8
    ptrs[5] = NULL  # kc needed once a block can complete
    assert _prefill(lib, _p(), max_seqlen=128, ptrs=ptrs) == ERR_NULL
    f32 = _p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64)
    assert _prefill(lib, f32, max_seqlen=(1 << 30)) == ERR_SHAPE  # grid would overflow


def test_row_offsets_fit_32_bits(lib):
    """The matrix-core kernels address rows with 32-bit byte offsets (1 KiB
    rows per KV head): longer sequences are refused, not wrapped."""
    assert _prefill(lib, _p(), max_seqlen=(1 << 21)) == ERR_SHAPE
    assert _prefill(lib, _p(num_q_heads=128, num_kv_heads=2), max_seqlen=(1 << 20)) == ERR_SHAPE
    assert _decode(lib, _p(), max_blocks=(1 << 21)) == ERR_SHAPE
    assert _decode(lib, _p(), ring=(1 << 21)) == ERR_SHAPE
    assert _prefill_chunk(lib, _p(), max_seqlen=(1 << 21) - 64, total=(1 << 21)) == ERR_SHAPE


def test_decode_validation(lib):
    assert _decode(lib, None) == ERR_NULL
    assert _decode(lib, _p(), ring=64) == ERR_SHAPE              # ring shorter than the window
    assert _decode(lib, _p(head_dim=128)) == ERR_UNSUPPORTED
    assert _decode(lib, _p(), batch=-1) == ERR_SHAPE
    assert _decode(lib, _p(), batch=0) == OK
    assert _decode(lib, _p(), ws=NULL) == ERR_WORKSPACE
    assert _decode(lib, _p(), ws_bytes=16) == ERR_WORKSPACE
    assert _decode(lib, _p(), ws=ctypes.c_void_p(0x1010)) == ERR_WORKSPACE  # not 256-byte aligned
    ptrs = [DUMMY] * 7
    ptrs[0] = NULL  # seqlens
    assert _decode(lib, _p(), ptrs=ptrs) == ERR_NULL


def test_workspace_sizes(lib):
    p = _p()
    assert hca.hca_decode_workspace_bytes(_p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64), 8, 10) == 0
    assert hca.hca_decode_workspace_bytes(_p(head_dim=100), 8, 10) == 0
    assert hca.hca_decode_workspace_bytes(p, -1, 10) == 0
    small = hca.hca_decode_workspace_bytes(p, 4, 8)
    big = hca.hca_decode_workspace_bytes(p, 4, 8192)
    assert 0 < small <= big
    # at least one bf16 partial O/l [64, 512] per (sequence, KV head)
    assert small >= 4 * 64 * 512 * 2
    # grows with the number of sequences
    assert hca.hca_decode_workspace_bytes(p, 64, 1024) > hca.hca_decode_workspace_bytes(p, 8, 1024)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libhca.so"))
    with pytest.raises(hca.HcaLibraryMissing):
        binding.library()


def _compress_chunk(lib, params, batch=1, max_rows=1, ring=128, ptrs=None):
    p = [DUMMY] * 11 if ptrs is None else ptrs
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_compress_chunk(pp, batch, max_rows, p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                                  ring, p[8], p[9], None)


def _ring_append(lib, params, batch=1, max_rows=1, ring=128, ptrs=None):
    p = [DUMMY] * 6 if ptrs is None else ptrs
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_ring_append(pp, batch, max_rows, p[0], p[1], p[2], p[3], p[4], p[5], ring, None)


def _prefill_chunk(lib, params, batch=1, max_seqlen=64, total=64, ring=128, ws=DUMMY, ws_bytes=1 << 40,
                   ptrs=None):
    p = [DUMMY] * 10 if ptrs is None else ptrs
    pp = ctypes.byref(params) if params is not None else None
    return lib.hca_attend_prefill_chunk(pp, batch, max_seqlen, total, *p, ring, DUMMY, ws, ws_bytes, None)


def test_chunk_validation(lib):
    """Host-side checks of the serving-path entry points (nothing is launched)."""
    assert _compress_chunk(lib, None) == ERR_NULL
    assert _compress_chunk(lib, _p(), ring=127) == ERR_SHAPE        # a block's older rows need 128 slots
    assert _compress_chunk(lib, _p(head_dim=100)) == ERR_UNSUPPORTED
    assert _compress_chunk(lib, _p(), batch=-1) == ERR_SHAPE
    assert _compress_chunk(lib, _p(), max_rows=0) == OK              # nothing to pool
    assert _compress_chunk(lib, _p(), batch=0) == OK
    ptrs = [DUMMY] * 11
    ptrs[4] = NULL  # v without vw / vc
    assert _compress_chunk(lib, _p(), ptrs=ptrs) == ERR_NULL
    ptrs = [DUMMY] * 11
    ptrs[1] = NULL  # pos0
    assert _compress_chunk(lib, _p(), ptrs=ptrs) == ERR_NULL

    assert _ring_append(lib, None) == ERR_NULL
    assert _ring_append(lib, _p(), ring=0) == ERR_SHAPE
    assert _ring_append(lib, _p(), max_rows=0) == OK
    ptrs = [DUMMY] * 6
    ptrs[5] = NULL  # vw without v
    assert _ring_append(lib, _p(), ptrs=ptrs) == ERR_NULL

    assert _prefill_chunk(lib, None) == ERR_NULL
    assert _prefill_chunk(lib, _p(), ring=100) == ERR_SHAPE          # ring shorter than the window
    assert _prefill_chunk(lib, _p(head_dim=256)) == ERR_UNSUPPORTED  # bf16 path: d == 512 only
    assert _prefill_chunk(lib, _p(), batch=0) == OK
    assert _prefill_chunk(lib, _p(), ws=NULL) == ERR_WORKSPACE
    assert _prefill_chunk(lib, _p(), ws_bytes=16) == ERR_WORKSPACE
    assert _prefill_chunk(lib, _p(), ws=ctypes.c_void_p(0x1010)) == ERR_WORKSPACE
    ptrs = [DUMMY] * 10
    ptrs[1] = NULL  # pos0
    assert _prefill_chunk(lib, _p(), ptrs=ptrs) == ERR_NULL


def test_chunk_workspace_sizes(lib):
    p = _p()
    # window - 1 halo rows per sequence plus the new rows, K and V, 1 KiB rows
    assert hca.hca_prefill_chunk_workspace_bytes(p, 1, 1000) == 2 * (1000 + 127) * 1024
    assert hca.hca_prefill_chunk_workspace_bytes(p, 3, 10) == 2 * (10 + 3 * 127) * 1024
    assert hca.hca_prefill_chunk_workspace_bytes(p, -1, 10) == 0
    f32 = _p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64, window=64)
    assert hca.hca_prefill_chunk_workspace_bytes(f32, 2, 5) == 2 * (((5 + 2 * 63) * 64 * 4 + 255) // 256 * 256)


def test_gated_vha_validation(lib):
    def call(params, gate=DUMMY, u=DUMMY, v=DUMMY, rank=8, max_seqlen=256):
        pp = ctypes.byref(params) if params is not None else None
        return lib.hca_attend_prefill_gated_vha(pp, 1, max_seqlen, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY,
                                                gate, u, v, rank, DUMMY, None)
    assert call(None) == ERR_NULL
    assert call(_p(), u=NULL) == ERR_NULL                    # U and V come together
    assert call(_p(), rank=0) == ERR_SHAPE
    assert call(_p(), rank=33) == ERR_SHAPE
    assert call(_p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64)) == ERR_UNSUPPORTED  # bf16 kernel only
    assert call(_p(), max_seqlen=0) == OK
    # no epilogue: plain prefill, also in fp32
    assert call(_p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64), gate=NULL, u=NULL, v=NULL, max_seqlen=0) == OK


def test_decode_and_chunk_epilogue_validation(lib):
    f32 = _p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64)
    # decode: params, batch, max_blocks, seqlens, cu_blocks, q, kc, vc, kw, vw, ring, gate, u, v, rank, o, ws, ws_bytes, stream
    def dec(params, u=DUMMY, v=DUMMY, rank=8, batch=1):
        return lib.hca_attend_decode_gated_vha(ctypes.byref(params), batch, 4, *([DUMMY] * 7), 128, DUMMY, u, v,
                                               rank, DUMMY, DUMMY, 1 << 40, None)
    assert dec(_p(), v=NULL) == ERR_NULL
    assert dec(_p(), rank=40) == ERR_SHAPE
    assert dec(f32) == ERR_UNSUPPORTED
    assert dec(_p(), batch=0) == OK

    def chk(params, u=DUMMY, v=DUMMY, rank=8, batch=1):
        return lib.hca_attend_prefill_chunk_gated_vha(ctypes.byref(params), batch, 64, 64, *([DUMMY] * 10), 128,
                                                      DUMMY, u, v, rank, DUMMY, DUMMY, 1 << 40, None)
    assert chk(_p(), u=NULL) == ERR_NULL
    assert chk(_p(), rank=0) == ERR_SHAPE
    assert chk(_p(dtype=hca.HCA_F32, num_q_heads=4, head_dim=64, window=64)) == ERR_UNSUPPORTED
    assert chk(_p(), batch=0) == OK


def test_backward_validation(lib):
    """hca_attend_prefill_lse / hca_attend_prefill_backward reject bad
    arguments on the host (and the workspace size query agrees)."""
    p = _p()
    n_ws = lib.hca_attend_prefill_backward_workspace_bytes(ctypes.byref(p), 1, 8192, 64, 8192)
    assert n_ws > 8 * 8192 * 512  # at least the fp32 row partials
    assert lib.hca_attend_prefill_backward_workspace_bytes(ctypes.byref(_p(dtype=hca.HCA_F32)), 1, 8192, 64, 8192) == 0
    assert lib.hca_attend_prefill_backward_workspace_bytes(ctypes.byref(_p(head_dim=128)), 1, 8192, 64, 8192) == 0

    def bwd(params=p, batch=1, max_seqlen=300, ntok=300, nblk=2, w=DUMMY, dw=DUMMY, ws=DUMMY, ws_bytes=1 << 40,
            ptr=DUMMY):
        pp = ctypes.byref(params) if params is not None else None
        return lib.hca_attend_prefill_backward(pp, batch, max_seqlen, ntok, nblk, ptr, ptr, ptr, ptr, ptr, w, ptr,
                                               ptr, ptr, ptr, ptr, ptr, ptr, ptr, dw, ws, ws_bytes, None)

    assert bwd(params=None) == ERR_NULL
    assert bwd(params=_p(dtype=hca.HCA_F32)) == ERR_UNSUPPORTED
    assert bwd(params=_p(num_q_heads=32)) == ERR_UNSUPPORTED
    assert bwd(batch=-1) == ERR_SHAPE
    assert bwd(ntok=100) == ERR_SHAPE          # fewer tokens than the longest sequence
    assert bwd(nblk=3) == ERR_SHAPE            # more entries than complete blocks
    assert bwd(w=NULL) == ERR_NULL
    assert bwd(dw=NULL) == ERR_NULL
    assert bwd(ws=NULL) == ERR_WORKSPACE
    assert bwd(ws_bytes=16) == ERR_WORKSPACE
    assert bwd(ptr=NULL) == ERR_NULL
    # the lse forward: bf16 only, lse required
    args = [ctypes.byref(p), 1, 300] + [DUMMY] * 8
    assert lib.hca_attend_prefill_lse(*args, NULL, None) == ERR_NULL
    pf = _p(dtype=hca.HCA_F32)
    assert lib.hca_attend_prefill_lse(ctypes.byref(pf), 1, 300, *([DUMMY] * 8), DUMMY, None) == ERR_UNSUPPORTED


def test_dsa_validation(lib):
    """hca_dsa_decode rejects bad sizes, missing pointers and a short
    workspace on the host; empty batches are a no-op."""
    need = lib.hca_dsa_decode_workspace_bytes(4, 131072, 2048)
    assert need >= 4 * 131072 * 4  # the keys alone
    assert lib.hca_dsa_decode_workspace_bytes(4, 131072, 0) == 0

    def dsa(batch=2, max_seqlen=1000, topk=64, scale=0.0, ptr=DUMMY, ws=DUMMY, ws_bytes=1 << 40):
        return lib.hca_dsa_decode(batch, max_seqlen, topk, scale, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ws,
                                  ws_bytes, None)

    assert dsa(topk=0) == ERR_SHAPE
    assert dsa(batch=-1) == ERR_SHAPE
    assert dsa(batch=70000) == ERR_SHAPE
    assert dsa(scale=float("nan")) == ERR_SHAPE
    assert dsa(batch=0) == OK
    assert dsa(max_seqlen=0) == OK
    assert dsa(ptr=NULL) == ERR_NULL
    assert dsa(ws=NULL) == ERR_WORKSPACE
    assert dsa(ws_bytes=100) == ERR_WORKSPACE


def test_probe_validation(lib):
    """The measurement probes reject missing buffers and sizes out of range
    on the host."""
    assert lib.hca_probe_stream_read(NULL, 1 << 20, DUMMY, 64, None) == ERR_NULL
    assert lib.hca_probe_stream_read(DUMMY, 1 << 20, NULL, 64, None) == ERR_NULL
    assert lib.hca_probe_stream_read(DUMMY, 0, DUMMY, 64, None) == ERR_SHAPE
    assert lib.hca_probe_stream_read(DUMMY, 1000, DUMMY, 64, None) == ERR_SHAPE  # not a multiple of 16
    assert lib.hca_probe_stream_read(DUMMY, 1 << 20, DUMMY, 0, None) == ERR_SHAPE
    assert lib.hca_probe_stream_lds(NULL, 1 << 20, DUMMY, 64, None) == ERR_NULL
    assert lib.hca_probe_stream_lds(DUMMY, 1 << 20, NULL, 64, None) == ERR_NULL
    assert lib.hca_probe_stream_lds(DUMMY, 49151, DUMMY, 64, None) == ERR_SHAPE  # not one whole tile
    assert lib.hca_probe_stream_lds(DUMMY, 1 << 20, DUMMY, 0, None) == ERR_SHAPE
    assert lib.hca_probe_mfma_bf16(100, 256, NULL, None) == ERR_NULL
    assert lib.hca_probe_mfma_bf16(0, 256, DUMMY, None) == ERR_SHAPE
    assert lib.hca_probe_mfma_bf16(100, 70000, DUMMY, None) == ERR_SHAPE
    assert lib.hca_probe_lds_read(2, 100, 256, DUMMY, None) == ERR_SHAPE
    assert lib.hca_probe_lds_read(0, 0, 256, DUMMY, None) == ERR_SHAPE
    assert lib.hca_probe_lds_read(1, 100, 256, NULL, None) == ERR_NULL


def test_decode_noalloc_validation(lib):
    """The allocation-free decode entry point checks its arguments like
    hca_attend_decode, and refuses a batch whose partials would not fit its
    static scratch, all before any HIP call."""
    p = _p()
    args = [DUMMY] * 7
    assert lib.hca_attend_decode_noalloc(None, 4, 10, *args, 128, DUMMY, None) == ERR_NULL
    assert lib.hca_attend_decode_noalloc(ctypes.byref(p), -1, 10, *args, 128, DUMMY, None) == ERR_SHAPE
    assert lib.hca_attend_decode_noalloc(ctypes.byref(p), 4, 10, *args, 64, DUMMY, None) == ERR_SHAPE  # ring < W
    assert lib.hca_attend_decode_noalloc(ctypes.byref(p), 4, 10, *args, 128, NULL, None) == ERR_NULL
    assert lib.hca_attend_decode_noalloc(ctypes.byref(p), 0, 10, *args, 128, DUMMY, None) == OK
    assert lib.hca_decode_workspace_bytes(ctypes.byref(p), 1024, 1024) > hca.DECODE_NOALLOC_SCRATCH_BYTES
    assert lib.hca_attend_decode_noalloc(ctypes.byref(p), 1024, 1024, *args, 128, DUMMY, None) == ERR_WORKSPACE
