"""ctypes binding of libhca (include/hca.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors must be
contiguous torch tensors on the current HIP device; outputs that are not
passed in are allocated with torch (device memory plumbing) before the call.
All work happens in the library's HIP kernels on torch's current stream.  If
libhca.so has not been built the first call raises HcaLibraryMissing: there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhca.so")

HCA_F32, HCA_BF16 = 0, 1
_DTYPES = {torch.float32: HCA_F32, torch.bfloat16: HCA_BF16}
EXPORTS = ("hca_compress", "hca_attend_prefill", "hca_decode_workspace_bytes",
           "hca_attend_decode", "hca_compress_chunk", "hca_ring_append",
           "hca_prefill_chunk_workspace_bytes", "hca_attend_prefill_chunk", "hca_attend_prefill_gated_vha",
           "hca_attend_decode_gated_vha", "hca_attend_prefill_chunk_gated_vha",
           "hca_attend_prefill_lse", "hca_attend_prefill_backward_workspace_bytes", "hca_attend_prefill_backward",
           "hca_dsa_decode_workspace_bytes", "hca_dsa_decode",
           "hca_probe_stream_read", "hca_probe_stream_lds", "hca_probe_mfma_bf16", "hca_probe_lds_read", "hca_attend_decode_noalloc",
           "hca_status_string", "hca_version")


class HcaLibraryMissing(ImportError):
    pass


class HcaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {hca_status_string(status)} ({status})")


class HcaParams(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
    ]


def make_params(num_q_heads, num_kv_heads, head_dim, window, dtype, block=128,
                softmax_scale=0.0) -> HcaParams:
    """dtype: torch.float32 / torch.bfloat16 or the hca_dtype code."""
    code = _DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return HcaParams(int(num_q_heads), int(num_kv_heads), int(head_dim), int(block),
                     int(window), float(softmax_scale), code)


_lib = None


def library() -> ctypes.CDLL:
    """Load libhca.so once; raises HcaLibraryMissing if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise HcaLibraryMissing(
            f"{LIB_PATH} is missing: build it with `python -m compressed_kv_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(HcaParams)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.hca_compress.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hca_compress.restype = ctypes.c_int
    lib.hca_attend_prefill.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hca_attend_prefill.restype = ctypes.c_int
    lib.hca_attend_prefill_gated_vha.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32,
                                                 vp, vp]
    lib.hca_attend_prefill_gated_vha.restype = ctypes.c_int
    lib.hca_attend_decode_gated_vha.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32,
                                                vp, vp, sz, vp]
    lib.hca_attend_decode_gated_vha.restype = ctypes.c_int
    lib.hca_attend_prefill_chunk_gated_vha.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                       i32, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.hca_attend_prefill_chunk_gated_vha.restype = ctypes.c_int
    lib.hca_decode_workspace_bytes.argtypes = [P, i32, i32]
    lib.hca_decode_workspace_bytes.restype = sz
    lib.hca_attend_decode.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, sz, vp]
    lib.hca_attend_decode.restype = ctypes.c_int
    lib.hca_compress_chunk.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.hca_compress_chunk.restype = ctypes.c_int
    lib.hca_ring_append.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.hca_ring_append.restype = ctypes.c_int
    lib.hca_prefill_chunk_workspace_bytes.argtypes = [P, i32, i32]
    lib.hca_prefill_chunk_workspace_bytes.restype = sz
    lib.hca_attend_prefill_chunk.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                             i32, vp, vp, sz, vp]
    lib.hca_attend_prefill_chunk.restype = ctypes.c_int
    lib.hca_attend_prefill_lse.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.hca_attend_prefill_lse.restype = ctypes.c_int
    lib.hca_attend_prefill_backward_workspace_bytes.argtypes = [P, i32, i32, i32, i32]
    lib.hca_attend_prefill_backward_workspace_bytes.restype = sz
    lib.hca_attend_prefill_backward.argtypes = [P, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hca_attend_prefill_backward.restype = ctypes.c_int
    lib.hca_dsa_decode_workspace_bytes.argtypes = [i32, i32, i32]
    lib.hca_dsa_decode_workspace_bytes.restype = sz
    lib.hca_dsa_decode.argtypes = [i32, i32, i32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.hca_dsa_decode.restype = ctypes.c_int
    lib.hca_attend_decode_noalloc.argtypes = [P, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.hca_attend_decode_noalloc.restype = ctypes.c_int
    lib.hca_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.hca_probe_stream_read.restype = ctypes.c_int
    lib.hca_probe_stream_lds.argtypes = [vp, sz, vp, i32, vp]
    lib.hca_probe_stream_lds.restype = ctypes.c_int
    lib.hca_probe_mfma_bf16.argtypes = [i32, i32, vp, vp]
    lib.hca_probe_mfma_bf16.restype = ctypes.c_int
    lib.hca_probe_lds_read.argtypes = [i32, i32, i32, vp, vp]
    lib.hca_probe_lds_read.restype = ctypes.c_int
    lib.hca_status_string.argtypes = [ctypes.c_int]
    lib.hca_status_string.restype = ctypes.c_char_p
    lib.hca_version.argtypes = []
    lib.hca_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def hca_status_string(status: int) -> str:
    return library().hca_status_string(int(status)).decode()


def hca_version() -> str:
    return library().hca_version().decode()


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise HcaError(fn, status)


def hca_compress(params: HcaParams, cu_seqlens, cu_blocks, total_blocks: int, k, w, v=None,
                 kc=None, vc=None, stream=None):
    """Pool complete 128-token blocks of k (and v).  Returns (kc, vc)."""
    batch = cu_seqlens.numel() - 1
    shape = (int(total_blocks), k.shape[1], k.shape[2])
    if kc is None:
        kc = torch.empty(shape, dtype=k.dtype, device=k.device)
    if v is not None and vc is None:
        vc = torch.empty(shape, dtype=v.dtype, device=v.device)
    st = library().hca_compress(ctypes.byref(params), batch, int(total_blocks), _ptr(cu_seqlens),
                                _ptr(cu_blocks), _ptr(k), _ptr(v), _ptr(w), _ptr(kc), _ptr(vc),
                                _stream(stream))
    _check("hca_compress", st)
    return kc, vc


def hca_attend_prefill(params: HcaParams, cu_seqlens, cu_blocks, max_seqlen: int, q, k, v, kc, vc,
                       o=None, stream=None):
    """Causal HCA attention for a packed batch.  Returns o [N_tok, Hq, d]."""
    batch = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    st = library().hca_attend_prefill(ctypes.byref(params), batch, int(max_seqlen), _ptr(cu_seqlens),
                                      _ptr(cu_blocks), _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                      _ptr(o), _stream(stream))
    _check("hca_attend_prefill", st)
    return o


def hca_attend_prefill_gated_vha(params: HcaParams, cu_seqlens, cu_blocks, max_seqlen: int, q, k, v, kc, vc,
                                 gate=None, vha_u=None, vha_v=None, o=None, stream=None):
    """hca_attend_prefill with the fused output gate (logits [N_tok, Hq]) and
    Virtual Head Attention mixing (U, V [Hkv, G, rank]).  Returns o."""
    batch = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    rank = 0 if vha_u is None else int(vha_u.shape[-1])
    st = library().hca_attend_prefill_gated_vha(ctypes.byref(params), batch, int(max_seqlen), _ptr(cu_seqlens),
                                                _ptr(cu_blocks), _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                                _ptr(gate), _ptr(vha_u), _ptr(vha_v), rank, _ptr(o),
                                                _stream(stream))
    _check("hca_attend_prefill_gated_vha", st)
    return o


def hca_attend_prefill_lse(params: HcaParams, cu_seqlens, cu_blocks, max_seqlen: int, q, k, v, kc, vc,
                           o=None, lse=None, stream=None):
    """hca_attend_prefill that also saves the per-row log-sum-exp of the
    scaled scores (fp32 [N_tok, Hq], natural log).  Returns (o, lse)."""
    batch = cu_seqlens.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    st = library().hca_attend_prefill_lse(ctypes.byref(params), batch, int(max_seqlen), _ptr(cu_seqlens),
                                          _ptr(cu_blocks), _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc),
                                          _ptr(o), _ptr(lse), _stream(stream))
    _check("hca_attend_prefill_lse", st)
    return o, lse


def hca_attend_prefill_backward_workspace_bytes(params: HcaParams, batch: int, total_tokens: int,
                                                total_blocks: int, max_seqlen: int) -> int:
    return int(library().hca_attend_prefill_backward_workspace_bytes(
        ctypes.byref(params), int(batch), int(total_tokens), int(total_blocks), int(max_seqlen)))


def new_backward_workspace(params: HcaParams, batch: int, total_tokens: int, total_blocks: int, max_seqlen: int,
                           device=None):
    """Workspace of the size hca_attend_prefill_backward needs."""
    n = hca_attend_prefill_backward_workspace_bytes(params, batch, total_tokens, total_blocks, max_seqlen)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device or torch.cuda.current_device())


def hca_attend_prefill_backward(params: HcaParams, cu_seqlens, cu_blocks, max_seqlen: int, total_blocks: int,
                                q, k, v, w, kc, vc, o, lse, dout, workspace=None, dq=None, dk=None, dv=None,
                                dw=None, stream=None):
    """Gradients (dq, dk, dv, dw) of a loss through pooling + prefill
    attention, given dout = dL/dO.  Returns (dq, dk, dv, dw)."""
    batch = cu_seqlens.numel() - 1
    ntok = q.shape[0]
    if workspace is None:
        workspace = new_backward_workspace(params, batch, ntok, total_blocks, max_seqlen, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dw = torch.empty(w.shape, dtype=torch.float32, device=q.device) if dw is None else dw
    ws_bytes = workspace.numel() * workspace.element_size()
    st = library().hca_attend_prefill_backward(
        ctypes.byref(params), batch, int(max_seqlen), int(ntok), int(total_blocks), _ptr(cu_seqlens),
        _ptr(cu_blocks), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(kc), _ptr(vc), _ptr(o), _ptr(lse), _ptr(dout),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(workspace), ws_bytes, _stream(stream))
    _check("hca_attend_prefill_backward", st)
    return dq, dk, dv, dw


def hca_dsa_decode_workspace_bytes(batch: int, max_seqlen: int, topk: int) -> int:
    return int(library().hca_dsa_decode_workspace_bytes(int(batch), int(max_seqlen), int(topk)))


def hca_dsa_decode(seqlens, cu_rows, max_seqlen: int, topk: int, q, qi, k, v, ki, workspace=None, o=None,
                   sel=None, softmax_scale: float = 0.0, stream=None):
    """Sparse-attention decode of the full-context layers: indexer scores,
    top-k selection and attention over the selection.  q bf16 [B, 64, 256],
    qi int8 [B, 128], k, v bf16 [rows, 256], ki int8 [rows, 128].
    Returns (o [B, 64, 256], sel int32 [B, topk])."""
    batch = seqlens.numel()
    if workspace is None:
        n = hca_dsa_decode_workspace_bytes(batch, max_seqlen, topk)
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q) if o is None else o
    sel = torch.empty((batch, int(topk)), dtype=torch.int32, device=q.device) if sel is None else sel
    st = library().hca_dsa_decode(int(batch), int(max_seqlen), int(topk), float(softmax_scale), _ptr(seqlens),
                                  _ptr(cu_rows), _ptr(q), _ptr(qi), _ptr(k), _ptr(v), _ptr(ki), _ptr(o), _ptr(sel),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("hca_dsa_decode", st)
    return o, sel


def hca_decode_workspace_bytes(params: HcaParams, batch: int, max_blocks: int) -> int:
    return int(library().hca_decode_workspace_bytes(ctypes.byref(params), int(batch), int(max_blocks)))


def new_decode_workspace(params: HcaParams, batch: int, max_blocks: int, device=None):
    """Workspace of the size hca_attend_decode needs (or None if it needs none)."""
    n = hca_decode_workspace_bytes(params, batch, max_blocks)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device or torch.cuda.current_device())


def hca_attend_decode(params: HcaParams, seqlens, cu_blocks, max_blocks: int, q, kc, vc, kw, vw,
                      workspace=None, o=None, stream=None):
    """One query per sequence against its cache.  Returns o [B, Hq, d]."""
    batch = seqlens.numel()
    if o is None:
        o = torch.empty_like(q)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = library().hca_attend_decode(ctypes.byref(params), batch, int(max_blocks), _ptr(seqlens),
                                     _ptr(cu_blocks), _ptr(q), _ptr(kc), _ptr(vc), _ptr(kw), _ptr(vw),
                                     int(kw.shape[1]), _ptr(o), _ptr(workspace), ws_bytes,
                                     _stream(stream))
    _check("hca_attend_decode", st)
    return o


def hca_attend_decode_gated_vha(params: HcaParams, seqlens, cu_blocks, max_blocks: int, q, kc, vc, kw, vw,
                                gate=None, vha_u=None, vha_v=None, workspace=None, o=None, stream=None):
    """hca_attend_decode with the fused gate (logits [B, Hq]) and head mixing."""
    batch = seqlens.numel()
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = new_decode_workspace(params, batch, max_blocks, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rank = 0 if vha_u is None else int(vha_u.shape[-1])
    st = library().hca_attend_decode_gated_vha(ctypes.byref(params), batch, int(max_blocks), _ptr(seqlens),
                                               _ptr(cu_blocks), _ptr(q), _ptr(kc), _ptr(vc), _ptr(kw), _ptr(vw),
                                               int(kw.shape[1]), _ptr(gate), _ptr(vha_u), _ptr(vha_v), rank,
                                               _ptr(o), _ptr(workspace), ws_bytes, _stream(stream))
    _check("hca_attend_decode_gated_vha", st)
    return o


# ---------------------------------------------------------------------------
# Serving with a cache: new rows at positions pos0[b] .. pos0[b] + n_b - 1.
# ---------------------------------------------------------------------------
def hca_compress_chunk(params: HcaParams, cu_seqlens, pos0, cu_blocks, max_rows: int, k, w, kw, kc,
                       v=None, vw=None, vc=None, stream=None):
    """Pool the blocks the new rows complete into kc (vc), in place."""
    batch = pos0.numel()
    st = library().hca_compress_chunk(ctypes.byref(params), batch, int(max_rows), _ptr(cu_seqlens),
                                      _ptr(pos0), _ptr(cu_blocks), _ptr(k), _ptr(v), _ptr(w), _ptr(kw),
                                      _ptr(vw), int(kw.shape[1]), _ptr(kc), _ptr(vc), _stream(stream))
    _check("hca_compress_chunk", st)
    return kc, vc


def hca_ring_append(params: HcaParams, cu_seqlens, pos0, max_rows: int, k, kw, v=None, vw=None,
                    stream=None):
    """Write the newest rows into the rings kw (vw), in place."""
    batch = pos0.numel()
    st = library().hca_ring_append(ctypes.byref(params), batch, int(max_rows), _ptr(cu_seqlens),
                                   _ptr(pos0), _ptr(k), _ptr(v), _ptr(kw), _ptr(vw), int(kw.shape[1]),
                                   _stream(stream))
    _check("hca_ring_append", st)
    return kw, vw


def hca_prefill_chunk_workspace_bytes(params: HcaParams, batch: int, total_rows: int) -> int:
    return int(library().hca_prefill_chunk_workspace_bytes(ctypes.byref(params), int(batch),
                                                           int(total_rows)))


def new_prefill_chunk_workspace(params: HcaParams, batch: int, total_rows: int, device=None):
    n = hca_prefill_chunk_workspace_bytes(params, batch, total_rows)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device or torch.cuda.current_device())


def hca_attend_prefill_chunk(params: HcaParams, cu_seqlens, pos0, cu_blocks, max_seqlen: int, q, k, v,
                             kc, vc, kw, vw, workspace=None, o=None, stream=None):
    """Attention of the new rows over the cache.  Returns o [N, Hq, d]."""
    batch = pos0.numel()
    total = q.shape[0]
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = new_prefill_chunk_workspace(params, batch, total, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = library().hca_attend_prefill_chunk(ctypes.byref(params), batch, int(max_seqlen), int(total),
                                            _ptr(cu_seqlens), _ptr(pos0), _ptr(cu_blocks), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(kc), _ptr(vc), _ptr(kw), _ptr(vw),
                                            int(kw.shape[1]), _ptr(o), _ptr(workspace), ws_bytes,
                                            _stream(stream))
    _check("hca_attend_prefill_chunk", st)
    return o


def hca_attend_prefill_chunk_gated_vha(params: HcaParams, cu_seqlens, pos0, cu_blocks, max_seqlen: int, q, k, v,
                                       kc, vc, kw, vw, gate=None, vha_u=None, vha_v=None, workspace=None, o=None,
                                       stream=None):
    """hca_attend_prefill_chunk with the fused gate (logits [N, Hq]) and head mixing."""
    batch = pos0.numel()
    total = q.shape[0]
    if o is None:
        o = torch.empty_like(q)
    if workspace is None:
        workspace = new_prefill_chunk_workspace(params, batch, total, q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    rank = 0 if vha_u is None else int(vha_u.shape[-1])
    st = library().hca_attend_prefill_chunk_gated_vha(
        ctypes.byref(params), batch, int(max_seqlen), int(total), _ptr(cu_seqlens), _ptr(pos0), _ptr(cu_blocks),
        _ptr(q), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), _ptr(kw), _ptr(vw), int(kw.shape[1]), _ptr(gate),
        _ptr(vha_u), _ptr(vha_v), rank, _ptr(o), _ptr(workspace), ws_bytes, _stream(stream))
    _check("hca_attend_prefill_chunk_gated_vha", st)
    return o


DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20  # HCA_DECODE_NOALLOC_SCRATCH_BYTES


def hca_attend_decode_noalloc(params: HcaParams, seqlens, cu_blocks, max_blocks: int, q, kc, vc, kw, vw, o,
                              stream=None):
    """hca_attend_decode without a workspace: the library's static per-device
    scratch holds the split partials (calls overlapping on one GPU race).
    `o` must be given: this path allocates nothing.  Returns o."""
    batch = seqlens.numel()
    st = library().hca_attend_decode_noalloc(ctypes.byref(params), batch, int(max_blocks), _ptr(seqlens),
                                             _ptr(cu_blocks), _ptr(q), _ptr(kc), _ptr(vc), _ptr(kw), _ptr(vw),
                                             int(kw.shape[1]), _ptr(o), _stream(stream))
    _check("hca_attend_decode_noalloc", st)
    return o


# ---------------------------------------------------------------------------
# Measurement probes (not the layer): ceilings the benchmark reads the hot
# path against.  Each returns the sink tensor it wrote.
# ---------------------------------------------------------------------------
def hca_probe_stream_read(buf, grid: int, sink=None, stream=None):
    """Read every byte of `buf` (contiguous, byte size a multiple of 16) once."""
    if sink is None:
        sink = torch.empty(4 * grid, dtype=torch.int32, device=buf.device)
    st = library().hca_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(grid),
                                         _stream(stream))
    _check("hca_probe_stream_read", st)
    return sink


PROBE_LDS_TILE = 49152  # bytes per tile of hca_probe_stream_lds


def hca_probe_stream_lds(buf, grid: int, sink=None, stream=None):
    """Read the whole 48 KiB tiles of `buf` once through LDS (direct
    buffer->LDS loads); returns the sink."""
    if sink is None:
        sink = torch.empty(4 * grid, dtype=torch.int32, device=buf.device)
    st = library().hca_probe_stream_lds(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), int(grid),
                                        _stream(stream))
    _check("hca_probe_stream_lds", st)
    return sink


def hca_probe_mfma_bf16(iters: int, grid: int, sink=None, device=None, stream=None):
    """grid x 4 wavefronts, each iters x 4 bf16 32x32x16 matrix-core products;
    sink[0] / sink[1] = shader-clock cycles / 100 MHz ticks of one loop."""
    if sink is None:
        sink = torch.empty(4 + 4 * grid, dtype=torch.float32, device=device or torch.cuda.current_device())
    st = library().hca_probe_mfma_bf16(int(iters), int(grid), _ptr(sink), _stream(stream))
    _check("hca_probe_mfma_bf16", st)
    return sink


def hca_probe_lds_read(mode: int, iters: int, grid: int, sink=None, device=None, stream=None):
    """LDS reads, mode 0: 16-byte rows (1 KiB per instruction); mode 1:
    transposed 8-byte V^T fragment reads (512 bytes per instruction)."""
    if sink is None:
        sink = torch.empty(4 * grid, dtype=torch.int32, device=device or torch.cuda.current_device())
    st = library().hca_probe_lds_read(int(mode), int(iters), int(grid), _ptr(sink), _stream(stream))
    _check("hca_probe_lds_read", st)
    return sink
