// Host side of the C ABI declared in include/hca.h: argument validation,
// dispatch by dtype, launch-error mapping.  No allocation, no
// synchronisation, no global mutable state.
#include <math.h>

#include <mutex>

#include "../../include/hca.h"
#include "hca_internal.h"

namespace {

constexpr int32_t kMaxHeadDim = 1024;

hca_status check_params(const hca_params* p) {
  if (!p) return HCA_ERR_NULL;
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 || p->window < 1)
    return HCA_ERR_SHAPE;
  if (p->num_q_heads % p->num_kv_heads) return HCA_ERR_SHAPE;
  if (p->num_kv_heads > 65535) return HCA_ERR_SHAPE;
  if (p->dtype != HCA_F32 && p->dtype != HCA_BF16) return HCA_ERR_UNSUPPORTED;
  if (p->block != hca::kBlock) return HCA_ERR_UNSUPPORTED;
  if (p->head_dim > kMaxHeadDim) return HCA_ERR_UNSUPPORTED;
  if (!(p->softmax_scale == p->softmax_scale)) return HCA_ERR_SHAPE;  // NaN
  return HCA_OK;
}

float scale_of(const hca_params* p) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.f / sqrtf((float)p->head_dim);
}

// The matrix-core path: 512-dim heads, 64 query heads per KV head.
bool mfma_shape(const hca_params* p) {
  return p->head_dim == 512 && p->num_q_heads / p->num_kv_heads == 64;
}

// The matrix-core kernels address a sequence's rows (raw, ring or cached
// entries) with 32-bit byte offsets from the sequence's first row.
bool mfma_rows_fit(const hca_params* p, long rows) {
  return rows * (long)p->num_kv_heads * p->head_dim * 2 < 0x7fffffffL;
}

hca_status from_hip(hipError_t e) { return e == hipSuccess ? HCA_OK : HCA_ERR_HIP; }

// Arguments of the fused attention epilogue (gate logits, mixing factors).
hca_status check_epilogue(const hca_params* p, const float* gate, const float* u, const float* v, int32_t rank) {
  if ((u == nullptr) != (v == nullptr)) return HCA_ERR_NULL;
  if (u && (rank < 1 || rank > 32)) return HCA_ERR_SHAPE;
  // fused into the matrix-core kernels (a whole KV group per workgroup)
  if ((gate || u) && p->dtype != HCA_BF16) return HCA_ERR_UNSUPPORTED;
  return HCA_OK;
}

int elem_bytes(const hca_params* p) { return p->dtype == HCA_BF16 ? 2 : 4; }

// Bytes of one staged plane (K or V) of a chunk call: every sequence's
// window - 1 halo rows plus its new rows, 256-byte aligned.
size_t staged_plane_bytes(const hca_params* p, int32_t batch, int32_t total_rows) {
  const size_t rows = (size_t)total_rows + (size_t)batch * (size_t)(p->window - 1);
  const size_t bytes = rows * (size_t)p->num_kv_heads * (size_t)p->head_dim * (size_t)elem_bytes(p);
  return (bytes + 255) / 256 * 256;
}

// Host checks and argument packing shared by the decode entry points
// (everything but the workspace).  The status is HCA_OK with nothing to do
// when batch == 0.
hca_status decode_args(const hca_params* params, int32_t batch, int32_t max_blocks, const int32_t* seqlens,
                       const int32_t* cu_blocks, const void* q, const void* kc, const void* vc, const void* kw,
                       const void* vw, int32_t ring_cap, const float* gate, const float* vha_u,
                       const float* vha_v, int32_t vha_rank, void* o, hca::DecodeArgs* a) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_blocks < 0 || batch > 65535) return HCA_ERR_SHAPE;
  if (ring_cap < params->window) return HCA_ERR_SHAPE;
  if (params->dtype == HCA_BF16 && !mfma_shape(params)) return HCA_ERR_UNSUPPORTED;
  if (params->dtype == HCA_BF16 && !(mfma_rows_fit(params, ring_cap) && mfma_rows_fit(params, max_blocks)))
    return HCA_ERR_SHAPE;
  st = check_epilogue(params, gate, vha_u, vha_v, vha_rank);
  if (st != HCA_OK) return st;
  if (batch == 0) return HCA_OK;
  if (!seqlens || !cu_blocks || !q || !kw || !vw || !o) return HCA_ERR_NULL;
  if (max_blocks > 0 && (!kc || !vc)) return HCA_ERR_NULL;
  a->batch = batch;
  a->max_blocks = max_blocks;
  a->hq = params->num_q_heads;
  a->hkv = params->num_kv_heads;
  a->d = params->head_dim;
  a->window = params->window;
  a->ring = ring_cap;
  a->scale = scale_of(params);
  a->seqlens = seqlens;
  a->cu_blocks = cu_blocks;
  a->q = q;
  a->kc = kc;
  a->vc = vc;
  a->kw = kw;
  a->vw = vw;
  a->o = o;
  a->ws = nullptr;
  a->gate = gate;
  a->mix_u = vha_u;
  a->mix_v = vha_v;
  a->mix_rank = vha_u ? vha_rank : 0;
  return HCA_OK;
}

// Scratch of hca_attend_decode_noalloc: the split partials of one decode call
// live in this file-scope device array instead of a caller workspace.  Each
// GPU holds its own copy (at its own address) until the process ends.  Host
// code never passes the array's name to a kernel (on the host it only stands
// for the symbol): it asks the runtime for the device address once per
// device, with that device current, and uses that pointer.
static __device__ __align__(256) unsigned char scratch[HCA_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (NULL on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] { slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch)); });
  return slot.err == hipSuccess ? slot.ptr : nullptr;
}

}  // namespace

extern "C" {

hca_status hca_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (!buf || !sink) return HCA_ERR_NULL;
  if (bytes == 0 || bytes % 16 || grid < 1 || grid > 65536) return HCA_ERR_SHAPE;
  return from_hip(hca::launch_probe_stream_read(buf, bytes, (unsigned*)sink, grid, (hipStream_t)stream));
}

hca_status hca_probe_stream_lds(const void* buf, size_t bytes, uint32_t* sink, int32_t grid, void* stream) {
  if (!buf || !sink) return HCA_ERR_NULL;
  if (hca::probe_stream_lds_bytes(bytes) == 0 || grid < 1 || grid > 65536) return HCA_ERR_SHAPE;
  return from_hip(hca::launch_probe_stream_lds(buf, bytes, (unsigned*)sink, grid, (hipStream_t)stream));
}

hca_status hca_probe_mfma_bf16(int32_t iters, int32_t grid, float* sink, void* stream) {
  if (!sink) return HCA_ERR_NULL;
  if (iters < 1 || grid < 1 || grid > 65536) return HCA_ERR_SHAPE;
  return from_hip(hca::launch_probe_mfma(iters, grid, sink, (hipStream_t)stream));
}

hca_status hca_probe_lds_read(int32_t mode, int32_t iters, int32_t grid, uint32_t* sink, void* stream) {
  if (!sink) return HCA_ERR_NULL;
  if ((mode != 0 && mode != 1) || iters < 1 || grid < 1 || grid > 65536) return HCA_ERR_SHAPE;
  return from_hip(hca::launch_probe_lds(mode, iters, grid, (unsigned*)sink, (hipStream_t)stream));
}

const char* hca_version(void) { return "0.1.0"; }

const char* hca_status_string(hca_status s) {
  switch (s) {
    case HCA_OK: return "HCA_OK";
    case HCA_ERR_NULL: return "HCA_ERR_NULL: a required pointer is NULL";
    case HCA_ERR_SHAPE: return "HCA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case HCA_ERR_UNSUPPORTED: return "HCA_ERR_UNSUPPORTED: shape or dtype not handled by this build";
    case HCA_ERR_WORKSPACE: return "HCA_ERR_WORKSPACE: decode workspace missing or too small";
    case HCA_ERR_HIP: return "HCA_ERR_HIP: the HIP runtime rejected a launch";
  }
  return "HCA_ERR_UNKNOWN";
}

hca_status hca_compress(const hca_params* params, int32_t batch, int32_t total_blocks,
                        const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* k,
                        const void* v, const float* w, void* kc, void* vc, void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || total_blocks < 0) return HCA_ERR_SHAPE;
  if (params->head_dim % 64) return HCA_ERR_UNSUPPORTED;
  if ((long)total_blocks * params->num_kv_heads > 0x7fffffffL) return HCA_ERR_SHAPE;
  if (total_blocks == 0) return HCA_OK;  // no output rows: any pointer may be NULL
  if ((v == nullptr) != (vc == nullptr)) return HCA_ERR_NULL;
  if (batch == 0) return HCA_ERR_SHAPE;  // entries without sequences
  if (!cu_seqlens || !cu_blocks || !k || !w || !kc) return HCA_ERR_NULL;
  hca::CompressArgs a{};
  a.batch = batch;
  a.total_blocks = total_blocks;
  a.hkv = params->num_kv_heads;
  a.d = params->head_dim;
  a.cu_seqlens = cu_seqlens;
  a.cu_blocks = cu_blocks;
  a.x[0] = k;
  a.x[1] = v;
  a.xc[0] = kc;
  a.xc[1] = vc;
  a.w = w;
  return from_hip(hca::launch_compress(params->dtype, a, (hipStream_t)stream));
}

hca_status hca_attend_prefill_gated_vha(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                        const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q,
                                        const void* k, const void* v, const void* kc, const void* vc,
                                        const float* gate, const float* vha_u, const float* vha_v,
                                        int32_t vha_rank, void* o, void* stream);

hca_status hca_attend_prefill(const hca_params* params, int32_t batch, int32_t max_seqlen,
                              const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q,
                              const void* k, const void* v, const void* kc, const void* vc,
                              void* o, void* stream) {
  return hca_attend_prefill_gated_vha(params, batch, max_seqlen, cu_seqlens, cu_blocks, q, k, v, kc, vc,
                                      nullptr, nullptr, nullptr, 0, o, stream);
}

static hca_status prefill_common(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                 const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q, const void* k,
                                 const void* v, const void* kc, const void* vc, const float* gate,
                                 const float* vha_u, const float* vha_v, int32_t vha_rank, void* o, float* lse,
                                 void* stream);

hca_status hca_attend_prefill_gated_vha(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                        const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q,
                                        const void* k, const void* v, const void* kc, const void* vc,
                                        const float* gate, const float* vha_u, const float* vha_v,
                                        int32_t vha_rank, void* o, void* stream) {
  return prefill_common(params, batch, max_seqlen, cu_seqlens, cu_blocks, q, k, v, kc, vc, gate, vha_u, vha_v,
                        vha_rank, o, nullptr, stream);
}

hca_status hca_attend_prefill_lse(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                  const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q, const void* k,
                                  const void* v, const void* kc, const void* vc, void* o, float* lse,
                                  void* stream) {
  const hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (params->dtype != HCA_BF16) return HCA_ERR_UNSUPPORTED;  // saved for the matrix-core backward
  if (batch > 0 && max_seqlen > 0 && !lse) return HCA_ERR_NULL;
  return prefill_common(params, batch, max_seqlen, cu_seqlens, cu_blocks, q, k, v, kc, vc, nullptr, nullptr, nullptr,
                        0, o, lse, stream);
}

static hca_status prefill_common(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                 const int32_t* cu_seqlens, const int32_t* cu_blocks, const void* q, const void* k,
                                 const void* v, const void* kc, const void* vc, const float* gate,
                                 const float* vha_u, const float* vha_v, int32_t vha_rank, void* o, float* lse,
                                 void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_seqlen < 0 || batch > 65535) return HCA_ERR_SHAPE;
  if (params->dtype == HCA_BF16 && !mfma_shape(params)) return HCA_ERR_UNSUPPORTED;
  if (params->dtype == HCA_F32 && (long)max_seqlen * params->num_q_heads > 0x7fffffffL)
    return HCA_ERR_SHAPE;
  if (params->dtype == HCA_BF16 && !mfma_rows_fit(params, max_seqlen)) return HCA_ERR_SHAPE;
  st = check_epilogue(params, gate, vha_u, vha_v, vha_rank);
  if (st != HCA_OK) return st;
  if (batch == 0 || max_seqlen == 0) return HCA_OK;
  if (!cu_seqlens || !cu_blocks || !q || !k || !v || !o) return HCA_ERR_NULL;
  if (max_seqlen >= hca::kBlock && (!kc || !vc)) return HCA_ERR_NULL;
  hca::PrefillArgs a{};  // whole sequences: pos0 NULL, halo 0
  a.batch = batch;
  a.max_seqlen = max_seqlen;
  a.hq = params->num_q_heads;
  a.hkv = params->num_kv_heads;
  a.d = params->head_dim;
  a.window = params->window;
  a.scale = scale_of(params);
  a.cu_seqlens = cu_seqlens;
  a.cu_blocks = cu_blocks;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = kc;
  a.vc = vc;
  a.o = o;
  a.gate = gate;
  a.mix_u = vha_u;
  a.mix_v = vha_v;
  a.mix_rank = vha_u ? vha_rank : 0;
  a.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  return from_hip(params->dtype == HCA_BF16 ? hca::launch_prefill_bf16(a, s)
                                            : hca::launch_prefill_f32(a, s));
}

size_t hca_attend_prefill_backward_workspace_bytes(const hca_params* params, int32_t batch, int32_t total_tokens,
                                                   int32_t total_blocks, int32_t max_seqlen) {
  if (check_params(params) != HCA_OK || batch < 0 || total_tokens < 0 || total_blocks < 0 || max_seqlen < 0) return 0;
  if (params->dtype != HCA_BF16 || !mfma_shape(params)) return 0;
  return hca::backward_workspace_bytes(batch, params->num_q_heads, params->num_kv_heads, total_tokens, total_blocks,
                                       max_seqlen, params->window);
}

hca_status hca_attend_prefill_backward(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                       int32_t total_tokens, int32_t total_blocks, const int32_t* cu_seqlens,
                                       const int32_t* cu_blocks, const void* q, const void* k, const void* v,
                                       const float* w, const void* kc, const void* vc, const void* o,
                                       const float* lse, const void* dout, void* dq, void* dk, void* dv, float* dw,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_seqlen < 0 || batch > 65535 || total_tokens < 0 || total_blocks < 0) return HCA_ERR_SHAPE;
  if (params->dtype != HCA_BF16 || !mfma_shape(params)) return HCA_ERR_UNSUPPORTED;
  if (!mfma_rows_fit(params, max_seqlen)) return HCA_ERR_SHAPE;
  if ((long)total_tokens < (long)max_seqlen || (long)total_blocks * hca::kBlock > (long)total_tokens)
    return HCA_ERR_SHAPE;
  if (!w || !dw) return HCA_ERR_NULL;  // dw [Hkv, 128] is written even without tokens
  const size_t need = hca::backward_workspace_bytes(batch, params->num_q_heads, params->num_kv_heads, total_tokens,
                                                    total_blocks, max_seqlen, params->window);
  if (!workspace || workspace_bytes < need) return HCA_ERR_WORKSPACE;
  const bool rows = batch > 0 && max_seqlen > 0;
  if (rows && (!cu_seqlens || !cu_blocks || !q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv))
    return HCA_ERR_NULL;
  if (rows && max_seqlen >= hca::kBlock && (!kc || !vc)) return HCA_ERR_NULL;
  hca::BackwardArgs a{};
  a.batch = rows ? batch : 0;
  a.max_seqlen = rows ? max_seqlen : 0;
  a.total_tokens = total_tokens;
  a.total_blocks = rows ? total_blocks : 0;
  a.hq = params->num_q_heads;
  a.hkv = params->num_kv_heads;
  a.d = params->head_dim;
  a.window = params->window;
  a.scale = scale_of(params);
  a.cu_seqlens = cu_seqlens;
  a.cu_blocks = cu_blocks;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kc = kc;
  a.vc = vc;
  a.o = o;
  a.dout = dout;
  a.w = w;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = dw;
  a.ws = workspace;
  return from_hip(hca::launch_backward_bf16(a, (hipStream_t)stream));
}

size_t hca_dsa_decode_workspace_bytes(int32_t batch, int32_t max_seqlen, int32_t topk) {
  if (batch < 0 || max_seqlen < 0 || topk < 1) return 0;
  return hca::dsa_workspace_bytes(batch, max_seqlen, topk);
}

hca_status hca_dsa_decode(int32_t batch, int32_t max_seqlen, int32_t topk, float softmax_scale,
                          const int32_t* seqlens, const int32_t* cu_rows, const void* q, const int8_t* qi,
                          const void* k, const void* v, const int8_t* ki, void* o, int32_t* sel, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (batch < 0 || batch > 65535 || max_seqlen < 0 || topk < 1) return HCA_ERR_SHAPE;
  if (!(softmax_scale == softmax_scale)) return HCA_ERR_SHAPE;  // NaN
  if ((long)batch * max_seqlen > 0x7fffffffL) return HCA_ERR_SHAPE;
  if (batch == 0 || max_seqlen == 0) return HCA_OK;
  if (!seqlens || !cu_rows || !q || !qi || !k || !v || !ki || !o || !sel) return HCA_ERR_NULL;
  const size_t need = hca::dsa_workspace_bytes(batch, max_seqlen, topk);
  if (!workspace || workspace_bytes < need) return HCA_ERR_WORKSPACE;
  hca::DsaArgs a{};
  a.batch = batch;
  a.max_seqlen = max_seqlen;
  a.topk = topk;
  a.scale = softmax_scale > 0.f ? softmax_scale : 1.f / 16.f;  // 1/sqrt(256)
  a.seqlens = seqlens;
  a.cu_rows = cu_rows;
  a.q = q;
  a.qi = (const signed char*)qi;
  a.k = k;
  a.v = v;
  a.ki = (const signed char*)ki;
  a.o = o;
  a.sel = sel;
  a.ws = workspace;
  return from_hip(hca::launch_dsa_decode(a, (hipStream_t)stream));
}

size_t hca_decode_workspace_bytes(const hca_params* params, int32_t batch, int32_t max_blocks) {
  if (check_params(params) != HCA_OK || batch < 0 || max_blocks < 0) return 0;
  if (params->dtype == HCA_F32) return 0;
  if (!mfma_shape(params)) return 0;
  return hca::decode_workspace_bytes_bf16(batch, params->num_kv_heads, max_blocks, params->window);
}

hca_status hca_attend_decode_gated_vha(const hca_params* params, int32_t batch, int32_t max_blocks,
                                       const int32_t* seqlens, const int32_t* cu_blocks, const void* q,
                                       const void* kc, const void* vc, const void* kw, const void* vw,
                                       int32_t ring_cap, const float* gate, const float* vha_u,
                                       const float* vha_v, int32_t vha_rank, void* o, void* workspace,
                                       size_t workspace_bytes, void* stream);

hca_status hca_attend_decode(const hca_params* params, int32_t batch, int32_t max_blocks,
                             const int32_t* seqlens, const int32_t* cu_blocks, const void* q,
                             const void* kc, const void* vc, const void* kw, const void* vw,
                             int32_t ring_cap, void* o, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return hca_attend_decode_gated_vha(params, batch, max_blocks, seqlens, cu_blocks, q, kc, vc, kw, vw, ring_cap,
                                     nullptr, nullptr, nullptr, 0, o, workspace, workspace_bytes, stream);
}

hca_status hca_attend_decode_gated_vha(const hca_params* params, int32_t batch, int32_t max_blocks,
                                       const int32_t* seqlens, const int32_t* cu_blocks, const void* q,
                                       const void* kc, const void* vc, const void* kw, const void* vw,
                                       int32_t ring_cap, const float* gate, const float* vha_u,
                                       const float* vha_v, int32_t vha_rank, void* o, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  hca::DecodeArgs a{};
  hca_status st = decode_args(params, batch, max_blocks, seqlens, cu_blocks, q, kc, vc, kw, vw, ring_cap, gate,
                              vha_u, vha_v, vha_rank, o, &a);
  if (st != HCA_OK || batch == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  if (params->dtype == HCA_F32) return from_hip(hca::launch_decode_f32(a, s));
  const size_t need =
      hca::decode_workspace_bytes_bf16(batch, params->num_kv_heads, max_blocks, params->window);
  if (!workspace || workspace_bytes < need) return HCA_ERR_WORKSPACE;
  if (((uintptr_t)workspace) & 255) return HCA_ERR_WORKSPACE;
  a.ws = workspace;
  return from_hip(hca::launch_decode_bf16(a, s));
}

hca_status hca_attend_decode_noalloc(const hca_params* params, int32_t batch, int32_t max_blocks,
                                     const int32_t* seqlens, const int32_t* cu_blocks, const void* q, const void* kc,
                                     const void* vc, const void* kw, const void* vw, int32_t ring_cap, void* o,
                                     void* stream) {
  hca::DecodeArgs a{};
  hca_status st = decode_args(params, batch, max_blocks, seqlens, cu_blocks, q, kc, vc, kw, vw, ring_cap, nullptr,
                              nullptr, nullptr, 0, o, &a);
  if (st != HCA_OK || batch == 0) return st;
  hipStream_t s = (hipStream_t)stream;
  if (params->dtype == HCA_F32) return from_hip(hca::launch_decode_f32(a, s));  // no scratch
  const size_t need =
      hca::decode_workspace_bytes_bf16(batch, params->num_kv_heads, max_blocks, params->window);
  if (need > HCA_DECODE_NOALLOC_SCRATCH_BYTES) return HCA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return HCA_ERR_HIP;
  // the split kernel writes every partial the merge kernel reads: nothing
  // in the scratch has to start at zero
  a.ws = ws;
  return from_hip(hca::launch_decode_bf16(a, s));
}

hca_status hca_compress_chunk(const hca_params* params, int32_t batch, int32_t max_rows,
                              const int32_t* cu_seqlens, const int32_t* pos0, const int32_t* cu_blocks,
                              const void* k, const void* v, const float* w, const void* kw,
                              const void* vw, int32_t ring_cap, void* kc, void* vc, void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_rows < 0 || batch > 65535) return HCA_ERR_SHAPE;
  if (params->head_dim % 64) return HCA_ERR_UNSUPPORTED;
  if (ring_cap < hca::kBlock) return HCA_ERR_SHAPE;  // a straddling block's older rows
  const long max_new = ((long)max_rows + hca::kBlock - 1) / hca::kBlock;
  if ((long)batch * max_new * params->num_kv_heads > 0x7fffffffL) return HCA_ERR_SHAPE;
  if (batch == 0 || max_rows == 0) return HCA_OK;
  if ((v == nullptr) != (vc == nullptr) || (v == nullptr) != (vw == nullptr)) return HCA_ERR_NULL;
  if (!cu_seqlens || !pos0 || !cu_blocks || !k || !w || !kw || !kc) return HCA_ERR_NULL;
  hca::CompressArgs a{};
  a.batch = batch;
  a.total_blocks = (int)(batch * max_new);
  a.hkv = params->num_kv_heads;
  a.d = params->head_dim;
  a.cu_seqlens = cu_seqlens;
  a.cu_blocks = cu_blocks;
  a.x[0] = k;
  a.x[1] = v;
  a.xc[0] = kc;
  a.xc[1] = vc;
  a.w = w;
  a.pos0 = pos0;
  a.ring[0] = kw;
  a.ring[1] = vw;
  a.ring_cap = ring_cap;
  a.max_new = (int)max_new;
  return from_hip(hca::launch_compress_chunk(params->dtype, a, (hipStream_t)stream));
}

hca_status hca_ring_append(const hca_params* params, int32_t batch, int32_t max_rows,
                           const int32_t* cu_seqlens, const int32_t* pos0, const void* k, const void* v,
                           void* kw, void* vw, int32_t ring_cap, void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_rows < 0 || batch > 65535 || ring_cap < 1) return HCA_ERR_SHAPE;
  if (params->head_dim % 64) return HCA_ERR_UNSUPPORTED;
  if (batch == 0 || max_rows == 0) return HCA_OK;
  if ((v == nullptr) != (vw == nullptr)) return HCA_ERR_NULL;
  if (!cu_seqlens || !pos0 || !k || !kw) return HCA_ERR_NULL;
  hca::ChunkRowsArgs a{};
  a.batch = batch;
  a.max_rows = max_rows;
  a.row_elems = params->num_kv_heads * params->head_dim;
  a.elem_bytes = elem_bytes(params);
  a.ring_cap = ring_cap;
  a.cu_seqlens = cu_seqlens;
  a.pos0 = pos0;
  a.x[0] = k;
  a.x[1] = v;
  a.ring[0] = kw;
  a.ring[1] = vw;
  return from_hip(hca::launch_ring_append(a, (hipStream_t)stream));
}

size_t hca_prefill_chunk_workspace_bytes(const hca_params* params, int32_t batch, int32_t total_rows) {
  if (check_params(params) != HCA_OK || batch < 0 || total_rows < 0) return 0;
  return 2 * staged_plane_bytes(params, batch, total_rows);
}

hca_status hca_attend_prefill_chunk_gated_vha(
    const hca_params* params, int32_t batch, int32_t max_seqlen, int32_t total_rows, const int32_t* cu_seqlens,
    const int32_t* pos0, const int32_t* cu_blocks, const void* q, const void* k, const void* v, const void* kc,
    const void* vc, const void* kw, const void* vw, int32_t ring_cap, const float* gate, const float* vha_u,
    const float* vha_v, int32_t vha_rank, void* o, void* workspace, size_t workspace_bytes, void* stream);

hca_status hca_attend_prefill_chunk(const hca_params* params, int32_t batch, int32_t max_seqlen,
                                    int32_t total_rows, const int32_t* cu_seqlens, const int32_t* pos0,
                                    const int32_t* cu_blocks, const void* q, const void* k, const void* v,
                                    const void* kc, const void* vc, const void* kw, const void* vw,
                                    int32_t ring_cap, void* o, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return hca_attend_prefill_chunk_gated_vha(params, batch, max_seqlen, total_rows, cu_seqlens, pos0, cu_blocks, q,
                                            k, v, kc, vc, kw, vw, ring_cap, nullptr, nullptr, nullptr, 0, o,
                                            workspace, workspace_bytes, stream);
}

hca_status hca_attend_prefill_chunk_gated_vha(
    const hca_params* params, int32_t batch, int32_t max_seqlen, int32_t total_rows, const int32_t* cu_seqlens,
    const int32_t* pos0, const int32_t* cu_blocks, const void* q, const void* k, const void* v, const void* kc,
    const void* vc, const void* kw, const void* vw, int32_t ring_cap, const float* gate, const float* vha_u,
    const float* vha_v, int32_t vha_rank, void* o, void* workspace, size_t workspace_bytes, void* stream) {
  hca_status st = check_params(params);
  if (st != HCA_OK) return st;
  if (batch < 0 || max_seqlen < 0 || total_rows < 0 || batch > 65535) return HCA_ERR_SHAPE;
  if (ring_cap < params->window) return HCA_ERR_SHAPE;
  if (params->head_dim % 64) return HCA_ERR_UNSUPPORTED;
  if (params->dtype == HCA_BF16 && !mfma_shape(params)) return HCA_ERR_UNSUPPORTED;
  if (params->dtype == HCA_F32 && (long)max_seqlen * params->num_q_heads > 0x7fffffffL)
    return HCA_ERR_SHAPE;
  const long halo = params->window - 1;
  if (params->dtype == HCA_BF16 && !mfma_rows_fit(params, (long)max_seqlen + halo)) return HCA_ERR_SHAPE;
  st = check_epilogue(params, gate, vha_u, vha_v, vha_rank);
  if (st != HCA_OK) return st;
  if (((long)total_rows + (long)batch * halo) * params->num_kv_heads * params->head_dim * elem_bytes(params) >
      0xffffffffL)
    return HCA_ERR_SHAPE;  // staged rows are addressed with 32-bit buffer offsets
  if (batch == 0 || max_seqlen == 0 || total_rows == 0) return HCA_OK;
  if (!cu_seqlens || !pos0 || !cu_blocks || !q || !k || !v || !kc || !vc || !kw || !vw || !o)
    return HCA_ERR_NULL;
  const size_t plane = staged_plane_bytes(params, batch, total_rows);
  if (!workspace || workspace_bytes < 2 * plane || (((uintptr_t)workspace) & 255)) return HCA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  hca::ChunkRowsArgs c{};
  c.batch = batch;
  c.max_rows = max_seqlen;
  c.row_elems = params->num_kv_heads * params->head_dim;
  c.elem_bytes = elem_bytes(params);
  c.ring_cap = ring_cap;
  c.halo = (int)halo;
  c.cu_seqlens = cu_seqlens;
  c.pos0 = pos0;
  c.x[0] = k;
  c.x[1] = v;
  c.ring[0] = const_cast<void*>(kw);  // only read by the staging copy
  c.ring[1] = const_cast<void*>(vw);
  c.stage[0] = workspace;
  c.stage[1] = (char*)workspace + plane;
  hipError_t e = hca::launch_stage_chunk(c, s);
  if (e != hipSuccess) return from_hip(e);
  hca::PrefillArgs a{};
  a.batch = batch;
  a.max_seqlen = max_seqlen;
  a.hq = params->num_q_heads;
  a.hkv = params->num_kv_heads;
  a.d = params->head_dim;
  a.window = params->window;
  a.scale = scale_of(params);
  a.cu_seqlens = cu_seqlens;
  a.cu_blocks = cu_blocks;
  a.q = q;
  a.k = c.stage[0];
  a.v = c.stage[1];
  a.kc = kc;
  a.vc = vc;
  a.o = o;
  a.pos0 = pos0;
  a.halo = (int)halo;
  a.gate = gate;
  a.mix_u = vha_u;
  a.mix_v = vha_v;
  a.mix_rank = vha_u ? vha_rank : 0;
  return from_hip(params->dtype == HCA_BF16 ? hca::launch_prefill_bf16(a, s)
                                            : hca::launch_prefill_f32(a, s));
}

}  // extern "C"
