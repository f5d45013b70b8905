// fp32 HCA attention (prefill and decode) on the vector ALUs.
//
// Each query attends to the complete compressed entries of its sequence and
// to the raw window of the most recent tokens, under one softmax (release
// blog "ERNIE 5.5 Flash Base", section 2.1, HCA paragraph; Zhidx article,
// section "1. Latent-Gated Sparse Attention").  This is the full-precision
// instance for small head dims and any head grouping: one wavefront per
// (query, query head), lanes split the head dimension, the running softmax
// (max, sum, weighted values) is kept in fp32 with exact exp, so results stay
// within a few ulp of the float64 definition.  It is not a throughput path.
#include "hca_internal.h"

namespace hca {
namespace {

constexpr int kMaxPerLane = 16;  // head_dim <= 64 * 16 = 1024

__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

struct Running {
  float m = -INFINITY, l = 0.f;
  float acc[kMaxPerLane];
};

// Fold one key/value row into the running softmax of one query row.
__device__ __forceinline__ void fold(Running& r, const float* qv, const float* krow,
                                     const float* vrow, int d, int lane, float scale) {
  float part = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < d) part = fmaf(qv[i], krow[c], part);
  }
  const float s = wave_sum(part) * scale;
  const float mn = fmaxf(r.m, s);
  const float alpha = expf(r.m - mn);  // 0 on the first key (m = -inf)
  const float p = expf(s - mn);
  r.l = r.l * alpha + p;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < d) r.acc[i] = fmaf(p, vrow[c], r.acc[i] * alpha);
  }
  r.m = mn;
}

__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  const int lane = threadIdx.x;
  const int qh = blockIdx.x % a.hq;
  const int i = blockIdx.x / a.hq;          // query row within the sequence (chunk)
  const int b = blockIdx.y;
  const int start = a.cu_seqlens[b];
  if (i >= a.cu_seqlens[b + 1] - start) return;
  const int p0 = a.pos0 ? a.pos0[b] : 0;
  const int t = p0 + i;                     // its position
  const int g = a.hq / a.hkv, kvh = qh / g;
  const size_t rs = (size_t)a.hkv * a.d;   // elements between raw/compressed rows
  const float* q = (const float*)a.q + ((size_t)(start + i) * a.hq + qh) * a.d;
  // raw row of position s: start + b * halo + s - (p0 - halo)
  const long raw0 = (long)start + (long)b * a.halo - (p0 - a.halo);
  const float* k = (const float*)a.k + (size_t)kvh * a.d;
  const float* v = (const float*)a.v + (size_t)kvh * a.d;
  const float* kc = (const float*)a.kc + (size_t)a.cu_blocks[b] * rs + (size_t)kvh * a.d;
  const float* vc = (const float*)a.vc + (size_t)a.cu_blocks[b] * rs + (size_t)kvh * a.d;

  float qv[kMaxPerLane];
  Running r;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    qv[i] = c < a.d ? q[c] : 0.f;
    r.acc[i] = 0.f;
  }
  // complete blocks: 128(j+1) <= t+1
  const int n = (t + 1) / kBlock;
  for (int j = 0; j < n; ++j) fold(r, qv, kc + (size_t)j * rs, vc + (size_t)j * rs, a.d, lane, a.scale);
  // raw window max(0, t-W+1) .. t
  for (int s = max(0, t - a.window + 1); s <= t; ++s)
    fold(r, qv, k + (size_t)(raw0 + s) * rs, v + (size_t)(raw0 + s) * rs, a.d, lane, a.scale);

  float* o = (float*)a.o + ((size_t)(start + i) * a.hq + qh) * a.d;
  const float inv = 1.f / r.l;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < a.d) o[c] = r.acc[i] * inv;
  }
}

__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
  const int lane = threadIdx.x;
  const int qh = blockIdx.x;
  const int b = blockIdx.y;
  const int L = a.seqlens[b];
  const int t = L - 1;                      // the new token's position
  const int g = a.hq / a.hkv, kvh = qh / g;
  const size_t rs = (size_t)a.hkv * a.d;
  const float* q = (const float*)a.q + ((size_t)b * a.hq + qh) * a.d;
  const float* kc = (const float*)a.kc + (size_t)a.cu_blocks[b] * rs + (size_t)kvh * a.d;
  const float* vc = (const float*)a.vc + (size_t)a.cu_blocks[b] * rs + (size_t)kvh * a.d;
  const float* kw = (const float*)a.kw + (size_t)b * a.ring * rs + (size_t)kvh * a.d;
  const float* vw = (const float*)a.vw + (size_t)b * a.ring * rs + (size_t)kvh * a.d;

  float qv[kMaxPerLane];
  Running r;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    qv[i] = c < a.d ? q[c] : 0.f;
    r.acc[i] = 0.f;
  }
  const int n = (t + 1) / kBlock;
  for (int j = 0; j < n; ++j) fold(r, qv, kc + (size_t)j * rs, vc + (size_t)j * rs, a.d, lane, a.scale);
  for (int s = max(0, t - a.window + 1); s <= t; ++s) {
    const size_t slot = (size_t)(s % a.ring);  // ring: position s lives in slot s mod R
    fold(r, qv, kw + slot * rs, vw + slot * rs, a.d, lane, a.scale);
  }
  float* o = (float*)a.o + ((size_t)b * a.hq + qh) * a.d;
  const float inv = 1.f / r.l;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < a.d) o[c] = r.acc[i] * inv;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((unsigned)a.max_seqlen * a.hq, a.batch);
  prefill_f32_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.hq, a.batch);
  decode_f32_kernel<<<grid, 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace hca
