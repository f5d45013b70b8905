// Block pooling: every complete 128-token block of K (and V) becomes one
// cached entry (release blog "ERNIE 5.5 Flash Base", section 2.1, HCA
// paragraph).  The pooling function is a softmax(w_h)-weighted sum over the
// block's rows with a learned length-128 logit vector per KV head.
//
// HBM-bound (1 flop per byte).  One workgroup of 256 threads pools one
// (entry, KV head, tensor) over a column slice of CW elements:
//   - every thread owns 16 contiguous bytes of a row (VEC elements), TPR
//     threads cover the slice of one row, RPP = 256/TPR rows are read per pass,
//     so each load instruction reads whole rows of the slice (coalesced) and a
//     workgroup keeps 128 rows x CW elements in flight over a few passes;
//   - fp32 partial sums are reduced first across the rows held by one
//     wavefront (lane shuffles) and then across the 4 wavefronts through LDS.
//
// Chunk mode (CHUNK = true) pools the blocks that n new rows at positions
// p0 .. p0+n-1 of a sequence complete: block j with p0 <= 128j+127 <= p0+n-1.
// Its rows at positions >= p0 are the new rows; the earlier ones (at most
// 127) come from the sequence's raw ring, where position s sits in slot
// s % ring_cap.  The entry goes to index cu_blocks[b] + j of the cache.
#include "hca_internal.h"

namespace hca {
namespace {

template <typename T, int TPR, bool CHUNK>
__global__ __launch_bounds__(256) void compress_kernel(CompressArgs a, int cw) {
  constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte load
  constexpr int RPP = 256 / TPR;          // rows per pass
  constexpr int PASSES = kBlock / RPP;
  static_assert(kBlock % RPP == 0, "rows per pass must divide the block");
  __shared__ float p_s[4][kBlock];  // one copy per wavefront
  __shared__ float red_s[4][TPR * VEC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int entry_head = blockIdx.x;              // entry * hkv + head
  const int h = entry_head % a.hkv;
  const int c0 = blockIdx.y * cw;                 // first column of the slice
  const int which = blockIdx.z;                   // 0: K -> Kc, 1: V -> Vc
  const size_t rstride = (size_t)a.hkv * a.d;     // elements between tokens
  int entry, seq, j;                              // output entry; its sequence and block
  if (CHUNK) {
    // blockIdx.x = (b * max_new + x) * hkv + h: the x-th block completed by
    // sequence b's new rows, if there is one
    const int bx = entry_head / a.hkv;
    seq = bx / a.max_new;
    const int p0 = a.pos0[seq];
    const int n = a.cu_seqlens[seq + 1] - a.cu_seqlens[seq];
    j = p0 / kBlock + bx % a.max_new;
    // not completed by these rows, or past the sequence's cache capacity:
    // the whole workgroup leaves
    if (kBlock * (j + 1) > p0 + n || j >= a.cu_blocks[seq + 1] - a.cu_blocks[seq]) return;
    entry = a.cu_blocks[seq] + j;
  } else {
    entry = entry_head / a.hkv;
    // which sequence owns this entry: largest b with cu_blocks[b] <= entry
    int lo = 0, hi = a.batch;  // invariant: cu_blocks[lo] <= entry < cu_blocks[hi]
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (a.cu_blocks[mid] <= entry) lo = mid; else hi = mid;
    }
    seq = lo;
    j = entry - a.cu_blocks[lo];
  }

  const size_t col = (size_t)h * a.d + c0 + (tid % TPR) * VEC;  // this thread's first element in a row
  const int r0 = tid / TPR;

  // the pooling logits first: loads complete in issue order, so logits
  // issued after the rows would make the softmax below wait for every row
  const float w0 = a.w[h * kBlock + lane], w1 = a.w[h * kBlock + 64 + lane];
  __builtin_amdgcn_sched_barrier(0);
  // all of this thread's loads are issued before any is used, so a thread
  // keeps PASSES 16-byte loads in flight (the default schedule would wait
  // for each load before issuing the next)
  typedef T vec_t __attribute__((ext_vector_type(VEC)));
  vec_t xv[PASSES];
  if (CHUNK) {
    const int p0 = a.pos0[seq], tok0 = a.cu_seqlens[seq];
    const T* xnew = (const T*)a.x[which] + col;
    const T* ring = (const T*)a.ring[which] + col;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int pos = kBlock * j + ps * RPP + r0;
      const bool is_new = pos >= p0;
      const size_t row = is_new ? (size_t)(tok0 + (pos - p0)) : (size_t)seq * a.ring_cap + pos % a.ring_cap;
      xv[ps] = *(const vec_t*)((is_new ? xnew : ring) + row * rstride);
    }
  } else {
    const size_t tok0 = (size_t)a.cu_seqlens[seq] + (size_t)kBlock * j;
    const T* x = (const T*)a.x[which] + tok0 * rstride + col;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps)  // rows pooled once: non-temporal
      xv[ps] = __builtin_nontemporal_load((const vec_t*)(x + (size_t)(ps * RPP + r0) * rstride));
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of their uses

  // pooling weights p = softmax(w_h), max-subtracted, in fp32, while the
  // rows are in flight.  Every wavefront computes all 128 weights (two per
  // lane, wave-wide max and sum) and writes them to its own p_s row, which
  // only its lanes read afterwards: a wavefront-scope release / acquire
  // around a wave barrier orders the lanes' stores before the other lanes'
  // loads (no workgroup barrier, which would also wait for the row loads).
  {
    float mx = fmaxf(w0, w1);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float e0 = expf(w0 - mx), e1 = expf(w1 - mx);
    float sm = e0 + e1;
    for (int off = 32; off > 0; off >>= 1) sm += __shfl_xor(sm, off);
    p_s[wave][lane] = e0 / sm;
    p_s[wave][64 + lane] = e1 / sm;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  float acc[VEC];
#pragma unroll
  for (int c = 0; c < VEC; ++c) acc[c] = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const float pr = p_s[wave][ps * RPP + r0];
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] = fmaf(pr, to_f32(xv[ps][c]), acc[c]);
  }
  // reduce over the rows a wavefront holds (lanes that differ in the bits
  // above log2(TPR)), then over the 4 wavefronts
#pragma unroll
  for (int off = 32; off >= TPR; off >>= 1) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) acc[c] += __shfl_xor(acc[c], off);
  }
  if (lane < TPR) {
#pragma unroll
    for (int c = 0; c < VEC; ++c) red_s[wave][lane * VEC + c] = acc[c];
  }
  __syncthreads();
  for (int i = tid; i < TPR * VEC; i += 256) {
    float s = (red_s[0][i] + red_s[1][i]) + (red_s[2][i] + red_s[3][i]);
    T* out = (T*)a.xc[which] + ((size_t)entry * a.hkv + h) * a.d + c0;
    out[i] = from_f32<T>(s);
  }
}

template <typename T, bool CHUNK>
hipError_t launch_typed(const CompressArgs& a, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  // Largest column slice (at most 64 threads x 16 bytes per row, dividing d)
  // that still gives at least ~1024 workgroups; never below 64 elements.
  const long work = (long)a.total_blocks * a.hkv * (a.x[1] ? 2 : 1);  // chunk mode: an upper bound
  int cw = 64;
  for (int c = 64 * VEC; c >= 64; c >>= 1) {
    if (a.d % c) continue;
    cw = c;
    if (work * (a.d / c) >= 1024) break;
  }
  dim3 grid(a.total_blocks * a.hkv, a.d / cw, a.x[1] ? 2 : 1);
  const int tpr = cw / VEC;
  switch (tpr) {
    case 64: compress_kernel<T, 64, CHUNK><<<grid, 256, 0, s>>>(a, cw); break;
    case 32: compress_kernel<T, 32, CHUNK><<<grid, 256, 0, s>>>(a, cw); break;
    case 16: compress_kernel<T, 16, CHUNK><<<grid, 256, 0, s>>>(a, cw); break;
    case 8: compress_kernel<T, 8, CHUNK><<<grid, 256, 0, s>>>(a, cw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(int dtype, const CompressArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_typed<bf16, false>(a, s) : launch_typed<float, false>(a, s);
}

// Chunk mode: a.total_blocks = batch * max_new candidate blocks (the grid),
// most of them possibly empty.
hipError_t launch_compress_chunk(int dtype, const CompressArgs& a, hipStream_t s) {
  return dtype == 1 ? launch_typed<bf16, true>(a, s) : launch_typed<float, true>(a, s);
}

}  // namespace hca
