// Sparse-attention decode step of the full-context (MLA) layers on gfx950.
//
// What is computed (release blog "ERNIE 5.5 Flash Base", section 2.1; Zhidx
// article, section "1. Latent-Gated Sparse Attention"; model card: 256-dim
// heads in these layers): a lightweight indexer scores every past position
// of the query, and core attention runs only over the top-k positions, so
// its cost per query does not grow with the context.  The pages give no
// indexer form and no k; here (the readings of the library's header):
//   score(s) = qi . ki[s], one int8 head of width 128, exact in int32;
//   the k highest scores among positions 0 .. L-1, equal scores to the
//   smaller position, listed in increasing position order;
//   64 query heads of width 256 attend under one softmax (scale 1/16) to the
//   shared key/value rows of the selected positions.
//
// Kernels, in launch order:
//   dsa_zero_kernel    clears the per-sequence histogram of the score keys
//   dsa_score_kernel   (chunk of 4096 positions, sequence): integer scores
//                      with v_dot4 (sdot4), stored as keys u = score + 2^21
//                      in [0, 2^22]; adds its histogram of u >> 11 to the
//                      sequence's (global atomics on the non-empty bins)
//   dsa_select_kernel  (sequence): the exact threshold key by a two-level
//                      radix select (u >> 11 from the histogram, then u & 2047
//                      by one pass over the keys), then the selected
//                      positions in order: each thread counts its contiguous
//                      range, one block scan, each thread writes its range
//   dsa_attend_kernel  (split of 256 selected keys, sequence): 4 waves x 16
//                      heads on v_mfma_f32_16x16x32_bf16, gathered K and V
//                      rows double buffered in LDS, online softmax; writes
//                      m, l and O / l per split
//   dsa_merge_kernel   (sequence): combines the splits in order.
#include <algorithm>

#include "hca_internal.h"

namespace hca {
namespace {

constexpr int DD = 256;        // head width of the full-context layers
constexpr int DI = 128;        // indexer width (int8)
constexpr int HQ = 64;         // query heads
constexpr int CH = 4096;       // positions per scoring workgroup
constexpr int HBINS = 2049;    // bins of u >> 11 (u <= 2^22)
constexpr int LBINS = 2048;    // bins of u & 2047
constexpr int KEY_OFF = 1 << 21;
constexpr int SPLIT = 256;     // selected keys per attention workgroup
constexpr int TK = 32;         // keys per attention tile
constexpr int RS = 528;        // LDS bytes per staged key / value row (512 + 16)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float max_lanes16(float x) {
  // max over lanes l, l^16, l^32, l^48 (the four lanes that hold one head)
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dsa_zero_kernel(unsigned* hist, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) hist[i] = 0;
}

// ---------------------------------------------------------------------------
// Scores of positions [c CH, (c+1) CH) of sequence b: thread t takes
// positions c CH + t + 256 j.  The keys go to keys[b][position] (row stride
// max_seqlen), the histogram of u >> 11 to hist[b][HBINS].
__global__ __launch_bounds__(256) void dsa_score_kernel(DsaArgs a) {
  __shared__ unsigned hs[HBINS];
  const int c = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  const int p0 = c * CH;
  if (p0 >= L) return;
  for (int i = threadIdx.x; i < HBINS; i += 256) hs[i] = 0;
  // the query's 32 dwords of int8 (the same for every thread)
  const int* qw = (const int*)(a.qi + (size_t)b * DI);
  int q[DI / 4];
#pragma unroll
  for (int j = 0; j < DI / 4; ++j) q[j] = qw[j];
  __syncthreads();
  const size_t r0 = (size_t)a.cu_rows[b];
  unsigned* keys = a.keys + (size_t)b * a.max_seqlen;
  const int p1 = min(L, p0 + CH);
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const i32x4* kr = (const i32x4*)(a.ki + (r0 + p) * DI);
    int acc = 0;
#pragma unroll
    for (int j = 0; j < DI / 16; ++j) {
      const i32x4 kv = kr[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_sdot4(q[4 * j + e], kv[e], acc, false);
    }
    const unsigned u = (unsigned)(acc + KEY_OFF);
    keys[p] = u;
    atomicAdd(&hs[u >> 11], 1u);
  }
  __syncthreads();
  unsigned* gh = a.hist + (size_t)b * HBINS;
  for (int i = threadIdx.x; i < HBINS; i += 256)
    if (hs[i]) atomicAdd(&gh[i], hs[i]);
}

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one value per thread (256 threads), in thread
// order; returns the exclusive prefix and writes the total to *total.
__device__ __forceinline__ unsigned block_scan(unsigned v, unsigned* ws, unsigned* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned x = v;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) ws[wave] = x;
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += ws[w];
    tot += ws[w];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Sequence b: the selected positions, increasing, into sel[b][0 .. k) (-1
// after the first min(k, L)).
__global__ __launch_bounds__(256) void dsa_select_kernel(DsaArgs a) {
  __shared__ unsigned lh[LBINS];
  __shared__ unsigned wsum[4];
  __shared__ unsigned pick[4];  // hi bin, count above it, threshold key, ties to take
  const int b = blockIdx.x;
  const int L = a.seqlens[b];
  const int k = a.topk;
  int* sel = a.sel + (size_t)b * k;
  const unsigned* keys = a.keys + (size_t)b * a.max_seqlen;
  const int tid = threadIdx.x;
  if (L <= k) {  // every position
    for (int i = tid; i < k; i += 256) sel[i] = i < L ? i : -1;
    return;
  }
  // 1. hi bin from the histogram, counted from the top: thread t owns bins
  // HBINS-1-8t .. HBINS-8-8t (9 for the last thread)
  const unsigned* gh = a.hist + (size_t)b * HBINS;
  const int top = HBINS - 1 - 8 * tid;
  const int nb = tid == 255 ? HBINS - 8 * 255 : 8;
  unsigned cnt = 0;
  for (int i = 0; i < nb; ++i) cnt += gh[top - i];
  unsigned tot;
  const unsigned above = block_scan(cnt, wsum, &tot);  // keys in bins above this thread's
  if (above < (unsigned)k && above + cnt >= (unsigned)k) {
    unsigned acc = above;
    for (int i = 0; i < nb; ++i) {
      const unsigned h = gh[top - i];
      if (acc + h >= (unsigned)k) {
        pick[0] = top - i;
        pick[1] = acc;
        break;
      }
      acc += h;
    }
  }
  for (int i = tid; i < LBINS; i += 256) lh[i] = 0;
  __syncthreads();
  const unsigned hbin = pick[0], n_above = pick[1];
  // 2. low bits of the keys in the hi bin
  for (int p = tid; p < L; p += 256) {
    const unsigned u = keys[p];
    if ((u >> 11) == hbin) atomicAdd(&lh[u & 2047], 1u);
  }
  __syncthreads();
  {
    const int ltop = LBINS - 1 - 8 * tid;
    unsigned c2 = 0;
    for (int i = 0; i < 8; ++i) c2 += lh[ltop - i];
    unsigned t2;
    const unsigned ab = n_above + block_scan(c2, wsum, &t2);
    if (ab < (unsigned)k && ab + c2 >= (unsigned)k) {
      unsigned acc = ab;
      for (int i = 0; i < 8; ++i) {
        const unsigned h = lh[ltop - i];
        if (acc + h >= (unsigned)k) {
          pick[2] = (hbin << 11) | (unsigned)(ltop - i);
          pick[3] = (unsigned)k - acc;  // ties at the threshold to take, in position order
          break;
        }
        acc += h;
      }
    }
  }
  __syncthreads();
  const unsigned thr = pick[2], n_eq = pick[3];
  // 3. thread t scans positions [t R, (t+1) R): counts, scans, then writes
  const int R = (L + 255) / 256;
  const int q0 = min(L, tid * R), q1 = min(L, q0 + R);
  unsigned gt = 0, eq = 0;
  for (int p = q0; p < q1; ++p) {
    const unsigned u = keys[p];
    gt += u > thr;
    eq += u == thr;
  }
  unsigned t_gt, t_eq;
  const unsigned eq_before = block_scan(eq, wsum, &t_eq);
  const unsigned eq_take = eq_before >= n_eq ? 0u : min(eq, n_eq - eq_before);
  const unsigned out_before = block_scan(gt + eq_take, wsum, &t_gt);
  unsigned o = out_before, taken = 0;
  for (int p = q0; p < q1; ++p) {
    const unsigned u = keys[p];
    if (u > thr || (u == thr && taken < eq_take)) {
      if (u == thr) ++taken;
      if (o < (unsigned)k) sel[o] = p;  // the counts above make o < k; the guard keeps writes in the row
      ++o;
    }
  }
}

// ---------------------------------------------------------------------------
// Attention over split s (selected keys s SPLIT .. ) of sequence b: 256
// threads, wave w owns heads 16w .. 16w+15 (row l%16).  S^T = K Q^T (A = K
// rows from LDS, B = Q^T fragments), online softmax per head, O^T += V^T P^T
// (A = V^T by transposed LDS reads, B = P^T from the S^T accumulators with
// the keys in the k-slot order 4g+j, 16+4g+j of those reads).
// Workspace: m, l fp32 [B][nsplit][64], O / l bf16 [B][nsplit][64][256].
__device__ __forceinline__ bf16x8 lds_tr(const char HCA_LDS* base) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)base);
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)(base + 16 * RS));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

__global__ __launch_bounds__(256) void dsa_attend_kernel(DsaArgs a, int nsplit) {
  __shared__ __attribute__((aligned(16))) char kv_s[2][2 * TK * RS];
  const int s = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  const int nsel = min(L, a.topk);
  const int k0 = s * SPLIT;
  if (k0 >= nsel) return;
  const int k1 = min(nsel, k0 + SPLIT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int head = wave * 16 + r;
  const int* sel = a.sel + (size_t)b * a.topk;
  const size_t r0 = (size_t)a.cu_rows[b];
  const bf16* kg = (const bf16*)a.k;
  const bf16* vg = (const bf16*)a.v;

  bf16x8 qf[DD / 32];  // Q^T: lane l = head l%16, d = 32k + 8g .. +7
  {
    const bf16* qr = (const bf16*)a.q + ((size_t)b * HQ + head) * DD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DD / 32; ++kk) qf[kk] = *(const bf16x8*)(qr + 32 * kk);
  }
  // gather of one tile: thread t copies 16-byte chunks t, t+256 of the 32 K
  // rows and of the 32 V rows (32 chunks per row)
  auto load_tile = [&](int t0, bf16x8 (&st)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + 256 * j, row = c >> 5, col = c & 31;
      const int kk = t0 + row;
      const size_t pos = r0 + (size_t)min(max(sel[min(kk, k1 - 1)], 0), L - 1);  // clamp: rows of the sequence
      st[j] = *(const bf16x8*)(kg + pos * DD + 8 * col);
      st[4 + j] = *(const bf16x8*)(vg + pos * DD + 8 * col);
    }
  };
  auto store_tile = [&](char HCA_LDS* buf, const bf16x8 (&st)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + 256 * j, row = c >> 5, col = c & 31;
      *(bf16x8 HCA_LDS*)(buf + row * RS + 16 * col) = st[j];
      *(bf16x8 HCA_LDS*)(buf + TK * RS + row * RS + 16 * col) = st[4 + j];
    }
  };
  const float sc2 = a.scale * kLog2e;
  f32x4 o[DD / 16];
#pragma unroll
  for (int ct = 0; ct < DD / 16; ++ct) o[ct] = f32x4{};
  float m = -INFINITY, l = 0.f;
  bf16x8 st[8];
  load_tile(k0, st);
  store_tile((char HCA_LDS*)kv_s[0], st);
  __syncthreads();
  int buf = 0;
  for (int t0 = k0; t0 < k1; t0 += TK, buf ^= 1) {
    const bool more = t0 + TK < k1;
    if (more) load_tile(t0 + TK, st);  // in flight during this tile's math
    const char HCA_LDS* kb = (const char HCA_LDS*)kv_s[buf];
    const char HCA_LDS* vb = kb + TK * RS;
    f32x4 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < DD / 32; ++kk) {
      const bf16x8 a0 = *(const bf16x8 HCA_LDS*)(kb + r * RS + kk * 64 + g * 16);
      const bf16x8 a1 = *(const bf16x8 HCA_LDS*)(kb + (16 + r) * RS + kk * 64 + g * 16);
      s0 = mfma16(a0, qf[kk], s0);
      s1 = mfma16(a1, qf[kk], s1);
    }
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // keys t0 + 4g + i and t0 + 16 + 4g + i
      x[i] = t0 + 4 * g + i < k1 ? s0[i] * sc2 : -INFINITY;
      x[4 + i] = t0 + 16 + 4 * g + i < k1 ? s1[i] * sc2 : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
    const float mn = fmaxf(m, max_lanes16(mx));
    const float alpha = __builtin_amdgcn_exp2f(m - mn);  // m = -inf: 0
    bf16x8 pb;
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(x[i] - mn);
      pb[i] = (bf16)p;
      ls += (float)pb[i];
    }
    l = l * alpha + ls;
    m = mn;
#pragma unroll
    for (int ct = 0; ct < DD / 16; ++ct) o[ct] = o[ct] * alpha;
    const char HCA_LDS* vt = vb + (4 * g + (r >> 2)) * RS + 8 * (lane & 3);
#pragma unroll
    for (int ct = 0; ct < DD / 16; ++ct) o[ct] = mfma16(lds_tr(vt + 32 * ct), pb, o[ct]);
    __syncthreads();  // every wave is done with the other buffer
    if (more) store_tile((char HCA_LDS*)kv_s[buf ^ 1], st);
    __syncthreads();
  }
  // partial of this split: m (log2 units), l, O / l
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  const size_t prow = ((size_t)b * nsplit + s) * HQ + head;
  if (lane < 16) {
    a.part_m[prow] = m;
    a.part_l[prow] = lt;
  }
  const float inv = 1.f / lt;
  bf16* po = a.part_o + prow * DD + 4 * g;
#pragma unroll
  for (int ct = 0; ct < DD / 16; ++ct) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[ct][i] * inv);
    *(bf16x4*)(po + 16 * ct) = v;
  }
}

// Merge of the splits of sequence b in order: O = sum_s 2^(m_s - M) l_s O_s /
// sum_s 2^(m_s - M) l_s.  256 threads: thread t takes head t / 4 and
// columns 64 (t % 4) .. +63.
__global__ __launch_bounds__(256) void dsa_merge_kernel(DsaArgs a, int nsplit) {
  const int b = blockIdx.x;
  const int nsel = min(a.seqlens[b], a.topk);
  const int ns = (nsel + SPLIT - 1) / SPLIT;
  const int head = threadIdx.x >> 2, c0 = 64 * (threadIdx.x & 3);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_m[((size_t)b * nsplit + s) * HQ + head]);
  float acc[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) acc[i] = 0.f;
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const size_t prow = ((size_t)b * nsplit + s) * HQ + head;
    const float wgt = __builtin_amdgcn_exp2f(a.part_m[prow] - M) * a.part_l[prow];
    den += wgt;
    const bf16* po = a.part_o + prow * DD + c0;
#pragma unroll
    for (int i = 0; i < 64; i += 8) {
      const bf16x8 v = *(const bf16x8*)(po + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i + e] = __builtin_fmaf(wgt, (float)v[e], acc[i + e]);
    }
  }
  const float inv = 1.f / den;
  bf16* out = (bf16*)a.o + ((size_t)b * HQ + head) * DD + c0;
#pragma unroll
  for (int i = 0; i < 64; i += 8) {
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)(acc[i + e] * inv);
    *(bf16x8*)(out + i) = v;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t dsa_workspace_bytes(int batch, int max_seqlen, int topk) {
  const int nsplit = (std::min(max_seqlen, topk) + SPLIT - 1) / SPLIT;
  size_t n = 0;
  n += align256((size_t)batch * max_seqlen * sizeof(unsigned));   // keys
  n += align256((size_t)batch * HBINS * sizeof(unsigned));        // histogram
  n += 2 * align256((size_t)batch * nsplit * HQ * sizeof(float)); // m, l
  n += align256((size_t)batch * nsplit * HQ * DD * sizeof(bf16)); // O / l
  return n;
}

hipError_t launch_dsa_decode(DsaArgs a, hipStream_t s) {
  const int nsplit = (std::min(a.max_seqlen, a.topk) + SPLIT - 1) / SPLIT;
  char* w = (char*)a.ws;
  a.keys = (unsigned*)w;
  w += align256((size_t)a.batch * a.max_seqlen * sizeof(unsigned));
  a.hist = (unsigned*)w;
  w += align256((size_t)a.batch * HBINS * sizeof(unsigned));
  a.part_m = (float*)w;
  w += align256((size_t)a.batch * nsplit * HQ * sizeof(float));
  a.part_l = (float*)w;
  w += align256((size_t)a.batch * nsplit * HQ * sizeof(float));
  a.part_o = (bf16*)w;
  const int nh = a.batch * HBINS;
  dsa_zero_kernel<<<(nh + 255) / 256, 256, 0, s>>>(a.hist, nh);
  dsa_score_kernel<<<dim3((a.max_seqlen + CH - 1) / CH, a.batch), 256, 0, s>>>(a);
  dsa_select_kernel<<<a.batch, 256, 0, s>>>(a);
  dsa_attend_kernel<<<dim3(nsplit, a.batch), 256, 0, s>>>(a, nsplit);
  dsa_merge_kernel<<<a.batch, 256, 0, s>>>(a, nsplit);
  return hipGetLastError();
}

}  // namespace hca
