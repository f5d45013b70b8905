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
//   dsa_zero_kernel    clears the per-sequence histograms of the score keys
//   dsa_score_kernel   (chunk of 4096 positions, sequence): integer scores
//                      with v_dot4 (sdot4), 8 lanes per indexer row so that
//                      the loads are contiguous (and non-temporal: each row
//                      is read once), stored as keys u = score + 2^21 in
//                      [0, 2^22]; adds its histogram of u >> 11 to the
//                      sequence's (global atomics on the non-empty bins)
//   dsa_lohist_kernel, dsa_count_kernel, dsa_emit_kernel  (chunk,
//                      sequence): the exact threshold key by a two-level
//                      radix select (u >> 11 from the histogram, then u & 2047
//                      from a histogram of the keys in that bin), each
//                      chunk's counts, then the selected positions in order
//   dsa_attend_kernel  (split of 256 selected keys, sequence): 4 waves x 16
//                      heads on v_mfma_f32_16x16x32_bf16; the split's cache
//                      rows staged in LDS, two tiles of gathered K and V rows
//                      in flight in registers while one is computed from LDS,
//                      online softmax; writes m, l and O / l per split
//   dsa_merge_kernel   (8 heads, sequence): combines the splits in order.
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

// keys per sequence row of the key buffer: max_seqlen rounded up to a whole
// chunk, so a chunk's 4096 keys are always inside its row
__host__ __device__ inline int key_stride(int max_seqlen) { return (max_seqlen + CH - 1) / CH * CH; }

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
// Scores of positions [c CH, (c+1) CH) of sequence b.  Eight lanes share one
// indexer row (lane l reads bytes 16 (l%8) .. +15 of row l/8 of its group),
// so each wave load moves 8 whole rows (1 KiB, contiguous); three shuffles
// add the 8 partial dot products.  Wave w takes rows 32 i + 8 w + l/8 of the
// chunk, four groups per step in flight.  The keys go to keys[b][position],
// the histogram of u >> 11 to hist[b][HBINS].
__global__ __launch_bounds__(256) void dsa_score_kernel(DsaArgs a) {
  __shared__ unsigned hs[HBINS];
  const int c = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  const int p0 = c * CH;
  if (p0 >= L) return;
  for (int i = threadIdx.x; i < HBINS; i += 256) hs[i] = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, part = lane & 7;
  // this lane's 16 bytes of the indexer query
  const i32x4 q = *(const i32x4*)(a.qi + (size_t)b * DI + 16 * part);
  __syncthreads();
  const size_t r0 = (size_t)a.cu_rows[b];
  unsigned* keys = a.keys + (size_t)b * key_stride(a.max_seqlen);
  const int p1 = min(L, p0 + CH);
  for (int pb = p0 + 8 * wave + (lane >> 3); pb < p1; pb += 4 * 32) {
    i32x4 kv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int p = min(pb + 32 * x, p1 - 1);  // past the end: the last row again (not stored)
      kv[x] = __builtin_nontemporal_load((const i32x4*)(a.ki + (r0 + p) * DI + 16 * part));  // read once
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      int acc = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_sdot4(q[e], kv[x][e], acc, false);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      const int p = pb + 32 * x;
      if (part == 0 && p < p1) {
        const unsigned u = (unsigned)(acc + KEY_OFF);
        keys[p] = u;
        atomicAdd(&hs[u >> 11], 1u);
      }
    }
  }
  __syncthreads();
  unsigned* gh = a.hist + (size_t)b * HBINS;
  for (int i = threadIdx.x; i < HBINS; i += 256)
    if (hs[i]) atomicAdd(&gh[i], hs[i]);
}

// ---------------------------------------------------------------------------
// Keys are read four per lane (16 bytes): a group of 256 consecutive
// positions has lane l holding 4l .. 4l+3.  Rows of the key buffer are padded
// to whole chunks of CH positions; positions >= L are masked by index.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned wave_sum(unsigned v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// The selection runs on chunks of CH positions (the scoring's), in three
// kernels; each recomputes the same thresholds from the histograms, so all
// workgroups agree:
//   dsa_lohist_kernel  the hi bin (u >> 11) holding the k-th largest key,
//                      from the histogram; the chunk's histogram of the low
//                      bits of the keys in that bin, added to the sequence's;
//   dsa_count_kernel   the exact threshold key and the ties at it to take
//                      (from both histograms); the chunk's keys above the
//                      threshold and at it;
//   dsa_emit_kernel    the chunk's output offset and tie budget from the
//                      counts of the chunks before it; its selected
//                      positions in order (per wave: 1024 positions, ballot
//                      prefix counts).

// Wave 0: the first t in the 256 partial counts cnt[] (ordered from the top
// bin down) at which acc0 plus the running sum reaches k; res[0] = t,
// res[1] = acc0 plus the counts before t.  Lane l scans cnt[4l .. 4l+3].
__device__ __forceinline__ void first_reach(const unsigned* cnt, unsigned acc0, unsigned k, unsigned* res) {
  const int lane = threadIdx.x & 63;
  unsigned c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = cnt[4 * lane + e];
  const unsigned tot = c[0] + c[1] + c[2] + c[3];
  unsigned incl = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const unsigned long long m = __ballot(acc0 + incl >= k);
  const int first = m ? __builtin_ctzll(m) : 63;  // (every count reaches k: the bound keeps t < 256)
  if (lane == first) {
    unsigned acc = acc0 + incl - tot;
    int t = 4 * lane;
#pragma unroll
    for (int e = 0; e < 3; ++e) {
      if (acc + c[e] >= k) break;
      acc += c[e];
      ++t;
    }
    res[0] = (unsigned)t;
    res[1] = acc;
  }
}

// Bin selection shared by the selection kernels.  Thread t holds bins
// top - 8t .. top - 8t - 7 of a histogram in registers (thread 255 of the
// hi histogram also bin 0); `cnt` is 256 words of LDS, `res` 2, `pick` 4.
//   find_hi:        pick[0] = the hi bin holding the k-th largest key,
//                   pick[1] = keys in bins above it;
//   find_threshold: pick[2] = the k-th largest key, pick[3] = the keys equal
//                   to it that are selected (the first ones by position).
__device__ __forceinline__ void find_hi(const unsigned* gh, int k, unsigned* cnt, unsigned* res, unsigned* pick) {
  const int tid = threadIdx.x;
  const int top = HBINS - 1 - 8 * tid;
  unsigned h[9];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = gh[top - i];
  h[8] = tid == 255 ? gh[0] : 0u;
  unsigned c = 0;
#pragma unroll
  for (int i = 0; i < 9; ++i) c += h[i];
  cnt[tid] = c;
  __syncthreads();
  if (tid < 64) first_reach(cnt, 0u, (unsigned)k, res);
  __syncthreads();
  if (tid == (int)res[0]) {
    unsigned acc = res[1];
    int i = 0;
    while (i < 8 && acc + h[i] < (unsigned)k) acc += h[i++];
    pick[0] = (unsigned)(top - i);
    pick[1] = acc;
  }
  __syncthreads();
}

__device__ __forceinline__ void find_threshold(const unsigned* lo, int k, unsigned* cnt, unsigned* res,
                                               unsigned* pick) {
  const int tid = threadIdx.x;
  const int ltop = LBINS - 1 - 8 * tid;
  unsigned h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = lo[ltop - i];
  unsigned c = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) c += h[i];
  cnt[tid] = c;
  __syncthreads();
  if (tid < 64) first_reach(cnt, pick[1], (unsigned)k, res);
  __syncthreads();
  if (tid == (int)res[0]) {
    unsigned acc = res[1];
    int i = 0;
    while (i < 7 && acc + h[i] < (unsigned)k) acc += h[i++];
    pick[2] = (pick[0] << 11) | (unsigned)(ltop - i);
    pick[3] = (unsigned)k - acc;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void dsa_lohist_kernel(DsaArgs a, int kstride) {
  __shared__ unsigned lh[LBINS];
  __shared__ unsigned cnt[256];
  __shared__ unsigned res[2], pick[4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  if (L <= a.topk || c * CH >= L) return;
  for (int i = threadIdx.x; i < LBINS; i += 256) lh[i] = 0;
  find_hi(a.hist + (size_t)b * HBINS, a.topk, cnt, res, pick);
  const unsigned hbin = pick[0];
  const u32x4* keys4 = (const u32x4*)(a.keys + (size_t)b * kstride + (size_t)c * CH);
  const int n = min(CH, L - c * CH);
  for (int i = threadIdx.x; 4 * i < n; i += 256) {
    const u32x4 kv = keys4[i];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * i + e < n && (kv[e] >> 11) == hbin) atomicAdd(&lh[kv[e] & 2047], 1u);
  }
  __syncthreads();
  unsigned* gl = a.lohist + (size_t)b * LBINS;
  for (int i = threadIdx.x; i < LBINS; i += 256)
    if (lh[i]) atomicAdd(&gl[i], lh[i]);
}

__global__ __launch_bounds__(256) void dsa_count_kernel(DsaArgs a, int kstride, int nchunk) {
  __shared__ unsigned cnt[256];
  __shared__ unsigned res[2], pick[4];
  __shared__ unsigned red[2][4];
  const int c = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  if (L <= a.topk || c * CH >= L) return;
  find_hi(a.hist + (size_t)b * HBINS, a.topk, cnt, res, pick);
  find_threshold(a.lohist + (size_t)b * LBINS, a.topk, cnt, res, pick);
  const unsigned thr = pick[2];
  const u32x4* keys4 = (const u32x4*)(a.keys + (size_t)b * kstride + (size_t)c * CH);
  const int n = min(CH, L - c * CH);
  unsigned gt = 0, eq = 0;
  for (int i = threadIdx.x; 4 * i < n; i += 256) {
    const u32x4 kv = keys4[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = 4 * i + e < n;
      gt += in && kv[e] > thr;
      eq += in && kv[e] == thr;
    }
  }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[0][wave] = gt;
    red[1][wave] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned* out = a.chunk_cnt + ((size_t)b * nchunk + c) * 2;
    out[0] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    out[1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
    if (c == 0) {
      a.thr[2 * b] = thr;
      a.thr[2 * b + 1] = pick[3];
    }
  }
}

__global__ __launch_bounds__(256) void dsa_emit_kernel(DsaArgs a, int kstride, int nchunk) {
  __shared__ unsigned seg[2][4];  // per wave: keys above the threshold, ties at it
  __shared__ unsigned base[2];    // output offset and ties before this chunk
  const int c = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  const int k = a.topk;
  int* sel = a.sel + (size_t)b * k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (L <= k) {  // every position; chunk c writes slots [c CH, (c+1) CH) of the row
    for (int i = c * CH + tid; i < min(k, (c + 1) * CH); i += 256) sel[i] = i < L ? i : -1;
    return;
  }
  if (c * CH >= L) return;
  const unsigned thr = a.thr[2 * b], n_eq = a.thr[2 * b + 1];
  if (wave == 0) {  // the chunks before this one: keys above, ties seen; of those ties the first n_eq are taken
    unsigned gtb = 0, eqb = 0;
    const unsigned* cc = a.chunk_cnt + (size_t)b * nchunk * 2;
    for (int j = lane; j < c; j += 64) {
      gtb += cc[2 * j];
      eqb += cc[2 * j + 1];
    }
    gtb = wave_sum(gtb);
    eqb = wave_sum(eqb);
    if (lane == 0) {
      base[0] = gtb + min(eqb, n_eq);
      base[1] = eqb;
    }
  }
  const int n = min(CH, L - c * CH);
  const int p0c = c * CH;
  // wave w: positions [1024 w, 1024 (w+1)) of the chunk, four groups of 256
  const u32x4* keys4 = (const u32x4*)(a.keys + (size_t)b * kstride + (size_t)p0c);
  u32x4 kv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kv[j] = keys4[(4 * wave + j) * 64 + lane];  // inside the padded row
  unsigned gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = (4 * wave + j) * 256 + 4 * lane + e;
      gt += q < n && kv[j][e] > thr;
      eq += q < n && kv[j][e] == thr;
    }
  gt = wave_sum(gt);
  eq = wave_sum(eq);
  if (lane == 0) {
    seg[0][wave] = gt;
    seg[1][wave] = eq;
  }
  __syncthreads();
  unsigned out = base[0], eqb = base[1];
  for (int w = 0; w < wave; ++w) {
    const unsigned take = eqb >= n_eq ? 0u : min(seg[1][w], n_eq - eqb);
    out += seg[0][w] + take;
    eqb += seg[1][w];
  }
  const unsigned budget = eqb >= n_eq ? 0u : min(seg[1][wave], n_eq - eqb);  // ties this wave takes
  const unsigned long long below = (1ull << lane) - 1ull;
  unsigned ties_seen = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q0 = (4 * wave + j) * 256 + 4 * lane;
    bool g4[4], e4[4];
    unsigned ng = 0, ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g4[e] = q0 + e < n && kv[j][e] > thr;
      e4[e] = q0 + e < n && kv[j][e] == thr;
      ng += g4[e];
      ne += e4[e];
    }
    if (__ballot(ng + ne > 0) == 0) continue;
    unsigned te = 0, tt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned long long m = __ballot(e4[e]);
      te += __popcll(m & below);
      tt += __popcll(m);
    }
    const unsigned tb = ties_seen + te;
    const unsigned nt = tb >= budget ? 0u : min(ne, budget - tb);
    const unsigned mine = ng + nt;
    unsigned oe = 0, ot = 0;
#pragma unroll
    for (int bit = 0; bit < 3; ++bit) {  // mine <= 4
      const unsigned long long m = __ballot((mine >> bit) & 1u);
      oe += (unsigned)__popcll(m & below) << bit;
      ot += (unsigned)__popcll(m) << bit;
    }
    unsigned o = out + oe, taken = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (g4[e] || (e4[e] && taken < nt)) {
        if (e4[e]) ++taken;
        if (o < (unsigned)k) sel[o] = p0c + q0 + e;  // the counts make o < k; the guard keeps writes in the row
        ++o;
      }
    }
    out += ot;
    ties_seen += tt;
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

__global__ __launch_bounds__(256, 2) void dsa_attend_kernel(DsaArgs a, int nsplit) {
  __shared__ __attribute__((aligned(16))) char kv_s[2][2 * TK * RS];
  __shared__ int row_s[SPLIT];  // cache row of each selected key of the split
  const int s = blockIdx.x, b = blockIdx.y;
  const int L = a.seqlens[b];
  const int nsel = min(L, a.topk);
  const int k0 = s * SPLIT;
  if (k0 >= nsel) return;
  const int k1 = min(nsel, k0 + SPLIT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const int head = wave * 16 + r;
  const bf16* kg = (const bf16*)a.k;
  const bf16* vg = (const bf16*)a.v;
  {
    // slots past k1 repeat the last selected key (their scores are masked);
    // positions are clamped to the sequence's rows
    const int* sel = a.sel + (size_t)b * a.topk;
    const int kk = min(k0 + (int)threadIdx.x, k1 - 1);
    row_s[threadIdx.x] = a.cu_rows[b] + min(max(sel[kk], 0), L - 1);
  }

  bf16x8 qf[DD / 32];  // Q^T: lane l = head l%16, d = 32k + 8g .. +7
  {
    const bf16* qr = (const bf16*)a.q + ((size_t)b * HQ + head) * DD + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DD / 32; ++kk) qf[kk] = *(const bf16x8*)(qr + 32 * kk);
  }
  // gather of one tile: thread t copies 16-byte chunks t, t+256, t+512, t+768
  // of the 32 K rows and of the 32 V rows (32 chunks per row)
  auto load_tile = [&](int t0, bf16x8 (&st)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + 256 * j, row = c >> 5, col = c & 31;
      const size_t pos = (size_t)row_s[t0 - k0 + row];
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
  auto tile_math = [&](const char HCA_LDS* kb, int t0) {
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
  };
  // two tiles in flight: tile t0 + TK arrives in one register set while tile
  // t0 + 2 TK is issued into the other; buffers alternate with the tile
  char HCA_LDS* buf0 = (char HCA_LDS*)kv_s[0];
  char HCA_LDS* buf1 = (char HCA_LDS*)kv_s[1];
  bf16x8 st0[8], st1[8];
  __syncthreads();  // row_s
  load_tile(k0, st0);
  if (k0 + TK < k1) load_tile(k0 + TK, st1);
  store_tile(buf0, st0);
  __syncthreads();
  for (int t0 = k0; t0 < k1; t0 += 2 * TK) {
    if (t0 + 2 * TK < k1) load_tile(t0 + 2 * TK, st0);
    tile_math(buf0, t0);
    if (t0 + TK >= k1) break;  // uniform
    __syncthreads();  // every wave is done with buf1's previous tile
    store_tile(buf1, st1);
    __syncthreads();
    if (t0 + 3 * TK < k1) load_tile(t0 + 3 * TK, st1);
    tile_math(buf1, t0 + TK);
    if (t0 + 2 * TK >= k1) break;
    __syncthreads();
    store_tile(buf0, st0);
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
// sum_s 2^(m_s - M) l_s.  Workgroup (8 heads, sequence), thread = (head, 8
// columns); the splits' partials are loaded together, eight at a time, and
// combined in split order.
__global__ __launch_bounds__(256) void dsa_merge_kernel(DsaArgs a, int nsplit) {
  const int b = blockIdx.y;
  const int nsel = min(a.seqlens[b], a.topk);
  const int ns = (nsel + SPLIT - 1) / SPLIT;
  const int head = 8 * blockIdx.x + (threadIdx.x >> 5), c0 = 8 * (threadIdx.x & 31);
  const size_t prow0 = (size_t)b * nsplit * HQ + head;  // split s: prow0 + s HQ
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_m[prow0 + (size_t)s * HQ]);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  float den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 8) {
    bf16x8 v[8];
    float wgt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < ns) {
        const size_t prow = prow0 + (size_t)(s0 + j) * HQ;
        v[j] = *(const bf16x8*)(a.part_o + prow * DD + c0);
        wgt[j] = __builtin_amdgcn_exp2f(a.part_m[prow] - M) * a.part_l[prow];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < ns) {
        den += wgt[j];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(wgt[j], (float)v[j][e], acc[e]);
      }
    }
  }
  const float inv = 1.f / den;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (bf16)(acc[e] * inv);
  *(bf16x8*)((bf16*)a.o + ((size_t)b * HQ + head) * DD + c0) = o;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t dsa_workspace_bytes(int batch, int max_seqlen, int topk) {
  const int nsplit = (std::min(max_seqlen, topk) + SPLIT - 1) / SPLIT;
  size_t n = 0;
  n += align256((size_t)batch * key_stride(max_seqlen) * sizeof(unsigned));  // keys
  n += align256((size_t)batch * HBINS * sizeof(unsigned));        // histogram
  n += align256((size_t)batch * LBINS * sizeof(unsigned));        // low-bit histogram in the hi bin
  n += align256((size_t)batch * ((max_seqlen + CH - 1) / CH) * 2 * sizeof(unsigned));  // chunk counts
  n += align256((size_t)batch * 2 * sizeof(unsigned));            // threshold, ties
  n += 2 * align256((size_t)batch * nsplit * HQ * sizeof(float)); // m, l
  n += align256((size_t)batch * nsplit * HQ * DD * sizeof(bf16)); // O / l
  return n;
}

hipError_t launch_dsa_decode(DsaArgs a, hipStream_t s) {
  const int nsplit = (std::min(a.max_seqlen, a.topk) + SPLIT - 1) / SPLIT;
  char* w = (char*)a.ws;
  a.keys = (unsigned*)w;
  w += align256((size_t)a.batch * key_stride(a.max_seqlen) * sizeof(unsigned));
  const int nchunk = (a.max_seqlen + CH - 1) / CH;
  a.hist = (unsigned*)w;
  w += align256((size_t)a.batch * HBINS * sizeof(unsigned));
  a.lohist = (unsigned*)w;
  w += align256((size_t)a.batch * LBINS * sizeof(unsigned));
  a.chunk_cnt = (unsigned*)w;
  w += align256((size_t)a.batch * nchunk * 2 * sizeof(unsigned));
  a.thr = (unsigned*)w;
  w += align256((size_t)a.batch * 2 * sizeof(unsigned));
  a.part_m = (float*)w;
  w += align256((size_t)a.batch * nsplit * HQ * sizeof(float));
  a.part_l = (float*)w;
  w += align256((size_t)a.batch * nsplit * HQ * sizeof(float));
  a.part_o = (bf16*)w;
  // hist [B, HBINS] and lohist [B, LBINS] are adjacent (256-byte alignment padding between): one clear
  const int nh = (int)(((char*)a.chunk_cnt - (char*)a.hist) / sizeof(unsigned));
  dsa_zero_kernel<<<(nh + 255) / 256, 256, 0, s>>>(a.hist, nh);
  const dim3 chunks(nchunk, a.batch);
  const int ks = key_stride(a.max_seqlen);
  dsa_score_kernel<<<chunks, 256, 0, s>>>(a);
  dsa_lohist_kernel<<<chunks, 256, 0, s>>>(a, ks);
  dsa_count_kernel<<<chunks, 256, 0, s>>>(a, ks, nchunk);
  dsa_emit_kernel<<<dim3(std::max(nchunk, (a.topk + CH - 1) / CH), a.batch), 256, 0, s>>>(a, ks, nchunk);
  dsa_attend_kernel<<<dim3(nsplit, a.batch), 256, 0, s>>>(a, nsplit);
  dsa_merge_kernel<<<dim3(HQ / 8, a.batch), 256, 0, s>>>(a, nsplit);
  return hipGetLastError();
}

}  // namespace hca
