// bf16 HCA decode attention for 512-dim heads and 64 query heads per KV head
// on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// What is computed (release blog "ERNIE 5.5 Flash Base", section 2.1, HCA
// paragraph): the new token of each sequence, at position t = L-1, attends
// under one softmax (scale 1/sqrt(d)) to the sequence's complete compressed
// entries (floor(L/128) of them) and to its raw window, read from a ring
// buffer that holds position s in slot s % R.
//
// Design (gfx950): one workgroup of 4 wavefronts x 16 heads per (sequence,
// KV head, key split) streams its key range through LDS (tiles of 32 keys,
// double buffered) and writes partials (m, l in fp32, O/l in bf16) to the
// workspace; a second, fully parallel kernel merges them in split order, so
// the result is deterministic.  Scores use the transposed product S^T = K Q^T and the
// output O^T += V^T P^T as in prefill, with the softmax schedule of
// bf16_tiles.h (no accumulator rescaling).
#include <algorithm>

#include "bf16_tiles.h"

namespace hca {
namespace {

// ---------------------------------------------------------------------------
// Decode tiles: 16 query heads per wavefront on v_mfma_f32_16x16x32_bf16.
// Decode streams each key once from HBM and does 64 flops per byte, far
// below the matrix-core ridge, so it uses the narrower product: a wavefront
// then needs 128 accumulator and 64 query registers instead of 256 and 128.
// Layouts (16x16x32): A lane l = row l%16, k 8(l/16)..+7; B lane l = col
// l%16, k 8(l/16)..+7; D lane l = rows 4(l/16)..+3, col l%16.
// ---------------------------------------------------------------------------
constexpr int DSTEPS16 = D / 32;  // k-steps of the score product
constexpr int CTILES16 = D / 16;  // 16-column tiles of the output

struct Acc16 {
  f32x4 o[CTILES16];  // O^T: lane l holds row l%16, cols 16ct + 4(l/16) + i
  float m, l;
};

// Scores of one 32-key tile land as S^T in two 16x16 outputs: lane l holds
// row l%16 and key slots 4g + i (first output) and 16 + 4g + i (second),
// g = l/16.  P^T as the B operand of the 16x16x32 product needs for lane l
// the 8 keys k = 8g + j; taking j < 4 -> 4g + j and j >= 4 -> 16 + 4g + j-4
// makes P come straight from those accumulators, and the V^T A operand reads
// the same two 4-key runs with two transposed LDS reads.
template <int MODE>
__device__ __forceinline__ bool compute_tile16(const char HCA_LDS* kbuf, const char HCA_LDS* vbuf,
                                               const bf16x8 (&qf)[DSTEPS16], Acc16& st, float sc2,
                                               int lane, int koff, int voff, const RowMask& rm,
                                               int tile, bool masked, bool two_term) {
  constexpr int PF = 2;
  f32x4 s0 = {}, s1 = {};
  bf16x8 kf[2 * PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    kf[2 * k] = lds_k_frag(kbuf + koff + k * 64);
    kf[2 * k + 1] = lds_k_frag(kbuf + koff + 16 * KSTR + k * 64);
  }
#pragma unroll
  for (int k = 0; k < DSTEPS16; ++k) {
    const int r = (k % PF) * 2;
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[r], qf[k], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[r + 1], qf[k], s1, 0, 0, 0);
    if (k + PF < DSTEPS16) {
      kf[r] = lds_k_frag(kbuf + koff + (k + PF) * 64);
      kf[r + 1] = lds_k_frag(kbuf + koff + 16 * KSTR + (k + PF) * 64);
    }
  }
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s0[i];
    x[4 + i] = s1[i];
  }
  if (masked) {
    asm volatile("");  // keep this a branch: most tiles need no mask
    const int kk0 = tile * NT + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      x[i] = rm.valid(kk0 + (i >> 2) * 16 + (i & 3)) ? x[i] : -INFINITY;
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  mx = max_xor32(max_xor16(mx)) * sc2;  // lanes l, l^16, l^32, l^48 share row l%16
  if (MODE == kMaxOnly) {
    st.m = fmaxf(st.m, mx);
    return false;
  }
  bool over = false;
  if (MODE == kLazy) {
    if (st.m == -INFINITY) st.m = mx;
    over = mx > st.m + kHeadroom;
  }
  const float nm = st.m == -INFINITY ? 0.f : -st.m;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sc2, nm));
  u32x4 ua, va = {};
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ua[j] = pack2_bf16(x[2 * j], x[2 * j + 1]);
    ls = sum2_bf16(ua[j], ls);
  }
  if (two_term) {
    asm volatile("");  // a branch, not a select: only short key lists take it
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      va[j] = pack2_bf16(x[2 * j] - bf16_lo(ua[j]), x[2 * j + 1] - bf16_hi(ua[j]));
      ls = sum2_bf16(va[j], ls);
    }
  }
  st.l += ls;
  const bf16x8 pa = __builtin_bit_cast(bf16x8, ua), qa = __builtin_bit_cast(bf16x8, va);
  const int parts = two_term ? 2 : 1;
  for (int part = 0; part < parts; ++part) {
    const bf16x8 bp = part ? qa : pa;
    bf16x8 vf[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) vf[u] = lds_v_frag16(vbuf + voff + u * 32);
#pragma unroll
    for (int ct = 0; ct < CTILES16; ++ct) {
      st.o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[ct % PF], bp, st.o[ct], 0, 0, 0);
      if (ct + PF < CTILES16) vf[ct % PF] = lds_v_frag16(vbuf + voff + (ct + PF) * 32);
    }
  }
  return MODE == kLazy && __any(over);
}

__device__ __forceinline__ void zero_acc16(Acc16& st) {
#pragma unroll
  for (int ct = 0; ct < CTILES16; ++ct) st.o[ct] = f32x4{};
  st.m = -INFINITY;
  st.l = 0.f;
}

template <int MODE>
__device__ __forceinline__ bool tile_pass16(const KeySource& ks, int t_begin, int t_end,
                                            const bf16x8 (&qf)[DSTEPS16], Acc16& st, float sc2,
                                            const RowMask& rm, int wave, int lane,
                                            char HCA_LDS* kv0, char HCA_LDS* kv1, int* flag,
                                            bool two_term) {
  const int g = lane >> 4;
  const int koff = (lane & 15) * KSTR + g * 16;
  const int voff = NT * KSTR + (4 * g + ((lane & 15) >> 2)) * VSTR + 4 * (lane & 3) * 2;
  if (MODE == kLazy && threadIdx.x == 0) flag[0] = flag[1] = 0;
  issue_tile<4, true, true, kStreamed>(ks, t_begin, kv0, kv0 + NT * KSTR, wave, lane);
  wait_vm_all();
  __syncthreads();
  for (int tile = t_begin; tile < t_end; tile += 2) {  // two buffers, unrolled (see tile_pass)
    if (tile + 1 < t_end) issue_tile<4, true, true, kStreamed>(ks, tile + 1, kv1, kv1 + NT * KSTR, wave, lane);
    bool over = compute_tile16<MODE>(kv0, kv0, qf, st, sc2, lane, koff, voff, rm, tile,
                                     tile_needs_mask(tile, rm.nc, rm.nkeys), two_term);
    if (MODE == kLazy && over && lane == 0) flag[0] = 1;
    wait_vm_all();
    __syncthreads();
    if (MODE == kLazy && flag[0]) return true;
    if (tile + 1 >= t_end) break;
    if (tile + 2 < t_end) issue_tile<4, true, true, kStreamed>(ks, tile + 2, kv0, kv0 + NT * KSTR, wave, lane);
    over = compute_tile16<MODE>(kv1, kv1, qf, st, sc2, lane, koff, voff, rm, tile + 1,
                                tile_needs_mask(tile + 1, rm.nc, rm.nkeys), two_term);
    if (MODE == kLazy && over && lane == 0) flag[1] = 1;
    wait_vm_all();
    __syncthreads();
    if (MODE == kLazy && flag[1]) return true;
  }
  return false;
}

__device__ __forceinline__ void attend_tiles16(const KeySource& ks, int t_begin, int t_end,
                                               const bf16x8 (&qf)[DSTEPS16], Acc16& st, float sc2,
                                               const RowMask& rm, int wave, int lane,
                                               char HCA_LDS* kv0, char HCA_LDS* kv1, int* flag) {
  const bool two_term = rm.nkeys <= kTwoTermKeys;
  zero_acc16(st);
  if (!tile_pass16<kLazy>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag,
                          two_term))
    return;
  __syncthreads();
  zero_acc16(st);
  tile_pass16<kMaxOnly>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag, two_term);
  tile_pass16<kFixed>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag, two_term);
}

// ---------------------------------------------------------------------------
// Decode: split kernel grid (max_splits, batch, Hkv), 256 threads (4
// wavefronts x 16 heads), then the merge kernel.
// Workspace: fp32 m and l [B*Hkv][splits][64], then bf16 O [B*Hkv][splits]
// [64][512] normalised by its own l (a convex combination of value rows).
// O / l in bf16 halves the partial traffic (written, then read back by the
// merge); its rounding (<= 2^-9 relative) survives the merge's convex
// combination unchanged, next to the output's own bf16 rounding.
// ---------------------------------------------------------------------------
struct WsLayout {
  float* m;
  float* l;
  bf16* o;
};

__host__ __device__ inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline WsLayout ws_layout(void* ws, int batch, int hkv, int splits) {
  WsLayout w;
  char* p = (char*)ws;
  const size_t units = (size_t)batch * hkv;
  w.m = (float*)p;
  p += round_up(units * splits * G * sizeof(float), 256);
  w.l = (float*)p;
  p += round_up(units * splits * G * sizeof(float), 256);
  w.o = (bf16*)p;
  return w;
}

// Workgroup w runs on XCD w % 8 (round-robin dispatch).  The splits of one
// (sequence, KV head) unit get ids xcd + 8 (split + max_splits g), unit =
// xcd + 8 g: they share an XCD and its L2 (the query rows are fetched from
// HBM once) and are dispatched close together.
__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a, int tps, int max_splits) {
  __shared__ __attribute__((aligned(16))) char kv0_s[NT * KSTR + NT * VSTR];
  __shared__ __attribute__((aligned(16))) char kv1_s[NT * KSTR + NT * VSTR];
  __shared__ int flag_s[2];

  const int wg = (int)blockIdx.x;
  const int split = (wg >> 3) % max_splits;
  const int unit_id = (wg & 7) + 8 * ((wg >> 3) / max_splits);
  if (unit_id >= a.batch * a.hkv) return;
  const int b = unit_id / a.hkv, kvh = unit_id % a.hkv;
  const int L = a.seqlens[b];
  const int t = L - 1;                        // the new token's position
  const int nc = L / kBlock;                  // complete blocks: 128(j+1) <= t+1
  const int nraw = min(a.window, L);
  const int lo = L - nraw;
  const int nkeys = nc + nraw;
  const int ntiles = (nkeys + NT - 1) / NT;
  const int nsplit = (ntiles + tps - 1) / tps;
  if (split >= nsplit) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = wave * 16 + (lane & 15);    // head within the KV group
  const int head = kvh * G + row;

  KeySource ks;
  ks.rstride = a.hkv * D * (int)sizeof(bf16);
  {
    const size_t rs = (size_t)ks.rstride;
    const size_t head_off = (size_t)kvh * D * sizeof(bf16);
    const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
    ks.comp_k = make_rsrc((const char*)a.kc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
    ks.comp_v = make_rsrc((const char*)a.vc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
    ks.raw_k = make_rsrc((const char*)a.kw + (size_t)b * a.ring * rs + head_off, (size_t)a.ring * rs);
    ks.raw_v = make_rsrc((const char*)a.vw + (size_t)b * a.ring * rs + head_off, (size_t)a.ring * rs);
  }
  ks.nc = nc;
  ks.nkeys = nkeys;
  ks.raw0 = lo % a.ring;
  ks.ring = a.ring;

  RowMask rm;
  rm.nc = nc;
  rm.nkeys = nkeys;
  rm.nvis_c = nc;
  rm.r0 = nc;
  rm.r1 = nkeys - 1;

  // Q^T fragments: lane l holds head row l%16, elements 32k + 8(l/16) .. +7
  bf16x8 qf[DSTEPS16];
  const bf16* qrow = (const bf16*)a.q + ((size_t)b * a.hq + head) * D + 8 * (lane >> 4);
#pragma unroll
  for (int k = 0; k < DSTEPS16; ++k) qf[k] = *(const bf16x8*)(qrow + 32 * k);
  Acc16 st;
  const float sc2 = a.scale * kLog2e;
  const int t_begin = split * tps;
  const int t_end = min(ntiles, t_begin + tps);
  attend_tiles16(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, (char HCA_LDS*)kv0_s,
                 (char HCA_LDS*)kv1_s, flag_s);

  // this split's partial result: m, l and O / l
  const WsLayout w = ws_layout(a.ws, a.batch, a.hkv, max_splits);
  const size_t unit = (size_t)b * a.hkv + kvh;
  const size_t prow = (unit * max_splits + split) * G + row;
  float l_tot = st.l + __shfl_xor(st.l, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (lane < 16) {
    w.m[prow] = st.m;
    w.l[prow] = l_tot;
  }
  // O / l of the wave's 16 rows, staged in LDS (the tile buffers are free:
  // the last pass ended with no load in flight and a barrier after its last
  // fragment reads) and stored as whole 1 KiB rows, 16 bytes per lane: the
  // accumulator layout would otherwise store 32-byte pieces of 16 rows per
  // instruction.
  const float inv = 1.f / l_tot;
  char HCA_LDS* stg = (char HCA_LDS*)kv0_s + wave * 16 * KSTR;
  {
    char HCA_LDS* rowp = stg + (lane & 15) * KSTR + 8 * (lane >> 4);
#pragma unroll
    for (int ct = 0; ct < CTILES16; ++ct) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)(st.o[ct][i] * inv);
      *(bf16x4 HCA_LDS*)(rowp + 32 * ct) = v;
    }
  }
  // the wave reads rows its other lanes wrote: order the stores before the loads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  bf16* po = w.o + (prow - (lane & 15)) * D + 8 * lane;  // row wave*16 of this split, columns 8 lane ..
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *(bf16x8*)(po + (size_t)r * D) = *(const bf16x8 HCA_LDS*)(stg + r * KSTR + 16 * lane);
}

// Merge of the split partials: O = sum_s 2^(m_s - M) l_s O_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s, splits taken in order (deterministic).  Splits are
// read a batch at a time with all loads of a batch in flight together; a
// running M rescales what earlier batches added (exact when one batch
// covers all splits).
constexpr int kMergeBatch = 8;

// Merged O (normalised) of head r, columns c .. c+7 of one unit, splits
// read NB at a time (NB = 4 when the unit has at most 4 splits, so that no
// load repeats a split).
template <int NB>
__device__ __forceinline__ void merge_cols8(const WsLayout& w, int unit, int r, int c, int nsplit,
                                            int max_splits, float (&out)[8]) {
  const float* mrow = w.m + (size_t)unit * max_splits * G + r;
  const float* lrow = w.l + (size_t)unit * max_splits * G + r;
  const bf16* orow = w.o + ((size_t)unit * max_splits * G + r) * D + c;
  float M = -INFINITY, den = 0.f, n0[8] = {};
  for (int s0 = 0; s0 < nsplit; s0 += NB) {
    float mv[NB], lv[NB];
    bf16x8 ov[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int sp = min(s0 + j, nsplit - 1);  // repeats of the last split are dropped below
      mv[j] = mrow[(size_t)sp * G];
      lv[j] = lrow[(size_t)sp * G];
      ov[j] = *(const bf16x8*)(orow + (size_t)sp * G * D);
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (s0 + j < nsplit) Mb = fmaxf(Mb, mv[j]);
    if (Mb != M) {  // rescale what earlier batches added
      const float f = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
      den *= f;
#pragma unroll
      for (int i = 0; i < 8; ++i) n0[i] *= f;
      M = Mb;
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (s0 + j >= nsplit) break;
      const float wgt = __builtin_amdgcn_exp2f(mv[j] - M) * lv[j];
      den += wgt;
#pragma unroll
      for (int i = 0; i < 8; ++i) n0[i] = __builtin_fmaf(wgt, (float)ov[j][i], n0[i]);
    }
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = n0[i] * inv;
}

// Merge without epilogue: one workgroup of 4 wavefronts merges 4 heads of
// one (sequence, KV head) unit, wavefront = head, lane l = columns 8l ..
// 8l+7 (16-byte loads and stores).  The merge of unit u runs on XCD u % 8
// like its split workgroups, whose L2 may still hold the partials.
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int tps, int max_splits) {
  const int wg = (int)blockIdx.x;
  const int unit = (wg & 7) + 8 * ((wg >> 3) / (G / 4));  // b * Hkv + kvh
  if (unit >= a.batch * a.hkv) return;
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int r = ((wg >> 3) % (G / 4)) * 4 + (threadIdx.x >> 6);  // head within the KV group
  const int c = (threadIdx.x & 63) * 8;
  const int L = a.seqlens[b];
  const int nkeys = L / kBlock + min(a.window, L);
  const int nsplit = ((nkeys + NT - 1) / NT + tps - 1) / tps;
  const WsLayout w = ws_layout(a.ws, a.batch, a.hkv, max_splits);
  float n[8];
  if (nsplit <= 4)
    merge_cols8<4>(w, unit, r, c, nsplit, max_splits, n);
  else
    merge_cols8<kMergeBatch>(w, unit, r, c, nsplit, max_splits, n);
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)n[i];
  *(bf16x8*)((bf16*)a.o + ((size_t)b * a.hq + kvh * G + r) * D + c) = v;
}

// Merge with the attention epilogue (release blog "ERNIE 5.5 Flash Base",
// section 2.1, last paragraph: per-head output gate and Virtual Head
// Attention, a cross-head low-rank mixing with identity skip):
// y[h] = sigmoid(gate[b, h]) (O[h] + sum_r U[h, r] sum_h' V[h', r] O[h']).
// One workgroup of 512 threads covers all 64 heads of a unit for 64
// columns (the mixing runs across heads); thread t merges head t/8, columns
// 8(t%8) .. +7 (eight lanes read a 128-byte row segment), the merged tile
// goes through LDS, Z = V^T O and U Z are fp32 dot products.  Grid 8 x 8
// column slices x unit groups, XCD-aware like the split kernel.
constexpr int kEpiCols = 64;  // columns per workgroup of the epilogue merge (128-byte row segments)
__global__ __launch_bounds__(512) void decode_merge_epi_kernel(DecodeArgs a, int tps, int max_splits) {
  // rows padded to a multiple of 16 bytes: the tiles are read and written
  // four floats at a time
  __shared__ __attribute__((aligned(16))) float o_s[G][kEpiCols + 4];
  __shared__ __attribute__((aligned(16))) float z_s[32][kEpiCols + 4];
  __shared__ float v_s[G][33];  // V of the unit's KV head, [head][rank]
  __shared__ float u_s[G][33];  // U of the unit's KV head, [head][rank]
  const int wg = (int)blockIdx.x;
  const int unit = (wg & 7) + 8 * ((wg >> 3) / (D / kEpiCols));
  if (unit >= a.batch * a.hkv) return;
  const int slice = (wg >> 3) % (D / kEpiCols);
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int tid = threadIdx.x, hr = tid >> 3, cq = (tid & 7) * 8;
  const int L = a.seqlens[b];
  const int nkeys = L / kBlock + min(a.window, L);
  const int nsplit = ((nkeys + NT - 1) / NT + tps - 1) / tps;
  const WsLayout w = ws_layout(a.ws, a.batch, a.hkv, max_splits);
  const int c0 = kEpiCols * slice + cq;
  // the epilogue's inputs are loaded first, so that their latency overlaps
  // the merge's loads: this thread's share of U and V (G x rank <= 4 each
  // per thread, coalesced) and the gate logit
  const int rank = a.mix_u ? a.mix_rank : 0;
  float uu[4], vv[4];
  if (rank) {
    const float* ug = a.mix_u + (size_t)kvh * G * rank;
    const float* vg = a.mix_v + (size_t)kvh * G * rank;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = tid + 512 * j < G * rank;
      uu[j] = in ? ug[tid + 512 * j] : 0.f;
      vv[j] = in ? vg[tid + 512 * j] : 0.f;
    }
  }
  const float glogit = a.gate ? a.gate[(size_t)b * a.hq + kvh * G + hr] : 0.f;
  float y[8];
  if (nsplit <= 4)
    merge_cols8<4>(w, unit, hr, c0, nsplit, max_splits, y);
  else
    merge_cols8<kMergeBatch>(w, unit, hr, c0, nsplit, max_splits, y);
  if (rank) {
    *(f32x4*)&o_s[hr][cq] = f32x4{y[0], y[1], y[2], y[3]};
    *(f32x4*)&o_s[hr][cq + 4] = f32x4{y[4], y[5], y[6], y[7]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 512 * j;
      if (e < G * rank) {
        v_s[e / rank][e % rank] = vv[j];
        u_s[e / rank][e % rank] = uu[j];
      }
    }
    __syncthreads();
    // Z[rk][c] = sum_h V[h][rk] O[h][c] for 4 columns: two threads (lanes
    // e, e ^ 1) per item, 32 heads each, summed by a lane exchange
    for (int e = tid; e < 2 * rank * (kEpiCols / 4); e += 512) {
      const int item = e >> 1, half = e & 1;
      const int rk = item / (kEpiCols / 4), c = (item % (kEpiCols / 4)) * 4;
      f32x4 z = {};
#pragma unroll 16
      for (int hh = 0; hh < G / 2; ++hh) {
        const int h = 2 * hh + half;
        const float vh = v_s[h][rk];
        const f32x4 oh = *(const f32x4*)&o_s[h][c];
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = fmaf(vh, oh[i], z[i]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] += __shfl_xor(z[i], 1);
      if (!half) *(f32x4*)&z_s[rk][c] = z;
    }
    __syncthreads();
#pragma unroll
    for (int rk = 0; rk < 32; ++rk) {
      if (rk < rank) {
        const float ur = u_s[hr][rk];
        const f32x4 z0 = *(const f32x4*)&z_s[rk][cq], z1 = *(const f32x4*)&z_s[rk][cq + 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = fmaf(ur, z0[i], y[i]);
          y[4 + i] = fmaf(ur, z1[i], y[4 + i]);
        }
      }
    }
  }
  const float gsc = a.gate ? 1.f / (1.f + __expf(-glogit)) : 1.f;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)(y[i] * gsc);
  *(bf16x8*)((bf16*)a.o + ((size_t)b * a.hq + kvh * G + hr) * D + c0) = v;
}

}  // namespace

DecodePlan decode_plan(int batch, int hkv, int max_blocks, int window) {
  // keys of the longest sequence: its entries plus at most min(W, L) raw rows
  const long raw = std::min<long>(window, (long)kBlock * max_blocks + kBlock - 1);
  const int ntiles = (int)((max_blocks + raw + NT - 1) / NT);
  const long units = std::max<long>(1, (long)batch * hkv);
  // aim for about one workgroup per compute unit
  int splits = (int)std::min<long>(ntiles, std::max<long>(1, (256 + units - 1) / units));
  const int tps = (ntiles + splits - 1) / splits;
  splits = (ntiles + tps - 1) / tps;
  return DecodePlan{tps, splits};
}

size_t decode_workspace_bytes_bf16(int batch, int hkv, int max_blocks, int window) {
  const DecodePlan p = decode_plan(batch, hkv, max_blocks, window);
  const size_t units = (size_t)batch * hkv;
  return 2 * round_up(units * p.max_splits * G * sizeof(float), 256) +
         units * p.max_splits * G * D * sizeof(bf16);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const DecodePlan p = decode_plan(a.batch, a.hkv, a.max_blocks, a.window);
  const long groups = ((long)a.batch * a.hkv + 7) / 8;  // units per XCD slot
  decode_bf16_kernel<<<(unsigned)(8 * p.max_splits * groups), 256, 0, s>>>(a, p.tiles_per_split,
                                                                          p.max_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.gate || a.mix_u)
    decode_merge_epi_kernel<<<(unsigned)(8 * (D / kEpiCols) * groups), 512, 0, s>>>(a, p.tiles_per_split, p.max_splits);
  else
    decode_merge_kernel<<<(unsigned)(8 * (G / 4) * groups), 256, 0, s>>>(a, p.tiles_per_split, p.max_splits);
  return hipGetLastError();
}

}  // namespace hca
