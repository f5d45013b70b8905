// Backward of the bf16 HCA prefill (512-dim heads, 64 query heads per KV
// head) on CDNA4 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// What is differentiated (release blog "ERNIE 5.5 Flash Base", section 2.1,
// HCA paragraph; the model trains at long context per the model card): each
// query row attends under one softmax (scale 1/sqrt(d)) to the complete
// compressed entries of its sequence and to its raw window; an entry is the
// softmax(w)-weighted sum of the 128 raw rows of its block, K and V alike.
// For a loss with gradient dO at the output, per query row and visible key j:
//   P_j = exp(scale q.k_j - lse),  dP_j = dO.v_j,  D = dO.O,
//   dS_j = P_j (dP_j - D),
//   dq = scale sum_j dS_j k_j,  dk_j += scale dS_j q,  dv_j += P_j dO,
// the key/value gradients of entry c flow back to its block's raw rows as
// p_i dKc_c, and the pooling logits get dw = p (g - sum p g) with
// g_i = sum_c (dKc_c . K_{128c+i} + dVc_c . V_{128c+i}).
//
// Kernels, in launch order (lse comes from the forward):
//   bwd_dq_kernel   query-major, one position per workgroup (4 waves x 16
//                   heads): recomputes S and dP per 32-key tile, forms dS,
//                   accumulates dQ^T += K^T dS^T; also writes D = dO.O.
//   bwd_dkv_kernel  key-major: a workgroup keeps 32 keys (raw rows, or
//                   compressed entries) in LDS and streams the positions
//                   that see them, 32 heads at a time; raw tiles write
//                   dK, dV rows (fp32), compressed tiles write one partial
//                   per position split (deterministic, no atomics).
//   bwd_pool_kernel per 128-row block: sums an entry's partials, adds
//                   p_i dKc / p_i dVc to the raw-row gradients, rounds them
//                   to bf16 and writes the block's terms of g.
//   bwd_dw_kernel   sums g over all blocks and applies the softmax Jacobian.
#include <algorithm>

#include "bf16_tiles.h"

namespace hca {
namespace {

constexpr float kLn2 = 0.6931471805599453f;
constexpr int BSTR = 1040;           // LDS bytes per staged Q / dO row
constexpr int SSTR = 33;             // fp32 stride of the staged S / dP rows (one per key)
constexpr int DQ_TILES = D / 16;     // 16-column tiles of dQ^T
constexpr int KSTEPS = D / 32;       // k-steps of a 512-long contraction

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposed A (or B) fragment of a 16x16x32 product from row-major bf16
// rows in LDS (row stride `stride` bytes): lane l gets column l%16 of rows
// 4g + j (j < 4) and 16 + 4g + j, g = l/16; `base` already holds the lane
// offset (4g + (l%16)/4) * stride + 8 (l%4) plus the column tile.
__device__ __forceinline__ bf16x8 lds_tr_frag(const char HCA_LDS* base, int stride) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)base);
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)(base + 16 * stride));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Key rows of one sequence and KV head as buffer resources (K and V raw
// rows, compressed entries).
__device__ __forceinline__ void seq_sources(const BackwardArgs& a, int b, int kvh, int start, int len,
                                            KeySource& ks) {
  ks.rstride = a.hkv * D * (int)sizeof(bf16);
  const size_t rs = (size_t)ks.rstride;
  const size_t head_off = (size_t)kvh * D * sizeof(bf16);
  const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
  ks.comp_k = make_rsrc((const char*)a.kc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
  ks.comp_v = make_rsrc((const char*)a.vc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
  ks.raw_k = make_rsrc((const char*)a.k + (size_t)start * rs + head_off, (size_t)len * rs);
  ks.raw_v = make_rsrc((const char*)a.v + (size_t)start * rs + head_off, (size_t)len * rs);
  ks.ring = 0;
}

// ---------------------------------------------------------------------------
// dQ: grid (max_seqlen, batch, Hkv), 256 threads; wave w owns heads
// 16w .. 16w+15 of the KV group (row r = l%16).  Per 32-key tile (double
// buffered in LDS like decode):
//   S^T, dP^T [32 keys x 16 heads] = K Q^T, V dO^T   (2 x 16 k-steps each)
//   dS = P (dP - D) with P = exp2(S sc2 - lse2), keys past the list zeroed
//   dQ^T [512 x 16] += K^T dS^T: B = dS^T straight from the accumulators
//     (lane l: head l%16, keys 4g+i and 16+4g+i, the k-slot order of the
//     transposed K reads), A = K^T by transposed LDS reads.
// ---------------------------------------------------------------------------
struct DqState {
  f32x4 acc[DQ_TILES];  // dQ^T: lane l holds head l%16, d = 16 ct + 4 g + i
};

__device__ __forceinline__ void dq_tile(const char HCA_LDS* kbuf, const char HCA_LDS* vbuf,
                                        const bf16x8 (&qf)[KSTEPS], const bf16x8 (&df)[KSTEPS], DqState& st,
                                        float sc2, float lse2, float dd, int lane, int tile, int nkeys) {
  const int g = lane >> 4, r = lane & 15;
  f32x4 s0 = {}, s1 = {}, p0 = {}, p1 = {};
  const char HCA_LDS* ka = kbuf + r * KSTR + g * 16;
  const char HCA_LDS* va = vbuf + r * VSTR + g * 16;
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) {
    const bf16x8 k0 = lds_k_frag(ka + k * 64), k1 = lds_k_frag(ka + 16 * KSTR + k * 64);
    const bf16x8 v0 = lds_k_frag(va + k * 64), v1 = lds_k_frag(va + 16 * VSTR + k * 64);
    s0 = mfma16(k0, qf[k], s0);
    s1 = mfma16(k1, qf[k], s1);
    p0 = mfma16(v0, df[k], p0);
    p1 = mfma16(v1, df[k], p1);
  }
  bf16x8 bds;
  const int kk0 = tile * NT + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pa = kk0 + i < nkeys ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], sc2, -lse2)) : 0.f;
    const float pb = kk0 + 16 + i < nkeys ? __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], sc2, -lse2)) : 0.f;
    bds[i] = (bf16)(pa * (p0[i] - dd));
    bds[4 + i] = (bf16)(pb * (p1[i] - dd));
  }
  const char HCA_LDS* kt = kbuf + (4 * g + (r >> 2)) * KSTR + 8 * (lane & 3);
#pragma unroll
  for (int ct = 0; ct < DQ_TILES; ++ct) st.acc[ct] = mfma16(lds_tr_frag(kt + 32 * ct, KSTR), bds, st.acc[ct]);
}

__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BackwardArgs a) {
  __shared__ __attribute__((aligned(16))) char kv0_s[NT * KSTR + NT * VSTR];
  __shared__ __attribute__((aligned(16))) char kv1_s[NT * KSTR + NT * VSTR];
  const int t = blockIdx.x, b = blockIdx.y, kvh = blockIdx.z;
  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;
  if (t >= len) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;
  const int head = kvh * G + wave * 16 + (lane & 15);
  const size_t tok = (size_t)start + t;

  KeySource ks;
  seq_sources(a, b, kvh, start, len, ks);
  const int nc = (t + 1) / kBlock;
  const int lo = max(0, t - a.window + 1);
  ks.nc = nc;
  ks.nkeys = nc + (t - lo + 1);
  ks.raw0 = lo;
  const int ntiles = (ks.nkeys + NT - 1) / NT;
  char HCA_LDS* kv0 = (char HCA_LDS*)kv0_s;
  char HCA_LDS* kv1 = (char HCA_LDS*)kv1_s;
  issue_tile<4>(ks, 0, kv0, kv0 + NT * KSTR, wave, lane);

  // Q^T and dO^T fragments (lane l: head l%16, d = 32k + 8g .. +7), and
  // D = dO . O of the row
  const size_t roff = (tok * a.hq + head) * D + 8 * g;
  const bf16* qrow = (const bf16*)a.q + roff;
  const bf16* drow = (const bf16*)a.dout + roff;
  const bf16* orow = (const bf16*)a.o + roff;
  bf16x8 qf[KSTEPS], df[KSTEPS];
  float dd = 0.f;
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) {
    qf[k] = *(const bf16x8*)(qrow + 32 * k);
    df[k] = *(const bf16x8*)(drow + 32 * k);
    const bf16x8 ov = *(const bf16x8*)(orow + 32 * k);
#pragma unroll
    for (int i = 0; i < 8; ++i) dd = __builtin_fmaf((float)df[k][i], (float)ov[i], dd);
  }
  dd += __shfl_xor(dd, 16);
  dd += __shfl_xor(dd, 32);
  if (lane < 16) a.delta[tok * a.hq + head] = dd;
  const float lse2 = a.lse[tok * a.hq + head] * kLog2e;
  const float sc2 = a.scale * kLog2e;

  DqState st;
#pragma unroll
  for (int ct = 0; ct < DQ_TILES; ++ct) st.acc[ct] = f32x4{};
  wait_vm_all();
  __syncthreads();
  for (int tile = 0; tile < ntiles; tile += 2) {
    if (tile + 1 < ntiles) issue_tile<4>(ks, tile + 1, kv1, kv1 + NT * KSTR, wave, lane);
    dq_tile(kv0, kv0 + NT * KSTR, qf, df, st, sc2, lse2, dd, lane, tile, ks.nkeys);
    wait_vm_all();
    __syncthreads();
    if (tile + 1 >= ntiles) break;
    if (tile + 2 < ntiles) issue_tile<4>(ks, tile + 2, kv0, kv0 + NT * KSTR, wave, lane);
    dq_tile(kv1, kv1 + NT * KSTR, qf, df, st, sc2, lse2, dd, lane, tile + 1, ks.nkeys);
    wait_vm_all();
    __syncthreads();
  }
  bf16* out = (bf16*)a.dq + (tok * a.hq + head) * D + 4 * g;
#pragma unroll
  for (int ct = 0; ct < DQ_TILES; ++ct) {
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)(st.acc[ct][i] * a.scale);
    *(bf16x4*)(out + 16 * ct) = v;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: grid (raw_tiles + comp_tiles * nsplit, batch, Hkv), 256 threads.
// Workgroup x < raw_tiles owns raw rows 32x .. 32x+31 of the sequence and
// the positions that see them (x*32 .. x*32+31+W-1); the others own
// compressed entries 32c .. 32c+31 (c = (x - raw_tiles) / nsplit) and split
// s of the positions that see entry 32c (those from 128 (32c+1) - 1 on, in
// runs of `pch`).  Per position and half of the 64 heads (a "step"):
//   stage the 32 Q rows and 32 dO rows in LDS;
//   waves 0, 1: S^T [32 keys x 16 rows] = K Q^T; waves 2, 3: dP^T = V dO^T
//     (rows 16 (w&1) ..); both to LDS as fp32;
//   all threads: P = exp2(S sc2 - lse2) on visible (key, position) pairs,
//     dS = P (dP - D), both as bf16 A operands [key][rows in k-slot order];
//   wave w, columns 128w .. 128w+127: dV += P^T dO, dK += dS^T Q
//     (B = the staged rows read transposed).
// ---------------------------------------------------------------------------
struct DkvLds {
  char HCA_LDS* kt;   // 32 K rows (KSTR)
  char HCA_LDS* vt;   // 32 V rows (VSTR)
  char HCA_LDS* qs;   // 32 staged Q rows (BSTR)
  char HCA_LDS* ds;   // 32 staged dO rows (BSTR)
  float HCA_LDS* sx;  // S  [32 keys][SSTR]
  float HCA_LDS* px;  // dP [32 keys][SSTR]
  char HCA_LDS* pa;   // P^T  bf16 [32 keys][32 rows, k-slot order]
  char HCA_LDS* sa;   // dS^T bf16 [32 keys][32 rows, k-slot order]
  float HCA_LDS* rs;  // lse2 [32], D [32] of the staged rows
};

// Byte offset of (key, row) in the P^T / dS^T operand buffers: lane l of an
// A fragment reads key 16m + l%16, rows 4g + j and 16 + 4g + j (g = l/16),
// the k-slot order of the transposed reads of the staged rows.
__device__ __forceinline__ int kslot_off(int key, int row) {
  return key * 64 + ((row & 15) >> 2) * 16 + ((row >> 4) * 4 + (row & 3)) * 2;
}

__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(BackwardArgs a, int raw_tiles, int nsplit, int pch) {
  __shared__ __attribute__((aligned(16))) char kt_s[NT * KSTR];
  __shared__ __attribute__((aligned(16))) char vt_s[NT * VSTR];
  __shared__ __attribute__((aligned(16))) char qs_s[32 * BSTR];
  __shared__ __attribute__((aligned(16))) char ds_s[32 * BSTR];
  __shared__ __attribute__((aligned(16))) float sx_s[NT * SSTR];
  __shared__ __attribute__((aligned(16))) float px_s[NT * SSTR];
  __shared__ __attribute__((aligned(16))) char pa_s[NT * 64];
  __shared__ __attribute__((aligned(16))) char sa_s[NT * 64];
  __shared__ __attribute__((aligned(16))) float rs_s[64];

  const int b = blockIdx.y, kvh = blockIdx.z;
  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;
  const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
  const int x = blockIdx.x;
  const bool comp = x >= raw_tiles;
  int key0, t_begin, t_end, ctile = 0, split = 0;
  if (!comp) {
    key0 = x * NT;
    if (key0 >= len) return;
    t_begin = key0;
    t_end = min(len, key0 + NT - 1 + a.window);
  } else {
    ctile = (x - raw_tiles) / nsplit;
    split = (x - raw_tiles) % nsplit;
    key0 = ctile * NT;
    if (key0 >= nb) return;
    const int first = kBlock * (key0 + 1) - 1;  // first position that sees entry key0
    t_begin = first + split * pch;
    if (t_begin >= len) return;
    t_end = min(len, t_begin + pch);
  }
  const int nkey = min(NT, (comp ? nb : len) - key0);  // keys of the tile that exist

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  DkvLds L;
  L.kt = (char HCA_LDS*)kt_s;
  L.vt = (char HCA_LDS*)vt_s;
  L.qs = (char HCA_LDS*)qs_s;
  L.ds = (char HCA_LDS*)ds_s;
  L.sx = (float HCA_LDS*)sx_s;
  L.px = (float HCA_LDS*)px_s;
  L.pa = (char HCA_LDS*)pa_s;
  L.sa = (char HCA_LDS*)sa_s;
  L.rs = (float HCA_LDS*)rs_s;

  // the 32 keys: slots of a key list that is all compressed or all raw
  KeySource ks;
  seq_sources(a, b, kvh, start, len, ks);
  ks.nc = comp ? nb : 0;
  ks.nkeys = comp ? nb : len;
  ks.raw0 = 0;
  issue_tile<4>(ks, key0 / NT, L.kt, L.vt, wave, lane);

  const float sc2 = a.scale * kLog2e;
  f32x4 acc_v[2][8], acc_k[2][8];  // [key half m][16-column tile u]: keys 16m + 4g + i, d = 128w + 16u + l%16
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc_v[m][u] = acc_k[m][u] = f32x4{};

  const size_t rstride = (size_t)a.hq * D * sizeof(bf16);
  for (int t = t_begin; t < t_end; ++t) {
    const size_t tok = (size_t)start + t;
    for (int hh = 0; hh < 2; ++hh) {
      // stage the 32 Q and dO rows (heads 32hh .. of the group) of position t
      {
        const size_t off = tok * rstride + (size_t)(kvh * G + 32 * hh) * D * sizeof(bf16);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)a.q + off, 32 * D * sizeof(bf16));
        const __amdgpu_buffer_rsrc_t rd = make_rsrc((const char*)a.dout + off, 32 * D * sizeof(bf16));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = wave * 8 + i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (void HCA_LDS*)(L.qs + row * BSTR), 16,
                                                   row * D * (int)sizeof(bf16) + lane * 16, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (void HCA_LDS*)(L.ds + row * BSTR), 16,
                                                   row * D * (int)sizeof(bf16) + lane * 16, 0, 0, 0);
        }
        if (threadIdx.x < 32) {
          const size_t ri = tok * a.hq + kvh * G + 32 * hh + threadIdx.x;
          L.rs[threadIdx.x] = a.lse[ri] * kLog2e;
          L.rs[32 + threadIdx.x] = a.delta[ri];
        }
      }
      wait_vm_all();
      __syncthreads();
      // S^T (waves 0, 1) or dP^T (waves 2, 3) of rows 16 (w & 1) .. +15
      {
        const bool is_dp = wave >= 2;
        const int rh = wave & 1;
        const char HCA_LDS* A = (is_dp ? L.vt : L.kt) + r * (is_dp ? VSTR : KSTR) + g * 16;
        const int astr16 = 16 * (is_dp ? VSTR : KSTR);
        const char HCA_LDS* B = (is_dp ? L.ds : L.qs) + (16 * rh + r) * BSTR + g * 16;
        f32x4 c0 = {}, c1 = {};
#pragma unroll
        for (int k = 0; k < KSTEPS; ++k) {
          const bf16x8 bq = lds_k_frag(B + k * 64);
          c0 = mfma16(lds_k_frag(A + k * 64), bq, c0);
          c1 = mfma16(lds_k_frag(A + astr16 + k * 64), bq, c1);
        }
        float HCA_LDS* dst = is_dp ? L.px : L.sx;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dst[(4 * g + i) * SSTR + 16 * rh + r] = c0[i];
          dst[(16 + 4 * g + i) * SSTR + 16 * rh + r] = c1[i];
        }
      }
      __syncthreads();
      // P and dS of the 32 x 32 (key, row) pairs, 4 per thread
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = threadIdx.x * 4 + u;
        const int key = e >> 5, row = e & 31;
        const int kk = key0 + key;
        const bool vis = key < nkey && (comp ? kBlock * (kk + 1) <= t + 1 : (kk <= t && t - kk < a.window));
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(L.sx[key * SSTR + row], sc2, -L.rs[row])) : 0.f;
        const float dsv = p * (L.px[key * SSTR + row] - L.rs[32 + row]);
        const int o = kslot_off(key, row);
        *(bf16 HCA_LDS*)(L.pa + o) = (bf16)p;
        *(bf16 HCA_LDS*)(L.sa + o) = (bf16)dsv;
      }
      __syncthreads();
      // dV += P^T dO, dK += dS^T Q over the wave's 128 columns
      {
        const int tro = (4 * g + (r >> 2)) * BSTR + 8 * (lane & 3) + wave * 256;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 ap = *(const bf16x8 HCA_LDS*)(L.pa + (16 * m + r) * 64 + g * 16);
          const bf16x8 as = *(const bf16x8 HCA_LDS*)(L.sa + (16 * m + r) * 64 + g * 16);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            acc_v[m][u] = mfma16(ap, lds_tr_frag(L.ds + tro + 32 * u, BSTR), acc_v[m][u]);
            acc_k[m][u] = mfma16(as, lds_tr_frag(L.qs + tro + 32 * u, BSTR), acc_k[m][u]);
          }
        }
      }
      __syncthreads();
    }
  }

  // results: raw rows to the fp32 row gradients, compressed entries to this
  // split's partial
  float* dst_k;
  float* dst_v;
  size_t rstr;  // floats between consecutive keys
  if (!comp) {
    const size_t base = ((size_t)start + key0) * a.hkv + kvh;
    dst_k = a.dk_rows + base * D;
    dst_v = a.dv_rows + base * D;
    rstr = (size_t)a.hkv * D;
  } else {
    const size_t slot = ((((size_t)b * a.hkv + kvh) * a.comp_tiles + ctile) * nsplit + split) * NT;
    dst_k = a.part_k + slot * D;
    dst_v = a.part_v + slot * D;
    rstr = D;
  }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 16 * m + 4 * g + i;
      if (key >= nkey) continue;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int col = wave * 128 + 16 * u + r;
        dst_k[key * rstr + col] = acc_k[m][u][i] * a.scale;
        dst_v[key * rstr + col] = acc_v[m][u][i];
      }
    }
}

// ---------------------------------------------------------------------------
// Pooling backward: grid (ceil(max_seqlen / 128), batch, Hkv), 256 threads.
// Block j of a sequence: when complete, dKc / dVc of entry j = the sum of
// its tile's partials over the splits that exist for this sequence; every
// row i of the block gets dK = dK_rows + p_i dKc (rounded to bf16), dV
// likewise, and g_i = dKc . K_i + dVc . V_i is stored for the dw kernel.
// A trailing partial block only rounds its rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pool_kernel(BackwardArgs a, int nsplit, int pch) {
  __shared__ float dkc_s[D];
  __shared__ float dvc_s[D];
  __shared__ float p_s[kBlock];
  const int j = blockIdx.x, b = blockIdx.y, kvh = blockIdx.z;
  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;
  if (j * kBlock >= len) return;
  const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
  const bool full = j < nb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (full) {
    // p = softmax(w_kvh), one wave
    if (wave == 0) {
      const float w0 = a.w[kvh * kBlock + lane], w1 = a.w[kvh * kBlock + 64 + lane];
      float mx = fmaxf(w0, w1);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float e0 = __expf(w0 - mx), e1 = __expf(w1 - mx);
      float s = e0 + e1;
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
      p_s[lane] = e0 / s;
      p_s[64 + lane] = e1 / s;
    }
    const int ctile = j / NT, kk = j % NT;
    const int first = kBlock * (ctile * NT + 1) - 1;
    const int ns = (len - first + pch - 1) / pch;
    const size_t slot0 = (((size_t)b * a.hkv + kvh) * a.comp_tiles + ctile) * nsplit;
    for (int c = threadIdx.x; c < D; c += 256) {
      float sk = 0.f, sv = 0.f;
      for (int s = 0; s < ns; ++s) {
        const size_t o = ((slot0 + s) * NT + kk) * D + c;
        sk += a.part_k[o];
        sv += a.part_v[o];
      }
      dkc_s[c] = sk;
      dvc_s[c] = sv;
    }
  }
  __syncthreads();
  // rows: wave w takes rows w, w+4, ...; lane l columns 8l .. 8l+7
  const int rows = min(kBlock, len - j * kBlock);
  for (int i = wave; i < rows; i += 4) {
    const size_t row = ((size_t)start + j * kBlock + i) * a.hkv + kvh;
    const float* rk = a.dk_rows + row * D + 8 * lane;
    const float* rv = a.dv_rows + row * D + 8 * lane;
    bf16x8 ok, ov;
    float gi = 0.f;
    const float pi = full ? p_s[i] : 0.f;
    const bf16x8 kx = *(const bf16x8*)((const bf16*)a.k + row * D + 8 * lane);
    const bf16x8 vx = *(const bf16x8*)((const bf16*)a.v + row * D + 8 * lane);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float ck = full ? dkc_s[8 * lane + e] : 0.f, cv = full ? dvc_s[8 * lane + e] : 0.f;
      ok[e] = (bf16)(rk[e] + pi * ck);
      ov[e] = (bf16)(rv[e] + pi * cv);
      gi = __builtin_fmaf(ck, (float)kx[e], __builtin_fmaf(cv, (float)vx[e], gi));
    }
    *(bf16x8*)((bf16*)a.dk + row * D + 8 * lane) = ok;
    *(bf16x8*)((bf16*)a.dv + row * D + 8 * lane) = ov;
    if (full) {
      for (int o = 32; o > 0; o >>= 1) gi += __shfl_xor(gi, o);
      if (lane == 0) a.gbuf[(((size_t)a.cu_blocks[b] + j) * a.hkv + kvh) * kBlock + i] = gi;
    }
  }
}

// dw: one workgroup of 128 threads per KV head: g_i summed over every
// complete block, then dw = p (g - sum_k p_k g_k).
__global__ __launch_bounds__(128) void bwd_dw_kernel(BackwardArgs a) {
  __shared__ float red[2][2];
  const int kvh = blockIdx.x, i = threadIdx.x, lane = i & 63, wave = i >> 6;
  float gs = 0.f;
  for (int e = 0; e < a.total_blocks; ++e) gs += a.gbuf[((size_t)e * a.hkv + kvh) * kBlock + i];
  const float wi = a.w[kvh * kBlock + i];
  float mx = wi;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  mx = fmaxf(red[0][0], red[0][1]);
  const float ei = __expf(wi - mx);
  float s = ei, sg = ei * gs;
  for (int o = 32; o > 0; o >>= 1) {
    s += __shfl_xor(s, o);
    sg += __shfl_xor(sg, o);
  }
  __syncthreads();
  if (lane == 0) {
    red[0][wave] = s;
    red[1][wave] = sg;
  }
  __syncthreads();
  const float tot = red[0][0] + red[0][1];
  const float pg = (red[1][0] + red[1][1]) / tot;  // sum_k p_k g_k
  a.dw[kvh * kBlock + i] = ei / tot * (gs - pg);
}

}  // namespace

BackwardPlan backward_plan(int batch, int hkv, int max_seqlen, int window) {
  BackwardPlan p;
  const int max_blocks = max_seqlen / kBlock;
  p.raw_tiles = (max_seqlen + NT - 1) / NT;
  p.comp_tiles = (max_blocks + NT - 1) / NT;
  p.pch = std::max(64, (max_seqlen + 255) / 256);
  p.nsplit = std::max(1, (max_seqlen + p.pch - 1) / p.pch);
  (void)batch;
  (void)hkv;
  (void)window;
  return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t backward_workspace_bytes(int batch, int hq, int hkv, int total_tokens, int total_blocks, int max_seqlen,
                                int window) {
  const BackwardPlan p = backward_plan(batch, hkv, max_seqlen, window);
  size_t n = 0;
  n += align256((size_t)total_tokens * hq * sizeof(float));                          // delta
  n += 2 * align256((size_t)total_tokens * hkv * D * sizeof(float));                 // dk_rows, dv_rows
  n += 2 * align256((size_t)batch * hkv * p.comp_tiles * p.nsplit * NT * D * sizeof(float));  // partials
  n += align256((size_t)std::max(total_blocks, 1) * hkv * kBlock * sizeof(float));  // g
  return n;
}

hipError_t launch_backward_bf16(BackwardArgs a, hipStream_t s) {
  const BackwardPlan p = backward_plan(a.batch, a.hkv, a.max_seqlen, a.window);
  a.comp_tiles = p.comp_tiles;
  char* w = (char*)a.ws;
  a.delta = (float*)w;
  w += align256((size_t)a.total_tokens * a.hq * sizeof(float));
  a.dk_rows = (float*)w;
  w += align256((size_t)a.total_tokens * a.hkv * D * sizeof(float));
  a.dv_rows = (float*)w;
  w += align256((size_t)a.total_tokens * a.hkv * D * sizeof(float));
  const size_t part = align256((size_t)a.batch * a.hkv * p.comp_tiles * p.nsplit * NT * D * sizeof(float));
  a.part_k = (float*)w;
  w += part;
  a.part_v = (float*)w;
  w += part;
  a.gbuf = (float*)w;

  if (a.batch > 0 && a.max_seqlen > 0) {
    bwd_dq_kernel<<<dim3(a.max_seqlen, a.batch, a.hkv), 256, 0, s>>>(a);
    const int items = p.raw_tiles + p.comp_tiles * p.nsplit;
    bwd_dkv_kernel<<<dim3(items, a.batch, a.hkv), 256, 0, s>>>(a, p.raw_tiles, p.nsplit, p.pch);
    bwd_pool_kernel<<<dim3((a.max_seqlen + kBlock - 1) / kBlock, a.batch, a.hkv), 256, 0, s>>>(a, p.nsplit, p.pch);
  }
  bwd_dw_kernel<<<a.hkv, 128, 0, s>>>(a);  // no complete block: g = 0, dw = 0
  return hipGetLastError();
}

}  // namespace hca
