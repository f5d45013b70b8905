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
#include <type_traits>

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
  // K and V row fragments one k-step ahead (a deeper prefetch spills)
  bf16x8 f[2][4];
  f[0][0] = lds_k_frag(ka);
  f[0][1] = lds_k_frag(ka + 16 * KSTR);
  f[0][2] = lds_k_frag(va);
  f[0][3] = lds_k_frag(va + 16 * VSTR);
#pragma unroll
  for (int k = 0; k < KSTEPS; ++k) {
    const int c = k & 1, n = c ^ 1;
    if (k + 1 < KSTEPS) {
      f[n][0] = lds_k_frag(ka + (k + 1) * 64);
      f[n][1] = lds_k_frag(ka + 16 * KSTR + (k + 1) * 64);
      f[n][2] = lds_k_frag(va + (k + 1) * 64);
      f[n][3] = lds_k_frag(va + 16 * VSTR + (k + 1) * 64);
    }
    s0 = mfma16(f[c][0], qf[k], s0);
    s1 = mfma16(f[c][1], qf[k], s1);
    p0 = mfma16(f[c][2], df[k], p0);
    p1 = mfma16(f[c][3], df[k], p1);
    __builtin_amdgcn_sched_barrier(0);
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
  bf16x8 a[2];
  a[0] = lds_tr_frag(kt, KSTR);
#pragma unroll
  for (int ct = 0; ct < DQ_TILES; ++ct) {
    if (ct + 1 < DQ_TILES) a[(ct + 1) & 1] = lds_tr_frag(kt + 32 * (ct + 1), KSTR);
    st.acc[ct] = mfma16(a[ct & 1], bds, st.acc[ct]);
    __builtin_amdgcn_sched_barrier(0);
  }
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
  // One tile per iteration with the buffers chosen at run time: a loop
  // unrolled by two (one copy per buffer) made the register allocator keep
  // both copies' values, spill the Q and dO fragments, and reload them
  // behind waits that also waited for the next tile's loads.
#pragma unroll 1
  for (int tile = 0; tile < ntiles; ++tile) {
    char HCA_LDS* cur = (tile & 1) ? kv1 : kv0;
    char HCA_LDS* nxt = (tile & 1) ? kv0 : kv1;
    if (tile + 1 < ntiles) issue_tile<4>(ks, tile + 1, nxt, nxt + NT * KSTR, wave, lane);
    dq_tile(cur, cur + NT * KSTR, qf, df, st, sc2, lse2, dd, lane, tile, ks.nkeys);
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
// dK, dV: grid (items, batch, Hkv), 256 threads.  An item is a tile of 64
// keys and a run of the positions that see them: raw tiles (rows 64x ..
// 64x+63 of the sequence; positions 64x .. 64x+63+W-1, in nsr runs of prr)
// first, then compressed tiles (entries 64c .. 64c+63; positions from
// 128 (64c+1) - 1 on, in nsc runs of pch).  Every item writes its own fp32
// partial [64 keys][d] for K and V; bwd_pool_kernel sums them in run order
// (deterministic).
//
// Wave w owns keys 16w .. 16w+15 of the tile and keeps K^T and V^T of them
// in registers (the B operands: lane l = key l%16, d = 32k + 8g .. +7).  A
// "step" is one position and 32 of its heads (rows), staged in LDS (Q and
// dO rows, lse and D; double buffered, filled by direct buffer->LDS loads
// during the previous step):
//   S = Q K^T, dP = dO V^T   [32 rows x 16 keys]: A = staged rows
//   P = exp2(S sc2 - lse2) on visible (row, key) pairs, dS = P (dP - D):
//     in the accumulator layout lane l holds key l%16 and rows 4g + i,
//     16 + 4g + i, which is the A layout of P^T / dS^T with the rows in the
//     k-slot order of the transposed reads below - no exchange needed;
//   dV += P^T dO, dK += dS^T Q   [16 keys x 512]: B = staged rows read
//     transposed; the accumulators (2 x 128 registers) are pinned to AGPRs.
// ---------------------------------------------------------------------------
constexpr int KT = 64;              // keys per item
constexpr int QSTAGE = 32 * BSTR;   // one staged half position of Q (or dO)

__device__ __forceinline__ void stage_rows(const BackwardArgs& a, size_t tok, int kvh, int hh,
                                           char HCA_LDS* buf, float HCA_LDS* rs, int wave, int lane) {
  const size_t row0 = tok * a.hq + kvh * G + 32 * hh;  // first of the 32 rows
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const bf16*)a.q + row0 * D, 32 * D * sizeof(bf16));
  const __amdgpu_buffer_rsrc_t rd = make_rsrc((const bf16*)a.dout + row0 * D, 32 * D * sizeof(bf16));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = wave * 8 + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (void HCA_LDS*)(buf + row * BSTR), 16,
                                             row * D * (int)sizeof(bf16) + lane * 16, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (void HCA_LDS*)(buf + QSTAGE + row * BSTR), 16,
                                             row * D * (int)sizeof(bf16) + lane * 16, 0, 0, 0);
  }
  if (wave == 0) {  // lse and D of the 32 rows: lanes 32.. read past the range (zeros)
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + row0, 32 * sizeof(float));
    const __amdgpu_buffer_rsrc_t rdl = make_rsrc(a.delta + row0, 32 * sizeof(float));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (void HCA_LDS*)rs, 4, lane * 4, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rdl, (void HCA_LDS*)(rs + 64), 4, lane * 4, 0, 0, 0);
  }
}

__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(BackwardArgs a, BackwardPlan pl) {
  // two staging buffers as distinct arrays: each step names its buffers at
  // compile time, so the compiler can tell that a step's LDS reads do not
  // touch the rows that the next step's direct loads are writing (with one
  // array indexed at run time it made every step wait for those loads)
  __shared__ __attribute__((aligned(16))) char st0_s[2 * QSTAGE];
  __shared__ __attribute__((aligned(16))) char st1_s[2 * QSTAGE];
  __shared__ __attribute__((aligned(16))) float rs0_s[128];
  __shared__ __attribute__((aligned(16))) float rs1_s[128];

  const int b = blockIdx.y, kvh = blockIdx.z;
  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;
  const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
  const int x = blockIdx.x;  // the item
  const int raw_items = pl.raw_tiles * pl.nsr;
  const bool comp = x >= raw_items;
  int key0, t_begin, t_end;
  if (!comp) {
    key0 = (x / pl.nsr) * KT;
    if (key0 >= len) return;
    const int t_last = min(len, key0 + KT - 1 + a.window);  // end of the positions that see the tile
    t_begin = key0 + (x % pl.nsr) * pl.prr;
    if (t_begin >= t_last) return;
    t_end = min(t_last, t_begin + pl.prr);
  } else {
    const int y = x - raw_items;
    key0 = (y / pl.nsc) * KT;
    if (key0 >= nb) return;
    t_begin = kBlock * (key0 + 1) - 1 + (y % pl.nsc) * pl.pch;
    if (t_begin >= len) return;
    t_end = min(len, t_begin + pl.pch);
  }
  const int nkey = min(KT, (comp ? nb : len) - key0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int kl = 16 * wave + r;      // the lane's key within the tile
  const int kk = key0 + kl;           // ... within the sequence (entry or raw position)

  // K^T and V^T fragments of the lane's key (past the end: the last key,
  // masked below)
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const size_t row = comp ? (size_t)(a.cu_blocks[b] + min(kk, nb - 1)) : (size_t)start + min(kk, len - 1);
    const bf16* kr = (const bf16*)(comp ? a.kc : a.k) + (row * a.hkv + kvh) * D + 8 * g;
    const bf16* vr = (const bf16*)(comp ? a.vc : a.v) + (row * a.hkv + kvh) * D + 8 * g;
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      kf[k] = *(const bf16x8*)(kr + 32 * k);
      vf[k] = *(const bf16x8*)(vr + 32 * k);
    }
  }
  f32x4 accv[D / 16], acck[D / 16];  // lane l: keys 16w + 4g + i, d = 16u + l%16
#pragma unroll
  for (int u = 0; u < D / 16; ++u) accv[u] = acck[u] = f32x4{};

  const float sc2 = a.scale * kLog2e;
  const int nsteps = 2 * (t_end - t_begin);
  char HCA_LDS* const st0 = (char HCA_LDS*)st0_s;
  char HCA_LDS* const st1 = (char HCA_LDS*)st1_s;
  float HCA_LDS* const rs0 = (float HCA_LDS*)rs0_s;
  float HCA_LDS* const rs1 = (float HCA_LDS*)rs1_s;
  stage_rows(a, (size_t)start + t_begin, kvh, 0, st0, rs0, wave, lane);
  wait_vm_all();
  __syncthreads();
  const int tro = (4 * g + (r >> 2)) * BSTR + 8 * (lane & 3);
  // step i: position t_begin + i/2, head half i%2, staged in buffer i%2
  auto step = [&](int i, auto parity) {
    constexpr int P = decltype(parity)::value;
    const int t = t_begin + (i >> 1);
    if (i + 1 < nsteps)
      stage_rows(a, (size_t)start + t_begin + ((i + 1) >> 1), kvh, 1 - P, P ? st0 : st1, P ? rs0 : rs1, wave, lane);
    const char HCA_LDS* qs = P ? st1 : st0;
    const char HCA_LDS* ds = qs + QSTAGE;
    const float HCA_LDS* rs = P ? rs1 : rs0;
    // S, dP of the 32 rows and the wave's 16 keys
    f32x4 sx[2] = {}, px[2] = {};
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int o = (16 * m + r) * BSTR + 64 * k + 16 * g;
        sx[m] = mfma16(lds_k_frag(qs + o), kf[k], sx[m]);
        px[m] = mfma16(lds_k_frag(ds + o), vf[k], px[m]);
      }
    }
    const bool vis = kl < nkey && (comp ? kBlock * (kk + 1) <= t + 1 : (kk <= t && t - kk < a.window));
    bf16x8 ap, as;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = 16 * m + 4 * g + j;
        const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sx[m][j], sc2, -rs[row] * kLog2e)) : 0.f;
        ap[4 * m + j] = (bf16)p;
        as[4 * m + j] = (bf16)(p * (px[m][j] - rs[64 + row]));
      }
    bf16x8 bo[2], bq[2];
    bo[0] = lds_tr_frag(ds + tro, BSTR);
    bq[0] = lds_tr_frag(qs + tro, BSTR);
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      if (u + 1 < D / 16) {
        bo[(u + 1) & 1] = lds_tr_frag(ds + tro + 32 * (u + 1), BSTR);
        bq[(u + 1) & 1] = lds_tr_frag(qs + tro + 32 * (u + 1), BSTR);
      }
      accv[u] = mfma16(ap, bo[u & 1], accv[u]);
      acck[u] = mfma16(as, bq[u & 1], acck[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vm_all();
    __syncthreads();
  };
  // nsteps is even (two head halves per position)
  for (int i = 0; i < nsteps; i += 2) {
    step(i, std::integral_constant<int, 0>{});
    step(i + 1, std::integral_constant<int, 1>{});
  }

  // this item's partial: keys 16w + 4g + i, columns 16u + l%16
  const size_t slot = (((size_t)b * a.hkv + kvh) * pl.items + x) * KT;
  float* pk = a.part_k + slot * D;
  float* pv = a.part_v + slot * D;
#pragma unroll
  for (int u = 0; u < D / 16; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t o = (size_t)(16 * wave + 4 * g + j) * D + 16 * u + r;
      pk[o] = acck[u][j] * a.scale;
      pv[o] = accv[u][j];
    }
}

// ---------------------------------------------------------------------------
// Pooling backward: grid (ceil(max_seqlen / 128), batch, Hkv), 256 threads.
// Row r of block j gets dK = sum of its raw tile's partials over the runs
// that exist, plus p_i dKc of entry j when the block is complete (dKc = the
// sum of the entry's partials), rounded to bf16; dV likewise; and the
// block's terms g_i = dKc . K_i + dVc . V_i for the dw kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pool_kernel(BackwardArgs a, BackwardPlan pl) {
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
  const size_t unit = ((size_t)b * a.hkv + kvh) * pl.items;
  if (full) {
    // p = softmax(w_kvh), one wave
    if (wave == 0) {
      const float w0 = a.w[kvh * kBlock + lane], w1 = a.w[kvh * kBlock + 64 + lane];
      float mx = fmaxf(w0, w1);
      for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      const float e0 = __expf(w0 - mx), e1 = __expf(w1 - mx);
      float sm = e0 + e1;
      for (int o = 32; o > 0; o >>= 1) sm += __shfl_xor(sm, o);
      p_s[lane] = e0 / sm;
      p_s[64 + lane] = e1 / sm;
    }
    const int ctile = j / KT, key = j % KT;
    const int first = kBlock * (ctile * KT + 1) - 1;
    const int ns = (len - first + pl.pch - 1) / pl.pch;
    const size_t item0 = unit + (size_t)pl.raw_tiles * pl.nsr + (size_t)ctile * pl.nsc;
    for (int c = threadIdx.x; c < D; c += 256) {
      float sk = 0.f, sv = 0.f;
      for (int sp0 = 0; sp0 < ns; sp0 += 8) {  // eight runs' loads in flight, added in run order
        float bk[8], bv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (sp0 + u < ns) {
            const size_t o = ((item0 + sp0 + u) * KT + key) * D + c;
            bk[u] = a.part_k[o];
            bv[u] = a.part_v[o];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (sp0 + u < ns) {
            sk += bk[u];
            sv += bv[u];
          }
        }
      }
      dkc_s[c] = sk;
      dvc_s[c] = sv;
    }
  }
  __syncthreads();
  // rows: wave w takes rows w, w+4, ..., two per step (i and i + 4: the
  // loads of both are issued before either is used); lane l columns 8l ..
  // 8l+7.  The plan always has two runs per raw tile (nsr = 2).
  const int rows = min(kBlock, len - j * kBlock);
  for (int ib = wave; ib < rows; ib += 8) {
    f32x4 pk[2][2][2], pv[2][2][2];  // [row][run][half]
    bool use[2][2];
    bf16x8 kx[2], vx[2];
    size_t rowg[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = ib + 4 * h < rows ? ib + 4 * h : ib;  // past the end: load row ib again (not stored)
      const int rpos = j * kBlock + i;  // position in the sequence
      const int rtile = rpos / KT;
      const int t_last = min(len, rtile * KT + KT - 1 + a.window);
      const size_t item0 = unit + (size_t)rtile * pl.nsr;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        use[h][sp] = rtile * KT + sp * pl.prr < t_last;
        if (use[h][sp]) {
          const size_t o = ((item0 + sp) * KT + rpos % KT) * D + 8 * lane;
          pk[h][sp][0] = *(const f32x4*)(a.part_k + o);
          pk[h][sp][1] = *(const f32x4*)(a.part_k + o + 4);
          pv[h][sp][0] = *(const f32x4*)(a.part_v + o);
          pv[h][sp][1] = *(const f32x4*)(a.part_v + o + 4);
        }
      }
      rowg[h] = ((size_t)start + rpos) * a.hkv + kvh;
      kx[h] = *(const bf16x8*)((const bf16*)a.k + rowg[h] * D + 8 * lane);
      vx[h] = *(const bf16x8*)((const bf16*)a.v + rowg[h] * D + 8 * lane);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int i = ib + 4 * h;
      if (i >= rows) break;  // uniform per wave
      float dk8[8] = {}, dv8[8] = {};
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {  // runs in order, as in the single-row form
        if (use[h][sp]) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dk8[e] += pk[h][sp][0][e];
            dk8[4 + e] += pk[h][sp][1][e];
            dv8[e] += pv[h][sp][0][e];
            dv8[4 + e] += pv[h][sp][1][e];
          }
        }
      }
      bf16x8 ok, ov;
      float gi = 0.f;
      const float pi = full ? p_s[i] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ck = full ? dkc_s[8 * lane + e] : 0.f, cv = full ? dvc_s[8 * lane + e] : 0.f;
        ok[e] = (bf16)(dk8[e] + pi * ck);
        ov[e] = (bf16)(dv8[e] + pi * cv);
        gi = __builtin_fmaf(ck, (float)kx[h][e], __builtin_fmaf(cv, (float)vx[h][e], gi));
      }
      *(bf16x8*)((bf16*)a.dk + rowg[h] * D + 8 * lane) = ok;
      *(bf16x8*)((bf16*)a.dv + rowg[h] * D + 8 * lane) = ov;
      if (full) {
        for (int o = 32; o > 0; o >>= 1) gi += __shfl_xor(gi, o);
        if (lane == 0) a.gbuf[(((size_t)a.cu_blocks[b] + j) * a.hkv + kvh) * kBlock + i] = gi;
      }
    }
  }
}

// dw: one workgroup of 128 threads per KV head: g_i summed over every
// complete block, then dw = p (g - sum_k p_k g_k).
__global__ __launch_bounds__(128) void bwd_dw_kernel(BackwardArgs a) {
  __shared__ float red[2][2];
  const int kvh = blockIdx.x, i = threadIdx.x, lane = i & 63, wave = i >> 6;
  float gs = 0.f;
  for (int e0 = 0; e0 < a.total_blocks; e0 += 16) {  // sixteen loads in flight, added in block order
    float g[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (e0 + u < a.total_blocks) g[u] = a.gbuf[((size_t)(e0 + u) * a.hkv + kvh) * kBlock + i];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (e0 + u < a.total_blocks) gs += g[u];
  }
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
  p.raw_tiles = (max_seqlen + KT - 1) / KT;
  p.nsr = 2;  // runs of the positions that see a raw tile (64 + W - 1 of them)
  p.prr = (KT - 1 + window + p.nsr - 1) / p.nsr;
  p.comp_tiles = (max_blocks + KT - 1) / KT;
  p.pch = std::max(64, (max_seqlen + 255) / 256);
  p.nsc = std::max(1, (max_seqlen + p.pch - 1) / p.pch);
  p.items = p.raw_tiles * p.nsr + p.comp_tiles * p.nsc;
  (void)batch;
  (void)hkv;
  return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t backward_workspace_bytes(int batch, int hq, int hkv, int total_tokens, int total_blocks, int max_seqlen,
                                int window) {
  const BackwardPlan p = backward_plan(batch, hkv, max_seqlen, window);
  size_t n = 0;
  n += align256((size_t)total_tokens * hq * sizeof(float));                                    // delta
  n += 2 * align256((size_t)batch * hkv * p.items * KT * D * sizeof(float));                   // partials
  n += align256((size_t)std::max(total_blocks, 1) * hkv * kBlock * sizeof(float));            // g
  return n;
}

hipError_t launch_backward_bf16(BackwardArgs a, hipStream_t s) {
  const BackwardPlan p = backward_plan(a.batch, a.hkv, a.max_seqlen, a.window);
  char* w = (char*)a.ws;
  a.delta = (float*)w;
  w += align256((size_t)a.total_tokens * a.hq * sizeof(float));
  const size_t part = align256((size_t)a.batch * a.hkv * p.items * KT * D * sizeof(float));
  a.part_k = (float*)w;
  w += part;
  a.part_v = (float*)w;
  w += part;
  a.gbuf = (float*)w;

  if (a.batch > 0 && a.max_seqlen > 0) {
    bwd_dq_kernel<<<dim3(a.max_seqlen, a.batch, a.hkv), 256, 0, s>>>(a);
    bwd_dkv_kernel<<<dim3(p.items, a.batch, a.hkv), 256, 0, s>>>(a, p);
    bwd_pool_kernel<<<dim3((a.max_seqlen + kBlock - 1) / kBlock, a.batch, a.hkv), 256, 0, s>>>(a, p);
  }
  bwd_dw_kernel<<<a.hkv, 128, 0, s>>>(a);  // no complete block: g = 0, dw = 0
  return hipGetLastError();
}

}  // namespace hca
