// bf16 HCA prefill attention for 512-dim heads and 64 query heads per KV
// head on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// What is computed: release blog "ERNIE 5.5 Flash Base", section 2.1, HCA
// paragraph, and Zhidx article, section "1. Latent-Gated Sparse Attention":
// query t attends under one softmax (scale 1/sqrt(d)) to the complete
// compressed entries j with 128(j+1) <= t+1, then to the raw window
// max(0, t-W+1) .. t.
//
// Design (gfx950):
//  * Head packing.  The 64 query heads of a KV head read the same keys, so a
//    workgroup of 4 wavefronts owns 64 heads x 2 adjacent positions.  Wave
//    w = 2 pw + hg holds the 32 score rows "heads 32hg .. +31 of position
//    t0 + pw": every row of a wave has the same key set.
//  * Transposed products keep every per-row quantity in one lane:
//      S^T[key, row] = K[key, :] . Q^T[:, row]        (A = K from LDS, B = Q^T
//                                                        resident in 128 VGPRs)
//      O^T[col, row] += V^T[col, key] . P^T[key, row]  (A = V^T by transposed LDS
//                                                        reads, B = P)
//    With the 32x32 output layout lane l holds row l%32, so the row max and
//    sum stay in the lane pair (l, l^32) and P is formed in the registers
//    that received S.
//  * Output split.  A wave accumulates O^T for all 64 heads of its position
//    over one column half (256 AGPRs): every V^T fragment read from LDS
//    feeds two MFMAs, one per head group.  The two waves of a position swap
//    their bf16 weights through LDS.
//  * Software pipeline.  Stage s issues, interleaved one by one, the score
//    MFMAs of tile s+1 and the output MFMAs of tile s-1, and spreads the
//    softmax of tile s (VALU) between them: the three are independent, so
//    the matrix cores never wait for the exponentials.  Meanwhile K(s+2) and
//    V(s) stream into LDS.  K, V and weight buffers alternate with the
//    stage's parity; the stage loop is unrolled by two so that every LDS
//    access names its buffer at compile time (the compiler then never makes
//    an LDS read wait for direct loads into another buffer).
//  * Softmax without rescaling (Mode in bf16_tiles.h): the 256 fp32
//    accumulators per lane stay in AGPRs and are only touched by the matrix
//    cores.  A pass whose scores climb more than 32 (log2 units) above a
//    row's first maximum restarts the workgroup in the exact two-pass
//    schedule.
//  * Short key lists (<= 64 keys) carry the weights as two bf16 terms
//    P = hi + lo, lo = bf16(P - hi) (~2^-16 relative instead of 2^-9): rows
//    that see only a few keys have few large weights whose rounding does not
//    average out.  They take a plain per-tile loop (at most two tiles) in
//    the same launch as the pipelined pairs.
#include "bf16_tiles.h"

namespace hca {
namespace {

constexpr int DSTEPS = D / 16;  // k-steps of the score product (32)

// s_waitcnt on the vector-memory count alone (gfx9 encoding: vmcnt bits 3:0
// and 15:14, expcnt and lgkmcnt at their "no wait" maxima).  The builtin
// updates the compiler's own count of outstanding loads.
template <int N>
__device__ __forceinline__ void wait_vm_count() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
constexpr int HCT = 8;          // 32-column output tiles per wave (256 columns)
constexpr int WSLOT = 2048;     // LDS bytes of one wave's bf16 weights of one tile (64 lanes x 32 B)
constexpr int OSTR = 528;       // LDS bytes per staged output half-row (512 + 16 pad)

// bf16 weights of one tile in B-operand order: hi[k2] feeds key step k2.
struct Wts {
  bf16x8 hi[2];
};

// Output accumulators and softmax state of one wave.
struct PState {
  f32x16 o[2][HCT];  // O^T [0] = own head group, [1] = the partner's: lane l
                     // holds head 32g + l%32 of the wave's position and
                     // columns 256hg + 32ct + 8(r/4) + 4(l/32) + r%4
  float m, l;        // state of the wave's own score rows (lane pair l, l^32;
                     // both lanes hold m, each a partial l)
};

// Everything a stage needs besides the registers it updates.  The LDS
// pointers are the addresses of distinct __shared__ arrays.
struct Ctx {
  KeySource ks;
  RowMask rm;
  char HCA_LDS* kb[2];
  char HCA_LDS* vb[2];
  char HCA_LDS* ws[2];  // weight slots [parity]: 4 waves x WSLOT
  int* flag;
  int lane, wave, n;
  int koff;   // this lane's K fragment offset in a K tile
  int voff;   // this lane's V^T fragment offset in a V tile (column half included)
  int wown;   // this wave's slot offset (+ lane * 16)
  int wpar;   // the partner's slot offset (+ lane * 16)
  float sc2;  // softmax scale * log2(e)
};

__device__ __forceinline__ void zero_state(PState& st) {
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int ct = 0; ct < HCT; ++ct) st.o[g][ct] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Visibility mask of one tile's scores (uniform branch at the caller: only
// tiles that contain an invisible slot pay for it).  Accumulator r of lane
// l holds key slot 8(r/4) + 4(l/32) + r%4 of the tile.
__device__ __forceinline__ void mask_scores(f32x16& s, const RowMask& rm, int tile, int lane) {
  const int kk0 = tile * NT + 4 * (lane >> 5);
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = rm.valid(kk0 + 8 * (r >> 2) + (r & 3)) ? s[r] : -INFINITY;
}

// Softmax work of one tile while it is spread over a stage's steps (see
// stage()): partial maxima, the lane-pair max and reference update, 16
// exponentials, then packing to bf16 and the row sum of exactly the rounded
// weights.
struct SmWork {
  float x[16];  // partial maxima, then weights
  float mx;     // row max, then the exponent offset
  u32x4 ua, ub;
  float la, lb;
  bool over;
};

// Score MFMA k of the chain in `acc` (inline, so that the accumulator stays
// in VGPRs while the 256 AGPRs hold O).
__device__ __forceinline__ void s_mfma(int k, f32x16& acc, const bf16x8& kf, const bf16x8& qf) {
  if (k == 0)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(kf), "v"(qf));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(kf), "v"(qf));
}

// V^T fragment f of the wave's column half: column tile f & 7, key step f >> 3.
__device__ __forceinline__ int vfrag_off(int f) { return (f >> 3) * 16 * VSTR + (f & 7) * 64; }

// One pipeline stage s with parity P = s & 1 (see the file comment): the
// score product of tile s+1 (K in kb[1-P]) into `sacc`, the softmax of tile
// s from `sprev` (weights into `own` and the wave's slot ws[P]) and the
// output product of tile s-1 (V in vb[1-P]; weights in `own` and the
// partner's from ws[1-P]).  PARTS selects the parts (kScore, kSoftmax,
// kOutput): the loop's stages run all three, so the hot loop is
// straight-line code and the accumulators never change registers; the first
// two and the last two stages of a pass run only the parts whose tiles
// exist.  A part whose tile lies outside [0, n) computes on stale (finite)
// buffer contents and contributes nothing: the softmax of a missing tile
// writes zero weights, and an output product with zero weights adds zero.
// Loads K(s+2) into kb[P] and V(s) into vb[P], and ends with the workgroup
// barrier.  A kLazy softmax that exceeds the headroom raises flag[0] for the
// rest of the pass.
constexpr int kScore = 1, kSoftmax = 2, kOutput = 4, kAllParts = 7;
template <int P, int MODE, int PARTS = kAllParts>
__device__ __forceinline__ void stage(const Ctx& c, int s, const bf16x8 (&qf)[DSTEPS], f32x16& sacc,
                                      f32x16& sprev, Wts& own, PState& st) {
  constexpr bool SC = (PARTS & kScore) != 0, SM = (PARTS & kSoftmax) != 0, OU = (PARTS & kOutput) != 0;
  const bool hm = s >= 0 && s < c.n;  // tile s exists
  const unsigned keep = hm ? ~0u : 0u;  // weights of a missing tile are zeroed (no branch)
  if (s + 2 < c.n) issue_tile<4, true, false>(c.ks, s + 2, c.kb[P], nullptr, c.wave, c.lane);
  if (hm) issue_tile<4, false, true>(c.ks, s, nullptr, c.vb[P], c.wave, c.lane);
  if (SM && hm && tile_needs_mask(s, c.rm.nc, c.rm.nkeys)) {
    asm volatile("");  // a branch: most tiles need no mask
    mask_scores(sprev, c.rm, s, c.lane);
  }
  Wts par;
  if constexpr (OU) {
    const char HCA_LDS* pin = c.ws[1 - P] + c.wpar;
    par.hi[0] = *(const bf16x8 HCA_LDS*)pin;
    par.hi[1] = *(const bf16x8 HCA_LDS*)(pin + 1024);
  }
  constexpr int KPF = 3;  // K fragments read three steps ahead
  bf16x8 kf[KPF], vf[3];
  const char HCA_LDS* kr = c.kb[1 - P] + c.koff;
  const char HCA_LDS* vr = c.vb[1 - P] + c.voff;
  if constexpr (SC) {
#pragma unroll
    for (int k = 0; k < KPF; ++k) kf[k] = lds_k_frag(kr + k * 32);
  }
  if constexpr (OU) {
    vf[0] = lds_v_frag(vr + vfrag_off(0));
    vf[1] = lds_v_frag(vr + vfrag_off(1));
  }

  SmWork w;
  // 32 steps: one score MFMA, one output MFMA, a slice of the softmax
#pragma unroll
  for (int j = 0; j < DSTEPS; ++j) {
    if constexpr (SC) {
      s_mfma(j, sacc, kf[j % KPF], qf[j]);
      if (j + KPF < DSTEPS) kf[j % KPF] = lds_k_frag(kr + (j + KPF) * 32);
    }
    if constexpr (OU) {
      // output step u = j: fragment f = u / 2, head group u % 2 (0 = own)
      const int f = j >> 1, g = j & 1;
      const bf16x8 b = g ? par.hi[f >> 3] : own.hi[f >> 3];
      st.o[g][f & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[f % 3], b, st.o[g][f & 7], 0, 0, 0);
      if (g == 1 && f + 2 < 16) vf[(f + 2) % 3] = lds_v_frag(vr + vfrag_off(f + 2));
    }
    if (!SM) {
      __builtin_amdgcn_sched_barrier(0);
      continue;
    }
    if (j == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) w.x[i] = fmaxf(sprev[i], sprev[i + 8]);
    }
    if (j == 1)
      w.mx = fmaxf(fmaxf(fmaxf(w.x[0], w.x[1]), fmaxf(w.x[2], w.x[3])),
                   fmaxf(fmaxf(w.x[4], w.x[5]), fmaxf(w.x[6], w.x[7])));
    if (j == 2) {
      const float mx = max_xor32(w.mx) * c.sc2;  // sc2 > 0: max(sc2 s) == sc2 max(s)
      w.over = false;
      if (MODE == kLazy) {
        if (hm && st.m == -INFINITY) st.m = mx;  // first visible keys of the row
        w.over = hm && mx > st.m + kHeadroom;
      }
      w.mx = st.m == -INFINITY ? 0.f : -st.m;  // a row with no visible key yet: 0
    }
    if (j >= 3 && j < 11) {  // two exponentials per step
      const int i = 2 * (j - 3);
      w.x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sprev[i], c.sc2, w.mx));
      w.x[i + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(sprev[i + 1], c.sc2, w.mx));
    }
    if (j >= 11 && j < 15) {  // pack the weights (B operand: 0..7, then 8..15)
      const int q = j - 11;
      if (q == 0) w.la = w.lb = 0.f;
      w.ua[q] = pack2_bf16(w.x[2 * q], w.x[2 * q + 1]) & keep;
      w.ub[q] = pack2_bf16(w.x[8 + 2 * q], w.x[9 + 2 * q]) & keep;
      w.la = sum2_bf16(w.ua[q], w.la);
      w.lb = sum2_bf16(w.ub[q], w.lb);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // a VALU read of an MFMA result needs up to 18 wait states; the compiler
  // does not see inside the inline MFMAs, so they are spent here (24)
  if constexpr (SC) asm volatile("s_nop 15\n\ts_nop 7" : "+v"(sacc));
  if constexpr (SM) {
    st.l += w.la + w.lb;
    own.hi[0] = __builtin_bit_cast(bf16x8, w.ua);
    own.hi[1] = __builtin_bit_cast(bf16x8, w.ub);
    char HCA_LDS* pout = c.ws[P] + c.wown;
    *(u32x4 HCA_LDS*)pout = w.ua;
    *(u32x4 HCA_LDS*)(pout + 1024) = w.ub;
    if (MODE == kLazy && __any(w.over) && c.lane == 0) c.flag[0] = 1;
  }
  wait_vm_all();
  __syncthreads();
}

// One software-pipelined pass over all n >= 3 tiles in schedule MODE (kLazy
// or kFixed): stages -1 .. n.  Stage -1 only scores tile 0 and stage 0 only
// scores tile 1 and weighs tile 0; the loop runs full stages in pairs from
// stage 1 while both of a pair's score products have tiles (for odd n its
// last stage scores a missing tile); the last two stages weigh and add the
// last tiles (for odd n the very last adds a missing tile with zero
// weights).  So at most one stage's worth of the products is spent on
// missing tiles.  Every part of a stage reads only buffers loaded in this
// pass.  K(0) must be in kb[0].  The pass always runs to its end (an exit in
// the middle makes the register allocator spill); the caller then reads
// flag[0] to learn whether a kLazy pass must be redone.
template <int MODE>
__device__ __forceinline__ void pipelined_pass(const Ctx& c, const bf16x8 (&qf)[DSTEPS], PState& st) {
  f32x16 sa = {}, sb = {};  // score accumulators, alternating roles with the parity
  Wts own;
  own.hi[0] = own.hi[1] = bf16x8{};
  stage<1, MODE, kScore>(c, -1, qf, sa, sb, own, st);
  stage<0, MODE, kScore | kSoftmax>(c, 0, qf, sb, sa, own, st);
  int s = 1;
  do {
    stage<1, MODE>(c, s, qf, sa, sb, own, st);
    stage<0, MODE>(c, s + 1, qf, sb, sa, own, st);
    s += 2;
  } while (s <= c.n - 2);
  stage<1, MODE, kSoftmax | kOutput>(c, s, qf, sa, sb, own, st);
  stage<0, MODE, kOutput>(c, s + 1, qf, sb, sa, own, st);
}

// Plain per-tile loop (no overlap between the products): short key lists
// with two-term weights (LO), and the row-max pass of the exact schedule
// (kMaxOnly, scores only).  K(0) (and V(0) unless kMaxOnly) must already be
// in kb[0] / vb[0].  Weight exchange through slot ws[0] (remainders ws[1])
// with a barrier on each side.  Raises flag[0] like stage().
template <int P, int MODE, bool LO>
__device__ __forceinline__ void plain_tile(const Ctx& c, int s, const bf16x8 (&qf)[DSTEPS], PState& st) {
  constexpr bool PV = MODE != kMaxOnly;
  if (s + 1 < c.n) issue_tile<4, true, PV>(c.ks, s + 1, c.kb[1 - P], c.vb[1 - P], c.wave, c.lane);
  const char HCA_LDS* kr = c.kb[P] + c.koff;
  f32x16 sc;  // one dependent chain: this loop is not the fast path
  {
    constexpr int KPF = 2;
    bf16x8 kf[KPF];
#pragma unroll
    for (int k = 0; k < KPF; ++k) kf[k] = lds_k_frag(kr + k * 32);
#pragma unroll
    for (int k = 0; k < DSTEPS; ++k) {
      s_mfma(k, sc, kf[k % KPF], qf[k]);
      if (k + KPF < DSTEPS) kf[k % KPF] = lds_k_frag(kr + (k + KPF) * 32);
    }
    asm volatile("s_nop 15\n\ts_nop 7" : "+v"(sc));
  }
  if (tile_needs_mask(s, c.rm.nc, c.rm.nkeys)) mask_scores(sc, c.rm, s, c.lane);
  float mx = sc[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
  mx = max_xor32(mx) * c.sc2;
  if (MODE == kMaxOnly) {
    st.m = fmaxf(st.m, mx);
    wait_vm_all();
    __syncthreads();
    return;
  }
  bool over = false;
  if (MODE == kLazy) {
    if (st.m == -INFINITY) st.m = mx;
    over = mx > st.m + kHeadroom;
  }
  const float nm = st.m == -INFINITY ? 0.f : -st.m;
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], c.sc2, nm));
  u32x4 ua, ub, va = {}, vb = {};
  float ls = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ua[q] = pack2_bf16(x[2 * q], x[2 * q + 1]);
    ub[q] = pack2_bf16(x[8 + 2 * q], x[9 + 2 * q]);
    ls = sum2_bf16(ub[q], sum2_bf16(ua[q], ls));
    if (LO) {
      va[q] = pack2_bf16(x[2 * q] - bf16_lo(ua[q]), x[2 * q + 1] - bf16_hi(ua[q]));
      vb[q] = pack2_bf16(x[8 + 2 * q] - bf16_lo(ub[q]), x[9 + 2 * q] - bf16_hi(ub[q]));
      ls = sum2_bf16(vb[q], sum2_bf16(va[q], ls));
    }
  }
  st.l += ls;
  // exchange the weights with the partner wave (slot ws[0]: hi, then lo in ws[1])
  {
    char HCA_LDS* o0 = c.ws[0] + c.wown;
    *(u32x4 HCA_LDS*)o0 = ua;
    *(u32x4 HCA_LDS*)(o0 + 1024) = ub;
    if (LO) {
      char HCA_LDS* o1 = c.ws[1] + c.wown;
      *(u32x4 HCA_LDS*)o1 = va;
      *(u32x4 HCA_LDS*)(o1 + 1024) = vb;
    }
    if (MODE == kLazy && __any(over) && c.lane == 0) c.flag[0] = 1;
  }
  __syncthreads();
  const char HCA_LDS* vr = c.vb[P] + c.voff;
#pragma unroll
  for (int part = 0; part < (LO ? 2 : 1); ++part) {
    bf16x8 b[2][2];  // [group own/partner][key step]
    b[0][0] = __builtin_bit_cast(bf16x8, part ? va : ua);
    b[0][1] = __builtin_bit_cast(bf16x8, part ? vb : ub);
    b[1][0] = *(const bf16x8 HCA_LDS*)(c.ws[part] + c.wpar);
    b[1][1] = *(const bf16x8 HCA_LDS*)(c.ws[part] + c.wpar + 1024);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      const bf16x8 vf = lds_v_frag(vr + vfrag_off(f));
#pragma unroll
      for (int g = 0; g < 2; ++g)
        st.o[g][f & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, b[g][f >> 3], st.o[g][f & 7], 0, 0, 0);
    }
  }
  wait_vm_all();
  __syncthreads();  // partner weights read, buffers of this parity free
}

template <int MODE, bool LO>
__device__ __forceinline__ void plain_pass(const Ctx& c, const bf16x8 (&qf)[DSTEPS], PState& st) {
  int s = 0;
  for (; s + 1 < c.n; s += 2) {
    plain_tile<0, MODE, LO>(c, s, qf, st);
    plain_tile<1, MODE, LO>(c, s + 1, qf, st);
  }
  if (s < c.n) plain_tile<0, MODE, LO>(c, s, qf, st);
}

// Start of a pass: clear the flag and slot ws[0], load K(0) (and V(0) for
// the plain loop).
__device__ __forceinline__ void pass_setup(const Ctx& c, bool with_v) {
  if (c.lane == 0 && c.wave == 0) c.flag[0] = c.flag[1] = 0;
  for (int o = threadIdx.x * 16; o < 4 * WSLOT; o += 256 * 16) *(u32x4 HCA_LDS*)(c.ws[0] + o) = u32x4{};
  if (with_v)
    issue_tile<4, true, true>(c.ks, 0, c.kb[0], c.vb[0], c.wave, c.lane);
  else
    issue_tile<4, true, false>(c.ks, 0, c.kb[0], nullptr, c.wave, c.lane);
  wait_vm_all();
  __syncthreads();
}

// All tiles: single-pass schedule first; if a row's scores grew past the
// headroom, the exact two-pass schedule (row max, then weights <= 1).  LO:
// two-term weights in the plain loop (short key lists).
template <bool LO>
__device__ __forceinline__ void attend_pair(const Ctx& c, const bf16x8 (&qf)[DSTEPS], PState& st) {
  zero_state(st);
  pass_setup(c, LO);
  if (LO)
    plain_pass<kLazy, true>(c, qf, st);
  else
    pipelined_pass<kLazy>(c, qf, st);
  if (!c.flag[0]) return;  // read after the pass's last barrier
  __syncthreads();         // every wave has read the flag
  zero_state(st);
  pass_setup(c, false);
  plain_pass<kMaxOnly, false>(c, qf, st);
  pass_setup(c, LO);
  if (LO)
    plain_pass<kFixed, true>(c, qf, st);
  else
    pipelined_pass<kFixed>(c, qf, st);
}

// Attention epilogue (release blog "ERNIE 5.5 Flash Base", section 2.1,
// last paragraph: a per-head output gate and a cross-head low-rank mixing
// with identity skip after attention): y = sigmoid(g) (O + U (V^T O)) over
// the 64 heads of the position, O = acc / l, for the wave's 256 columns.
// The wave holds all 64 heads (st.o[0]: heads 32hg + l%32, st.o[1]: the
// partner group) as O^T tiles, lane = head.  Per 32-column tile ct, two
// matrix-core products:
//   Z [ranks x cols] = V^T O: A = V^T (constant), B = O read back transposed
//     from bf16 rows (one per head) staged in the wave's own LDS buffer;
//   M^T = Z^T U^T: A = Z^T straight from Z's accumulators (lane = column),
//     B = U^T, from zero; then y = sigmoid(g) (acc / l + M) elementwise
//     (the accumulators are only read).
// The ranks run in the k-slot order Z's accumulator layout gives (lane
// group h: ranks 4h..4h+3, 8+4h..8+4h+3 of each 16), and V^T follows the
// head order of the transposed reads.  V^T, U^T and the gate come from LDS,
// loaded at the start of the pass.  y is rounded and written over the
// tile's staged columns (already read), then all 64 rows are stored.
constexpr float kLn2 = 0.6931471805599453f;
constexpr int MSTR = 520;  // LDS bytes per staged head row (64 rows fill a K buffer)

__device__ __forceinline__ int kslot_index(int h, int j) { return j < 4 ? 4 * h + j : 8 + 4 * h + (j - 4); }

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// Epilogue inputs in LDS, written at the start of the pass (the epilogue's
// global loads would otherwise stall every workgroup's tail): the mixing
// factors as bf16 MFMA fragments and the gate's sigmoid of both positions.
constexpr int kEpiV = 0;        // V^T: [rank 32][k-step 4][lane half 2][8 heads] bf16
constexpr int kEpiU = 4096;     // U^T: [head 64][k-step 2][lane half 2][8 ranks] bf16
constexpr int kEpiGate = 8192;  // [position 2][head 64] fp32
constexpr int kEpiBytes = 8704;

// O = acc / l for all 64 heads of the wave's position over its column half,
// rounded to bf16.  1/l of the partner's rows comes through LDS.  The
// half-rows are staged in the wave's own buffer, one head group (32 rows x
// OSTR bytes) at a time, and stored two per instruction (lanes 0-31 row 2i,
// lanes 32-63 row 2i+1; 512 contiguous bytes each).  EPI: the head mixing
// and the per-head gate first, with their inputs from `epi`.
template <bool EPI, bool INL>
__device__ __forceinline__ void store_output(const Ctx& c, PState& st, float* linv, bf16* obase,
                                             bool row_ok, const PrefillArgs& a, const char HCA_LDS* epi,
                                             float* lse_row, const char* pf0, const char* pf1) {
  // EPI: the lane index afresh from an opaque mbcnt (derived from the pass's
  // copy, lane & 31 stayed live across the whole pass and was spilled)
  int lane = c.lane;
  if constexpr (EPI) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  const int wave = c.wave, hg = wave & 1;
  const float lt = st.l + __shfl_xor(st.l, 32);
  const float inv_own = 1.f / lt;
  if (lane < 32) linv[wave * 32 + lane] = lt;  // the row sums; the partner divides itself
  __syncthreads();  // every wave is past its last tile: K/V buffers are free
  const float l_par = linv[(wave ^ 1) * 32 + (lane & 31)];
  const float inv_par = 1.f / l_par;
  // Fused epilogue only: warm this XCD's L2 with the query rows of the
  // workgroup that most likely runs next on it (kPrefetchAhead), whose
  // query loads (see prefill_body) then hit L2.  One dword of
  // every 128-byte line, issued after the barrier so that its fence does not
  // wait for them; the values only feed an empty asm statement at the very
  // end, so the wait for them comes after the output stores are issued.
  // (The plain kernel did not gain from this: +1 % at 128K.  Without it the
  // fused epilogue is 8 % slower at 8K and 4 % at 128K.)
  typedef const __attribute__((address_space(1))) unsigned* gptr;
  unsigned pfv[4] = {0u, 0u, 0u, 0u};
  if (EPI && pf0) {
    const int o = (wave * 64 + lane) * 256;  // 64 KiB per position: two lines per thread
    pfv[0] = *(gptr)(pf0 + o);
    pfv[1] = *(gptr)(pf0 + o + 128);
    if (pf1) {
      pfv[2] = *(gptr)(pf1 + o);
      pfv[3] = *(gptr)(pf1 + o + 128);
    }
  }
  if constexpr (EPI) asm volatile("" ::: "memory");  // the loads stay here
  auto consume = [&]() {
    if constexpr (EPI) asm volatile("" ::"v"(pfv[0]), "v"(pfv[1]), "v"(pfv[2]), "v"(pfv[3]));
  };
  if (!row_ok) {
    consume();
    return;
  }
  // log-sum-exp of the row's scaled scores (natural log): the weights are
  // exp2(s sc2 - m), so sum exp(scale s) = 2^m lt
  if (lse_row && lane < 32) lse_row[lane] = (st.m + __log2f(lt)) * kLn2;
  char HCA_LDS* stg = wave == 0 ? c.kb[0] : wave == 1 ? c.kb[1] : wave == 2 ? c.vb[0] : c.vb[1];
  if constexpr (EPI) {
    const int h = lane >> 5, r = lane & 31;
    const bool mix = a.mix_u != nullptr;
    const int rank = a.mix_rank;
    float gs[2] = {1.f, 1.f};  // gate of head group g (own, partner)
    if (a.gate) {
      const float HCA_LDS* gr = (const float HCA_LDS*)(epi + kEpiGate) + 64 * (wave >> 1) + r;
      gs[0] = gr[32 * hg];
      gs[1] = gr[32 * (hg ^ 1)];
    }
    // V^T (A of Z = V^T O, k-step s) and U^T (B of U Z, head group g, k-step s2)
    auto load_vt = [&](bf16x8(&vt)[4]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) vt[s] = *(const volatile bf16x8 HCA_LDS*)(epi + kEpiV + ((r * 4 + s) * 2 + h) * 16);
    };
    auto load_ut = [&](bf16x8(&ut)[2][2]) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          ut[g][s2] =
              *(const volatile bf16x8 HCA_LDS*)(epi + kEpiU + (((32 * (hg ^ g) + r) * 2 + s2) * 2 + h) * 16);
    };
    bf16x8 vt0[4], ut0[2][2];
    if (!INL && mix) {
      load_vt(vt0);
      load_ut(ut0);
    }
    const int off = (4 * h + ((lane & 15) >> 2)) * MSTR + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < HCT; ++ct) {
      // Two forms of the Z and mixing products.  Builtin MFMAs with V^T, U^T
      // held across the loop (the pipelined pairs: the compiler overlaps the
      // products with the VALU work and the LDS reads), and inline MFMAs
      // with VGPR accumulators, V^T, U^T read again for every column tile
      // (the two-term pairs).  The second form needs far fewer registers:
      // there, with the builtin form the allocator put the products'
      // operands in AGPRs and spilled the O accumulators it moved out of
      // them.  The compiler does not see inside an inline MFMA, so each asm
      // chain also spends the wait states around it: 5 before (its operands
      // may just have been written by the VALU) and 24 after (a VALU read of
      // the result, or a write to one of its operand registers, waits for
      // the matrix core).
      // this column tile of O (both head groups), read from the accumulators
      // once: staged as bf16 rows (row = head 0..63, the wave's own columns)
      // for the Z product's transposed reads, then reused for the output
      float ov[2][16];
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 16; ++i) ov[g][i] = st.o[g][ct][i];
      bf16x8 za[2], vt[4], ut[2][2];
      if (mix) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const float inv = g ? inv_par : inv_own;
          char HCA_LDS* rowp = stg + (32 * (hg ^ g) + r) * MSTR + h * 8 + 64 * ct;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = (bf16)(ov[g][4 * q4 + i] * inv);
            *(bf16x4 HCA_LDS*)(rowp + 16 * q4) = v;
          }
        }
        if constexpr (INL) {
          load_vt(vt);
          load_ut(ut);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) vt[s] = vt0[s];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) ut[g][s2] = ut0[g][s2];
        }
        bf16x8 bq[4];  // B = the staged O/l, k-step s (64 heads)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const char HCA_LDS* base = stg + off + 16 * s * MSTR + 64 * ct;
          const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)base);
          const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)(base + 8 * MSTR));
          bq[s] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        f32x16 z = {};
        if constexpr (INL) {
          asm volatile(
              "s_nop 4\n\t"
              "v_mfma_f32_32x32x16_bf16 %0, %1, %5, 0\n\t"
              "v_mfma_f32_32x32x16_bf16 %0, %2, %6, %0\n\t"
              "v_mfma_f32_32x32x16_bf16 %0, %3, %7, %0\n\t"
              "v_mfma_f32_32x32x16_bf16 %0, %4, %8, %0\n\t"
              "s_nop 15\n\ts_nop 7"
              : "=&v"(z)
              : "v"(vt[0]), "v"(vt[1]), "v"(vt[2]), "v"(vt[3]), "v"(bq[0]), "v"(bq[1]), "v"(bq[2]), "v"(bq[3]));
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt[s], bq[s], z, 0, 0, 0);
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int j = 0; j < 8; ++j) za[s2][j] = (bf16)z[8 * s2 + j];
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        f32x16 y = {};  // the mixing term of these 32 heads x 32 columns
        if (mix) {
          if constexpr (INL) {
            if (rank > 16)
              asm volatile(
                  "s_nop 4\n\t"
                  "v_mfma_f32_32x32x16_bf16 %0, %1, %3, 0\n\t"
                  "v_mfma_f32_32x32x16_bf16 %0, %2, %4, %0\n\t"
                  "s_nop 15\n\ts_nop 7"
                  : "=&v"(y)
                  : "v"(za[0]), "v"(za[1]), "v"(ut[g][0]), "v"(ut[g][1]));
            else
              asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0\n\ts_nop 15\n\ts_nop 7"
                           : "=&v"(y)
                           : "v"(za[0]), "v"(ut[g][0]));
          } else {
            y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[0], ut[g][0], y, 0, 0, 0);
            if (rank > 16) y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(za[1], ut[g][1], y, 0, 0, 0);
          }
        }
        const float inv = g ? inv_par : inv_own;
        char HCA_LDS* rowp = stg + (32 * (hg ^ g) + r) * MSTR + h * 8 + 64 * ct;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = (bf16)((ov[g][4 * q4 + i] * inv + y[4 * q4 + i]) * gs[g]);
          *(bf16x4 HCA_LDS*)(rowp + 16 * q4) = v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one column tile at a time
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
    // 64 rows x 512 bytes: lanes 0-31 row 2i, lanes 32-63 row 2i+1
    const int cw = r * 8;
#pragma unroll 4
    for (int i = 0; i < 32; ++i) {
      const int row = 2 * i + h;
      const char HCA_LDS* src = stg + row * MSTR + cw * 2;  // 8-byte aligned rows
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v0 = *(const u32x2 HCA_LDS*)src, v1 = *(const u32x2 HCA_LDS*)(src + 8);
      const u32x4 v = {v0[0], v0[1], v1[0], v1[1]};
      __builtin_nontemporal_store(v, (u32x4*)(obase + (size_t)row * D + cw));
    }
    consume();
    return;
  }
  const int hr = lane >> 5, cw = (lane & 31) * 8;
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float inv = g ? inv_par : inv_own;
    char HCA_LDS* rowp = stg + (lane & 31) * OSTR + (lane >> 5) * 8;
#pragma unroll
    for (int ct = 0; ct < HCT; ++ct)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(st.o[g][ct][4 * q4 + i] * inv);
        *(bf16x4 HCA_LDS*)(rowp + (32 * ct + 8 * q4) * 2) = v;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
    bf16* og = obase + (size_t)(32 * (hg ^ g)) * D;
    // streaming stores: each output row is written once and not read here
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int row = 2 * i + hr;
      __builtin_nontemporal_store(*(const bf16x8 HCA_LDS*)(stg + row * OSTR + cw * 2),
                                  (bf16x8*)(og + (size_t)row * D + cw));
    }
  }
  consume();
}

// The epilogue's inputs into LDS, once per workgroup: V^T and U^T of KV head
// kvh as bf16 fragments (rank rows past `mix_rank` zero) and the gate's
// sigmoid for the pair's positions (rows row0, row0 + 1; the second only if
// it exists).  In two steps around the query loads:
//  * issue_epilogue_inputs, before the query loads: U and V of the KV head
//    (fp32, 64 x rank each, contiguous) go into `ustage` and `vstage` (8 KiB
//    each: the weight slots, free until the pass starts) with direct loads,
//    one row of up to 1 KiB per instruction (a range check zero-fills the
//    rest of a partial row); the gate logits of the two positions (64 fp32
//    each) go straight into the gate area of `epi` with one dword per lane.
//    The query loads' wait then covers these too: no round trip of their own.
//  * build_epilogue_inputs (after every wave's rows have landed): each
//    thread gathers its 8 + 8 values from the stages, rounds them to bf16
//    and writes one V^T and one U^T fragment chunk, and threads 0..127 turn
//    their gate logit into its sigmoid in place.
constexpr int kEpiStageBytes = G * 32 * 4;  // one staged factor: 64 heads x rank <= 32, fp32
static_assert(kEpiStageBytes <= 4 * WSLOT, "a staged mixing factor fits in one weight slot array");

__device__ __forceinline__ void issue_epilogue_inputs(const PrefillArgs& a, char HCA_LDS* ustage,
                                                      char HCA_LDS* vstage, char HCA_LDS* epi, int kvh, int row0,
                                                      bool t1_ok, int wave, int lane) {
  if (a.mix_u) {
    const int bytes = G * a.mix_rank * (int)sizeof(float);
    const int rows = (bytes + 1023) / 1024;  // <= 8
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(a.mix_u + (size_t)kvh * G * a.mix_rank, (size_t)bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.mix_v + (size_t)kvh * G * a.mix_rank, (size_t)bytes);
    for (int row = wave; row < rows; row += 4) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ru, (void HCA_LDS*)(ustage + row * 1024), 16, lane * 16, row * 1024,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (void HCA_LDS*)(vstage + row * 1024), 16, lane * 16, row * 1024,
                                               0, 0);
    }
  }
  if (a.gate && wave < 2) {  // wave p loads position p's 64 logits (the first position again if p absent)
    const int row = row0 + (wave == 1 && t1_ok ? 1 : 0);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gate + (size_t)row * a.hq + kvh * G, G * sizeof(float));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (void HCA_LDS*)(epi + kEpiGate + wave * G * 4), 4, lane * 4, 0, 0,
                                             0);
  }
}

__device__ __forceinline__ void build_epilogue_inputs(const PrefillArgs& a, const char HCA_LDS* ustage,
                                                      const char HCA_LDS* vstage, char HCA_LDS* epi) {
  const int i8 = threadIdx.x, gh = i8 & 1;
  if (a.mix_u) {
    const int rank = a.mix_rank;
    const float HCA_LDS* us = (const float HCA_LDS*)ustage;
    const float HCA_LDS* vs = (const float HCA_LDS*)vstage;
    const int rv = i8 >> 3, sv = (i8 >> 1) & 3;  // V^T chunk: rank rv, heads 16 sv + kslot_index(gh, j)
    const int hu = i8 >> 2, su = (i8 >> 1) & 1;  // U^T chunk: head hu, ranks 16 su + kslot_index(gh, j)
    bf16x8 fv, fu;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int ru = 16 * su + kslot_index(gh, j);
      const float x = vs[(16 * sv + kslot_index(gh, j)) * rank + min(rv, rank - 1)];
      const float y = us[hu * rank + min(ru, rank - 1)];
      fv[j] = (bf16)(rv < rank ? x : 0.f);
      fu[j] = (bf16)(ru < rank ? y : 0.f);
    }
    *(bf16x8 HCA_LDS*)(epi + kEpiV + 16 * i8) = fv;
    *(bf16x8 HCA_LDS*)(epi + kEpiU + 16 * i8) = fu;
  }
  if (a.gate && i8 < 128) {  // position i8 / 64, head i8 % 64: read and written by this thread only
    float HCA_LDS* gp = (float HCA_LDS*)(epi + kEpiGate) + i8;
    *gp = sigmoid(*gp);
  }
}

// The Q^T fragments of one wave's 32 score rows (lane l: row l%32, elements
// 16k + 8(l/32) .. +7 of k-step k).  The rows are 32 KiB contiguous in HBM
// (qwave: heads 32hg .. +31 of one position); they come into `buf` with
// direct loads, one 1 KiB row per instruction (row offset in the scalar
// offset, lane offset fixed), and are read back with the K fragment pattern.
// Loading the fragments straight from HBM (each lane 16 bytes of 32
// different rows per instruction) touched every cache line four times and
// took about four times as long.
__device__ __forceinline__ void load_q(const bf16* qwave, char HCA_LDS* buf, int lane, int koff,
                                       bf16x8 (&qf)[DSTEPS]) {
  const __amdgpu_buffer_rsrc_t r = make_rsrc(qwave, (size_t)32 * D * sizeof(bf16));
#pragma unroll
  for (int row = 0; row < 32; ++row)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void HCA_LDS*)(buf + row * KSTR), 16, lane * 16,
                                             row * D * (int)sizeof(bf16), 0, 0);
  wait_vm_all();
#pragma unroll
  for (int k = 0; k < DSTEPS; ++k) qf[k] = lds_k_frag(buf + koff + k * 32);
}

// Keys of position pair (t0, t_last): the later position's complete entries
// plus the raw rows from the earlier position's window start to t_last.
__host__ __device__ inline int pair_keys(int t0, int t_last, int window) {
  const int lo = t0 - window + 1 > 0 ? t0 - window + 1 : 0;
  return (t_last + 1) / kBlock + (t_last - lo + 1);
}

// ---------------------------------------------------------------------------
// One position pair of one (sequence, KV head), pair index bx + pair0.  LO =
// true handles the pairs whose key list has at most kTwoTermKeys keys
// (two-term weights, plain loop), LO = false all others (pipelined); each
// skips the pairs of the other kind.
// ---------------------------------------------------------------------------
template <bool LO, bool EPI>
__device__ __forceinline__ void prefill_body(const PrefillArgs& a, int pair0, int bx, int pf_pair, char HCA_LDS* k0_s,
                                             char HCA_LDS* k1_s, char HCA_LDS* v0_s, char HCA_LDS* v1_s,
                                             char HCA_LDS* w0_s, char HCA_LDS* w1_s, int* flag_s, float* linv_s,
                                             char HCA_LDS* epi_s) {
  const int b = blockIdx.y, kvh = blockIdx.z;

  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;  // query rows (positions p0 .. p0+len-1)
  const int pair = bx + pair0;
  if (2 * pair >= len) return;
  const int p0 = a.pos0 ? a.pos0[b] : 0;
  {
    const int t0 = p0 + 2 * pair;
    const int t_last = 2 * pair + 1 < len ? t0 + 1 : t0;
    if ((pair_keys(t0, t_last, a.window) <= kTwoTermKeys) != LO) return;
  }
  // the fused epilogue takes the lane index from mbcnt, which the compiler
  // can recompute where it is needed: derived from threadIdx.x, it kept that
  // register live to the end and spilled it, and the reload's wait then
  // also waited for the L2 prefetch of the output epilogue
  const int lane = EPI ? __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) : threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pw = wave >> 1, hg = wave & 1;
  const bool t1_ok = 2 * pair + 1 < len;
  const int t0 = p0 + 2 * pair;  // positions
  const int t_last = t1_ok ? t0 + 1 : t0;
  const bool row_ok = pw == 0 || t1_ok;
  const int t = row_ok ? t0 + pw : t0;  // an absent second position recomputes t0
  const int qrow = start + (t - p0);    // its query / output row

  const int nc = (t_last + 1) / kBlock;      // entries visible to the later position
  const int lo = max(0, t0 - a.window + 1);  // oldest raw key of the earlier position
  const int nkeys = nc + (t_last - lo + 1);

  Ctx c;
  c.ks.rstride = a.hkv * D * (int)sizeof(bf16);
  {
    const size_t rs = (size_t)c.ks.rstride;
    const size_t head_off = (size_t)kvh * D * sizeof(bf16);
    const int nb = a.cu_blocks[b + 1] - a.cu_blocks[b];
    c.ks.comp_k = make_rsrc((const char*)a.kc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
    c.ks.comp_v = make_rsrc((const char*)a.vc + (size_t)a.cu_blocks[b] * rs + head_off, (size_t)nb * rs);
    // raw rows of the sequence: positions p0 - halo onward
    const size_t row0 = (size_t)start + (size_t)b * a.halo;
    c.ks.raw_k = make_rsrc((const char*)a.k + row0 * rs + head_off, (size_t)(len + a.halo) * rs);
    c.ks.raw_v = make_rsrc((const char*)a.v + row0 * rs + head_off, (size_t)(len + a.halo) * rs);
  }
  c.ks.nc = nc;
  c.ks.nkeys = nkeys;
  c.ks.raw0 = lo - (p0 - a.halo);
  c.ks.ring = 0;
  c.rm.nc = nc;
  c.rm.nkeys = nkeys;
  c.rm.nvis_c = (t + 1) / kBlock;
  c.rm.r0 = nc + max(t - a.window + 1, lo) - lo;
  c.rm.r1 = nc + t - lo;
  c.kb[0] = (char HCA_LDS*)k0_s;
  c.kb[1] = (char HCA_LDS*)k1_s;
  c.vb[0] = (char HCA_LDS*)v0_s;
  c.vb[1] = (char HCA_LDS*)v1_s;
  c.ws[0] = (char HCA_LDS*)w0_s;
  c.ws[1] = (char HCA_LDS*)w1_s;
  c.flag = flag_s;
  c.lane = lane;
  c.wave = wave;
  c.n = (nkeys + NT - 1) / NT;
  c.koff = (lane & 31) * KSTR + (lane >> 5) * 16;
  c.voff = (4 * (lane >> 5) + ((lane & 15) >> 2)) * VSTR + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2 +
           hg * HCT * 64;
  c.wown = wave * WSLOT + lane * 16;
  c.wpar = (wave ^ 1) * WSLOT + lane * 16;
  c.sc2 = a.scale * kLog2e;

  // Q^T fragments of the wave's 32 rows (heads 32hg .. +31 of position t),
  // staged through the wave's own tile buffer (see load_q); each buffer
  // names a distinct array, so the branches are uniform and compile-time.
  const bf16* qwave = (const bf16*)a.q + ((size_t)qrow * a.hq + kvh * G + 32 * hg) * D;
  bf16x8 qf[DSTEPS];
  {
    // the epilogue's inputs go first, into LDS the query staging leaves free
    if constexpr (EPI)
      issue_epilogue_inputs(a, c.ws[0], c.ws[1], epi_s, kvh, start + (t0 - p0), t1_ok, wave, lane);
    if (wave == 0)
      load_q(qwave, c.kb[0], lane, c.koff, qf);
    else if (wave == 1)
      load_q(qwave, c.kb[1], lane, c.koff, qf);
    else if (wave == 2)
      load_q(qwave, c.vb[0], lane, c.koff, qf);
    else
      load_q(qwave, c.vb[1], lane, c.koff, qf);
    __syncthreads();  // every wave holds its fragments and every staged input has landed
    if constexpr (EPI) {
      build_epilogue_inputs(a, c.ws[0], c.ws[1], epi_s);
      __syncthreads();  // the stages are read before the pass clears ws[0]
    }
  }

  PState st;
  attend_pair<LO>(c, qf, st);
  bf16* obase = (bf16*)a.o + ((size_t)qrow * a.hq + kvh * G) * D + hg * 256;
  float* lse_row = a.lse ? a.lse + (size_t)qrow * a.hq + kvh * G + 32 * hg : nullptr;
  const char* pf0 = nullptr;
  const char* pf1 = nullptr;
  if (pf_pair >= 0 && 2 * pf_pair < len) {
    const char* q0 = (const char*)a.q + ((size_t)(start + 2 * pf_pair) * a.hq + kvh * G) * D * sizeof(bf16);
    pf0 = q0;
    if (2 * pf_pair + 1 < len) pf1 = q0 + (size_t)a.hq * D * sizeof(bf16);
  }
  store_output<EPI, LO>(c, st, linv_s, obase, row_ok, a, epi_s, lse_row, pf0, pf1);
}

// Grid (lo_n + npairs - hi_begin, batch, Hkv), 256 threads: workgroup x <
// lo_n takes two-term pair x, the others pair hi_begin + x - lo_n.  Both
// kinds share one launch (and one LDS layout); the branch is uniform per
// workgroup, and the two bodies are separate inlined copies so neither
// carries the other's register state.
//
// Workgroup x runs on XCD x mod 8, and neighbouring pairs read mostly the
// same raw window rows.  In every run of 8 G pipelined workgroups, the G
// workgroups of one XCD take G consecutive pairs, so each XCD's L2 fetches
// the window rows of its own pairs instead of every row of the sequence
// (a permutation of the pairs; a tail shorter than 8 G keeps its order).
constexpr int kXcdGroup = 32;  // pairs per XCD per run: one per CU of an XCD
// Workgroups are dispatched in id order, each XCD taking every eighth; with
// 32 CUs per XCD busy, the workgroup that starts on an XCD when one ends
// there is about 256 ids later.  Its query rows are prefetched into L2.
constexpr int kPrefetchAhead = 8 * kXcdGroup;
__device__ __forceinline__ int xcd_local_pair(int u, int n) {
  const int full = n / (8 * kXcdGroup) * (8 * kXcdGroup);
  if (u >= full) return u;
  const int r = u & 7, s = u >> 3;
  return (s / kXcdGroup) * 8 * kXcdGroup + r * kXcdGroup + s % kXcdGroup;
}
template <bool EPI>
__global__ __launch_bounds__(256, 1) void prefill_bf16_kernel(PrefillArgs a, int lo_n, int hi_begin) {
  __shared__ __attribute__((aligned(16))) char k0_s[KTILE];
  __shared__ __attribute__((aligned(16))) char k1_s[KTILE];
  __shared__ __attribute__((aligned(16))) char v0_s[VTILE];
  __shared__ __attribute__((aligned(16))) char v1_s[VTILE];
  __shared__ __attribute__((aligned(16))) char w0_s[4 * WSLOT];
  __shared__ __attribute__((aligned(16))) char w1_s[4 * WSLOT];
  __shared__ int flag_s[2];
  __shared__ float linv_s[4 * 32];
  __shared__ __attribute__((aligned(16))) char epi_s[EPI ? kEpiBytes : 16];
#define HCA_LDS_ARGS (char HCA_LDS*)k0_s, (char HCA_LDS*)k1_s, (char HCA_LDS*)v0_s, (char HCA_LDS*)v1_s, \
    (char HCA_LDS*)w0_s, (char HCA_LDS*)w1_s, flag_s, linv_s, (char HCA_LDS*)epi_s
  if ((int)blockIdx.x < lo_n) {
    prefill_body<true, EPI>(a, 0, blockIdx.x, -1, HCA_LDS_ARGS);
  } else {
    const int n = gridDim.x - lo_n, x = blockIdx.x - lo_n;
    prefill_body<false, EPI>(a, hi_begin, xcd_local_pair(x, n),
                             EPI && x + kPrefetchAhead < n ? hi_begin + xcd_local_pair(x + kPrefetchAhead, n) : -1,
                             HCA_LDS_ARGS);
  }
#undef HCA_LDS_ARGS
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  const int npairs = (a.max_seqlen + 1) / 2;
  // Key counts grow with the pair index, so the two-term pairs are a prefix
  // of every sequence: pairs [0, lo_end) may be two-term (a lone last
  // position has one key less than a full pair), pairs [hi_begin, npairs)
  // may be not; each body checks every pair it is given.
  auto first_over = [&](bool lone) {  // first pair with more than kTwoTermKeys keys
    int lo = 0, hi = npairs;
    while (lo < hi) {
      const int m = lo + (hi - lo) / 2;
      if (pair_keys(2 * m, 2 * m + (lone ? 0 : 1), a.window) > kTwoTermKeys)
        hi = m;
      else
        lo = m + 1;
    }
    return lo;
  };
  // Chunks start at pos0 >= 0: any of the first lo_end pairs may be of
  // either kind, so the pipelined body also gets all of them.
  const int lo_end = first_over(true), hi_begin = a.pos0 ? 0 : first_over(false);
  const dim3 grid(lo_end + npairs - hi_begin, a.batch, a.hkv);
  if (a.gate || a.mix_u)
    prefill_bf16_kernel<true><<<grid, 256, 0, s>>>(a, lo_end, hi_begin);
  else
    prefill_bf16_kernel<false><<<grid, 256, 0, s>>>(a, lo_end, hi_begin);
  return hipGetLastError();
}

}  // namespace hca
