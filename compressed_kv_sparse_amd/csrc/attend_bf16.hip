// bf16 HCA attention for 512-dim heads and 64 query heads per KV head, on
// CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).
//
// What is computed (release blog "ERNIE 5.5 Flash Base", section 2.1, HCA
// paragraph; Zhidx article, section "1. Latent-Gated Sparse Attention"): each
// query attends, under one softmax scaled by 1/sqrt(d), to the complete
// compressed entries of its sequence (block j visible once 128(j+1) <= t+1)
// followed by the raw window max(0, t-W+1) .. t.  The model card gives the
// 512-dim heads; the Zhidx article the 64 query heads.
//
// Design (gfx950):
//  * Head packing.  All 64 query heads of one KV head read the same keys, so
//    a wavefront owns 32 query rows = 32 heads of ONE position: every row of
//    the wave has the same key set and the key tile is shared by 32 rows in
//    registers.  A prefill workgroup = 4 wavefronts = 64 heads x 2 adjacent
//    positions (their key sets differ in at most two keys, masked per row).
//  * Transposed products keep every per-row quantity inside one lane:
//      S^T[key, row] = K[key, :] . Q^T[:, row]      (A = K from LDS, B = Q in VGPRs)
//      O^T[col, row] += V^T[col, key] . P^T[key, row] (A = V^T via transposed LDS
//                                                      reads, B = P from VGPRs)
//    With the 32x32 MFMA output layout, lane l holds row l%32 of S^T and of
//    O^T, so the softmax row max/sum never leave the lane pair (l, l^32) and
//    P goes from the S accumulators straight into the B operand without LDS.
//  * Keys stream in tiles of 32 through LDS with direct global->LDS 16-byte
//    loads (one 1 KiB row per wave instruction, fully coalesced), double
//    buffered so the next tile is in flight during the current one's math.
//    K rows are padded to 1040 bytes and V rows to 1088 bytes so the 16-byte
//    K fragment reads and the transposed 8-byte V reads hit distinct banks.
//  * Softmax in base 2 (log2 e folded into the scale) without accumulator
//    rescaling: a row fixes its reference max m at the first tile where it
//    sees a key and uses exp2(s - m) from then on.  Weights stay <= 2^32 as
//    long as no later score exceeds m by more than 32 (in log2 units); if one
//    does, the whole workgroup restarts in an exact two-pass schedule (pass 1:
//    row max over all keys; pass 2: weights exp2(s - max) <= 1).  The 256 fp32
//    accumulators per lane therefore live in AGPRs and are only ever touched
//    by the matrix cores; softmax(x) = exp(x - c)/sum exp(x - c) holds for any
//    c, so the result is the same up to rounding.
//  * Decode: one workgroup of 4 wavefronts x 16 heads (v_mfma 16x16x32) per
//    (sequence, KV head, key split) writes fp32 partials (m, l, O/l) to the
//    workspace; a second, fully parallel kernel merges them in split order,
//    so the result is deterministic.
#include <algorithm>

#include "hca_internal.h"

#define HCA_GLOBAL __attribute__((address_space(1)))

namespace hca {
namespace {

constexpr int D = 512;           // head dim of this path
constexpr int G = 64;            // query heads per KV head
constexpr int NT = 32;           // keys per tile
constexpr int KSTR = 1040;       // LDS bytes per K row (1024 + 16 pad)
constexpr int VSTR = 1088;       // LDS bytes per V row (1024 + 64 pad)
constexpr int DSTEPS = D / 16;   // k-steps of the score product
constexpr int CTILES = D / 32;   // 32-column tiles of the output
constexpr float kHeadroom = 32.f;  // max growth over the reference, log2 units

// Workgroups whose key list is at most this long carry softmax weights as
// two bf16 terms.
constexpr int kTwoTermKeys = 64;

// Softmax schedule of one pass over the key tiles.
enum Mode { kLazy = 0, kMaxOnly = 1, kFixed = 2 };

// Where the keys of one workgroup come from.  Slot kappa < nc is compressed
// entry kappa of the sequence; slot kappa >= nc is raw position
// lo + (kappa - nc), stored at that row of raw_k/raw_v, or at row
// (lo + kappa - nc) % ring when ring > 0 (decode ring buffer).
struct KeySource {
  const char* comp_k;
  const char* comp_v;
  const char* raw_k;
  const char* raw_v;
  size_t rstride;  // bytes between consecutive rows (Hkv * D * 2)
  int nc, nkeys, ring;
  int raw0;        // row of the oldest raw key: lo, or lo % ring in a ring
};

// Which slots a row (one query position t) may see: compressed slots
// [0, nvis_c) and raw slots [r0, r1] (its window; r1 <= nkeys - 1).  nc and
// nkeys describe the workgroup's whole key list.
struct RowMask {
  int nc, nkeys, nvis_c, r0, r1;
  __device__ __forceinline__ bool valid(int kappa) const {
    return kappa < nvis_c || (unsigned)(kappa - r0) <= (unsigned)(r1 - r0);
  }
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Two floats to one dword of two bf16 (round to nearest even), first in the
// low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack2_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float bf16_lo(unsigned p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16_hi(unsigned p) { return __builtin_bit_cast(float, p & 0xffff0000u); }
// acc + both bf16 halves of p, exactly as the matrix core will see them
__device__ __forceinline__ float sum2_bf16(unsigned p, float acc) {
  const bf16x2 one = {(bf16)1.f, (bf16)1.f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
}
// max over lanes l and l^32 (v_permlane32_swap: no LDS round trip)
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
// max over lanes l and l^16
__device__ __forceinline__ float max_xor16(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Issue the direct global->LDS loads of key tile `tile`: NW wavefronts share
// the 32 K rows and 32 V rows; one instruction moves one 1 KiB row.  The row
// of slot kappa is base + kappa * rstride, where base is one of three
// pointers (compressed entries, raw rows, raw rows one ring length back); no
// per-row modulo is needed.
template <int NW>
__device__ __forceinline__ void issue_tile(const KeySource& ks, int tile, char HCA_LDS* kbuf,
                                           char HCA_LDS* vbuf, int wave, int lane) {
  constexpr int RPW = NT / NW;
  const ptrdiff_t rs = (ptrdiff_t)ks.rstride;
  const ptrdiff_t raw_shift = (ptrdiff_t)(ks.raw0 - ks.nc) * rs;  // raw slot kappa -> row raw0 + kappa - nc
  const ptrdiff_t wrap_shift = raw_shift - (ptrdiff_t)ks.ring * rs;
  const int wrap_from = ks.ring ? ks.nc - ks.raw0 + ks.ring : 0x7fffffff;  // first slot past the ring end
  const int a0 = tile * NT;
  const int kk0 = wave * RPW;
  // Common case: all 32 slots lie in one region and inside the key list, so
  // the rows are consecutive from one uniform base and each load only adds
  // a constant multiple of the row stride.
  const bool inside = a0 + NT <= ks.nkeys;
  const bool all_comp = a0 + NT <= ks.nc;
  const bool all_raw = a0 >= ks.nc && (a0 + NT <= wrap_from || a0 >= wrap_from);
  if (inside && (all_comp || all_raw)) {
    const ptrdiff_t shift = all_comp ? 0 : (a0 >= wrap_from ? wrap_shift : raw_shift);
    const ptrdiff_t first = (ptrdiff_t)(a0 + kk0) * rs + shift;
    const char* kb = (all_comp ? ks.comp_k : ks.raw_k) + first;
    const char* vb = (all_comp ? ks.comp_v : ks.raw_v) + first;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      __builtin_amdgcn_global_load_lds((const void HCA_GLOBAL*)(kb + r * rs + lane * 16),
                                       (void HCA_LDS*)(kbuf + (kk0 + r) * KSTR), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void HCA_GLOBAL*)(vb + r * rs + lane * 16),
                                       (void HCA_LDS*)(vbuf + (kk0 + r) * VSTR), 16, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int kk = kk0 + r;
    // slots past the end re-read the last key (finite data; masked later)
    const int kappa = min(a0 + kk, ks.nkeys - 1);
    const bool comp = kappa < ks.nc;
    const ptrdiff_t shift = comp ? 0 : (kappa >= wrap_from ? wrap_shift : raw_shift);
    const ptrdiff_t off = (ptrdiff_t)kappa * rs + shift + lane * 16;
    const char* ksrc = (comp ? ks.comp_k : ks.raw_k) + off;
    const char* vsrc = (comp ? ks.comp_v : ks.raw_v) + off;
    __builtin_amdgcn_global_load_lds((const void HCA_GLOBAL*)ksrc, (void HCA_LDS*)(kbuf + kk * KSTR),
                                     16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void HCA_GLOBAL*)vsrc, (void HCA_LDS*)(vbuf + kk * VSTR),
                                     16, 0, 0);
  }
}

// Copy `rows` rows of 1 KiB (consecutive in global memory) into LDS rows of
// KSTR bytes with direct loads, one row per wave instruction, and wait for
// them.  Used to bring a wavefront's query rows in with whole-row requests.
__device__ __forceinline__ void stage_rows(const char* src, char HCA_LDS* dst, int rows, int lane) {
  for (int r = 0; r < rows; ++r)
    __builtin_amdgcn_global_load_lds((const void HCA_GLOBAL*)(src + (size_t)r * D * sizeof(bf16) + lane * 16),
                                     (void HCA_LDS*)(dst + r * KSTR), 16, 0, 0);
  wait_vm_all();
}

// Softmax state of the 32 rows a wavefront owns (one row per lane pair
// l, l^32; both lanes of a pair hold the same m and a partial l).
struct Acc {
  f32x16 o[CTILES];  // O^T: lane l holds row l%32, cols 32ct + 8(i/4) + 4(l/32) + i%4
  float m, l;
};

__device__ __forceinline__ bf16x8 lds_k_frag(const char HCA_LDS* p) {
  return *(const bf16x8 HCA_LDS*)p;
}

// A fragment of V^T for one (32-column tile, 16-key step): two transposed
// 8-byte reads, keys {16k2 + 4h + j} and {16k2 + 8 + 4h + j}, j < 4.
__device__ __forceinline__ bf16x8 lds_v_frag(const char HCA_LDS* base) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)base);
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)(base + 8 * VSTR));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A fragment of V^T for one 16-column tile of the 16x16x32 product: keys
// {4g + j} and {16 + 4g + j}, j < 4, g = l/16.
__device__ __forceinline__ bf16x8 lds_v_frag16(const char HCA_LDS* base) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)base);
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 HCA_LDS*)(base + 16 * VSTR));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One key tile.  kLazy: scores, reference max fixed at the row's first
// visible key, weights and P.V; returns true (for the whole wave) if a score
// exceeded the reference by more than kHeadroom.  kMaxOnly: scores and row
// max only.  kFixed: like kLazy with m already exact.  `masked` (uniform)
// applies the per-row visibility test to every slot of the tile.  With
// `two_term` (uniform) the weights enter the P.V product as the sum of two
// bf16 numbers, P = hi + lo, lo = bf16(P - hi), which carries P to ~2^-16
// relative instead of 2^-9: rows that see only a few keys have few, large
// weights whose rounding does not average out.
template <int MODE>
__device__ __forceinline__ bool compute_tile(const char HCA_LDS* kbuf, const char HCA_LDS* vbuf,
                                             const bf16x8 (&qf)[DSTEPS], Acc& st, float sc2,
                                             int lane, int koff, int voff, const RowMask& rm,
                                             int tile, bool masked, bool two_term) {
  // S^T = K . Q^T: 32 k-steps split over two independent accumulator chains
  // (a single dependent chain runs the matrix core at ~60% with one wave per
  // SIMD).  The chains are issued as inline MFMAs with VGPR accumulators so
  // that the 256 AGPRs stay with O; K fragments are read KPF steps ahead.
  constexpr int KPF = 4;
  bf16x8 kf[KPF];
#pragma unroll
  for (int k = 0; k < KPF; ++k) kf[k] = lds_k_frag(kbuf + koff + k * 32);
  f32x16 s0, s1;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s0) : "v"(kf[0]), "v"(qf[0]));
  kf[0] = lds_k_frag(kbuf + koff + KPF * 32);
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s1) : "v"(kf[1]), "v"(qf[1]));
  kf[1] = lds_k_frag(kbuf + koff + (KPF + 1) * 32);
#pragma unroll
  for (int k = 2; k < DSTEPS; ++k) {
    if (k & 1)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s1) : "v"(kf[k % KPF]), "v"(qf[k]));
    else
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s0) : "v"(kf[k % KPF]), "v"(qf[k]));
    if (k + KPF < DSTEPS) kf[k % KPF] = lds_k_frag(kbuf + koff + (k + KPF) * 32);
  }
  // a VALU read of an MFMA result needs up to 18 wait states; the compiler
  // does not see inside the inline MFMAs, so they are spent here (24)
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(s0), "+v"(s1));
  f32x16 s = s0 + s1;
  // mask, then the row max over the lane pair; scores stay unscaled until
  // the exponent (sc2 > 0, so max(sc2 * s) == sc2 * max(s) exactly)
  if (masked) {
    asm volatile("");  // keep this a branch: most tiles need no mask
    const int kk0 = tile * NT + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 16; ++i)  // accumulator i holds key slot 8(i/4) + 4(l/32) + i%4
      s[i] = rm.valid(kk0 + 8 * (i >> 2) + (i & 3)) ? s[i] : -INFINITY;
  }
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = max_xor32(mx) * sc2;
  if (MODE == kMaxOnly) {
    st.m = fmaxf(st.m, mx);
    return false;
  }
  bool over = false;
  if (MODE == kLazy) {
    if (st.m == -INFINITY) st.m = mx;  // first visible keys of the row
    over = mx > st.m + kHeadroom;
  }
  const float nm = st.m == -INFINITY ? 0.f : -st.m;  // row with no visible key yet
  float w[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) w[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sc2, nm));
  // P as packed bf16 (B operand: weights 0..7 then 8..15); l sums the
  // rounded weights, i.e. exactly what enters the product
  u32x4 ua, ub, va = {}, vb = {};
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ua[j] = pack2_bf16(w[2 * j], w[2 * j + 1]);
    ub[j] = pack2_bf16(w[8 + 2 * j], w[9 + 2 * j]);
    la = sum2_bf16(ua[j], la);
    lb = sum2_bf16(ub[j], lb);
  }
  if (two_term) {
    asm volatile("");  // a branch, not a select: only short key lists take it
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      va[j] = pack2_bf16(w[2 * j] - bf16_lo(ua[j]), w[2 * j + 1] - bf16_hi(ua[j]));
      vb[j] = pack2_bf16(w[8 + 2 * j] - bf16_lo(ub[j]), w[9 + 2 * j] - bf16_hi(ub[j]));
      la = sum2_bf16(va[j], la);
      lb = sum2_bf16(vb[j], lb);
    }
  }
  st.l += la + lb;
  const bf16x8 pa = __builtin_bit_cast(bf16x8, ua), pb = __builtin_bit_cast(bf16x8, ub);
  const bf16x8 qa = __builtin_bit_cast(bf16x8, va), qb = __builtin_bit_cast(bf16x8, vb);
  const int parts = two_term ? 2 : 1;
  for (int part = 0; part < parts; ++part) {
    const bf16x8 ba = part ? qa : pa;
    const bf16x8 bb = part ? qb : pb;
    // step u: column tile u % 16 and key step u / 16, so consecutive MFMAs
    // accumulate into different tiles; V fragments read VPF steps ahead
    constexpr int VPF = 4;
    bf16x8 vf[VPF];
#pragma unroll
    for (int u = 0; u < VPF; ++u) vf[u] = lds_v_frag(vbuf + voff + (u >> 4) * 16 * VSTR + (u & 15) * 64);
#pragma unroll
    for (int u = 0; u < 2 * CTILES; ++u) {
      const int ct = u & 15, k2 = u >> 4;
      st.o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[u % VPF], k2 ? bb : ba, st.o[ct], 0, 0, 0);
      const int un = u + VPF;
      if (un < 2 * CTILES) vf[u % VPF] = lds_v_frag(vbuf + voff + (un >> 4) * 16 * VSTR + (un & 15) * 64);
    }
  }
  return MODE == kLazy && __any(over);
}

__device__ __forceinline__ bool tile_needs_mask(int tile, int nc, int nkeys) {
  // slots that can be invisible to a row: entry nc-1 (row t0 when the second
  // position completes a block), raw slot nc (oldest window key of the later
  // row), the last slot (newest key, invisible to the earlier row) and the tail
  const int a = tile * NT, b = a + NT;
  return (a <= nc && b > nc - 1) || b >= nkeys;
}

__device__ __forceinline__ void zero_acc(Acc& st) {
#pragma unroll
  for (int ct = 0; ct < CTILES; ++ct) st.o[ct] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
}

// One pass over tiles [t_begin, t_end) in schedule MODE.  Returns true (for
// every wave) if a kLazy pass stopped because the headroom was exceeded.
// The two LDS buffers are distinct arrays and the loop is unrolled by two,
// so which buffer a read touches is known at compile time: the compiler then
// does not make LDS reads of one buffer wait for the direct loads still in
// flight into the other.  The headroom test crosses waves through flag[0]
// (tiles in buffer 0) and flag[1] (buffer 1): a tile sets its slot before the
// barrier that ends it and every wave reads the slot right after that
// barrier; the other slot can only be set before the next barrier, so no wave
// sees a flag raised for a later tile.
template <int NW, int MODE>
__device__ __forceinline__ bool tile_pass(const KeySource& ks, int t_begin, int t_end,
                                          const bf16x8 (&qf)[DSTEPS], Acc& st, float sc2,
                                          const RowMask& rm, int wave, int lane, char HCA_LDS* kv0,
                                          char HCA_LDS* kv1, int* flag, bool two_term) {
  const int koff = (lane & 31) * KSTR + (lane >> 5) * 16;
  const int voff = NT * KSTR + (4 * (lane >> 5) + ((lane & 15) >> 2)) * VSTR +
                   (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  if (MODE == kLazy && threadIdx.x == 0) flag[0] = flag[1] = 0;
  issue_tile<NW>(ks, t_begin, kv0, kv0 + NT * KSTR, wave, lane);
  wait_vm_all();
  __syncthreads();
  for (int tile = t_begin; tile < t_end; tile += 2) {
    if (tile + 1 < t_end) issue_tile<NW>(ks, tile + 1, kv1, kv1 + NT * KSTR, wave, lane);
    bool over = compute_tile<MODE>(kv0, kv0, qf, st, sc2, lane, koff, voff, rm, tile,
                                   tile_needs_mask(tile, rm.nc, rm.nkeys), two_term);
    if (MODE == kLazy && over && lane == 0) flag[0] = 1;
    wait_vm_all();
    __syncthreads();
    if (MODE == kLazy && flag[0]) return true;
    if (tile + 1 >= t_end) break;
    if (tile + 2 < t_end) issue_tile<NW>(ks, tile + 2, kv0, kv0 + NT * KSTR, wave, lane);
    over = compute_tile<MODE>(kv1, kv1, qf, st, sc2, lane, koff, voff, rm, tile + 1,
                              tile_needs_mask(tile + 1, rm.nc, rm.nkeys), two_term);
    if (MODE == kLazy && over && lane == 0) flag[1] = 1;
    wait_vm_all();
    __syncthreads();
    if (MODE == kLazy && flag[1]) return true;
  }
  return false;
}

// All tiles of [t_begin, t_end): the single-pass schedule, then, only if a
// row's scores grew past the headroom, the exact two-pass schedule.
template <int NW>
__device__ __forceinline__ void attend_tiles(const KeySource& ks, int t_begin, int t_end,
                                             const bf16x8 (&qf)[DSTEPS], Acc& st, float sc2,
                                             const RowMask& rm, int wave, int lane,
                                             char HCA_LDS* kv0, char HCA_LDS* kv1, int* flag) {
  const bool two_term = rm.nkeys <= kTwoTermKeys;
  zero_acc(st);
  if (!tile_pass<NW, kLazy>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag,
                            two_term))
    return;
  __syncthreads();
  zero_acc(st);
  tile_pass<NW, kMaxOnly>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag, two_term);
  tile_pass<NW, kFixed>(ks, t_begin, t_end, qf, st, sc2, rm, wave, lane, kv0, kv1, flag, two_term);
}

// ---------------------------------------------------------------------------
// Prefill: grid (ceil(max_seqlen/2), batch, Hkv), 256 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256, 1) void prefill_bf16_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char kv0_s[NT * KSTR + NT * VSTR];
  __shared__ __attribute__((aligned(16))) char kv1_s[NT * KSTR + NT * VSTR];
  __shared__ int flag_s[2];

  const int b = blockIdx.y, kvh = blockIdx.z;
  const int start = a.cu_seqlens[b];
  const int len = a.cu_seqlens[b + 1] - start;
  // pairs in position order: measured 3-10% faster than heaviest-first
  // (and far faster than orders that group heavy pairs on some XCDs, since
  // workgroup i runs on XCD i % 8)
  const int pair = (int)blockIdx.x;
  if (2 * pair >= len) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t0 = 2 * pair;
  const bool t1_ok = t0 + 1 < len;
  const int t_last = t1_ok ? t0 + 1 : t0;
  const int pw = wave >> 1;                 // which of the two positions
  const bool row_ok = pw == 0 || t1_ok;
  const int t = row_ok ? t0 + pw : t0;      // an absent second position recomputes t0
  const int head = kvh * G + (wave & 1) * 32 + (lane & 31);

  const int nc = (t_last + 1) / kBlock;     // entries visible to the later position
  const int lo = max(0, t0 - a.window + 1);  // oldest raw key of the earlier position
  const int nkeys = nc + (t_last - lo + 1);

  KeySource ks;
  ks.rstride = (size_t)a.hkv * D * sizeof(bf16);
  const size_t head_off = (size_t)kvh * D * sizeof(bf16);
  ks.comp_k = (const char*)a.kc + (size_t)a.cu_blocks[b] * ks.rstride + head_off;
  ks.comp_v = (const char*)a.vc + (size_t)a.cu_blocks[b] * ks.rstride + head_off;
  ks.raw_k = (const char*)a.k + (size_t)start * ks.rstride + head_off;
  ks.raw_v = (const char*)a.v + (size_t)start * ks.rstride + head_off;
  ks.nc = nc;
  ks.nkeys = nkeys;
  ks.raw0 = lo;
  ks.ring = 0;

  RowMask rm;
  rm.nc = nc;
  rm.nkeys = nkeys;
  rm.nvis_c = (t + 1) / kBlock;
  rm.r0 = nc + max(t - a.window + 1, lo) - lo;
  rm.r1 = nc + t - lo;

  // The wave's 32 query rows (heads head0 .. head0+31 of position t) are
  // contiguous: stage them through LDS with whole-row loads, then read the
  // Q^T fragments (lane l: row l%32, elements 16k + 8(l/32) .. +7).  The key
  // buffers are idle before the first tile and after the last one.
  char HCA_LDS* stage = (char HCA_LDS*)((wave >> 1) ? kv1_s : kv0_s) + (wave & 1) * 32 * KSTR;
  const int head0 = kvh * G + (wave & 1) * 32;
  const size_t qrow0 = ((size_t)(start + t) * a.hq + head0) * D;
  bf16x8 qf[DSTEPS];
  stage_rows((const char*)((const bf16*)a.q + qrow0), stage, 32, lane);
  const int qoff = (lane & 31) * KSTR + (lane >> 5) * 16;
#pragma unroll
  for (int k = 0; k < DSTEPS; ++k) qf[k] = *(const bf16x8 HCA_LDS*)(stage + qoff + k * 32);
  __syncthreads();  // every wave holds its fragments before tile 0 lands
  Acc st;
  const float sc2 = a.scale * kLog2e;
  attend_tiles<4>(ks, 0, (nkeys + NT - 1) / NT, qf, st, sc2, rm, wave, lane, (char HCA_LDS*)kv0_s,
                  (char HCA_LDS*)kv1_s, flag_s);

  // O = acc / l, rounded to bf16, written to LDS in the accumulator layout
  // (lane l: row l%32, cols 32ct + 8q + 4(l/32) .. +3) and stored row by row
  const float inv = 1.f / (st.l + __shfl_xor(st.l, 32));
  if (!row_ok) return;
  const int ooff = (lane & 31) * KSTR + (lane >> 5) * 8;
#pragma unroll
  for (int ct = 0; ct < CTILES; ++ct) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = (bf16)(st.o[ct][4 * q4 + i] * inv);
      *(bf16x4 HCA_LDS*)(stage + ooff + (32 * ct + 8 * q4) * 2) = v;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's LDS writes are done
  bf16* orow = (bf16*)a.o + qrow0;
  for (int r = 0; r < 32; ++r)
    *(bf16x8*)(orow + (size_t)r * D + lane * 8) = *(const bf16x8 HCA_LDS*)(stage + r * KSTR + lane * 16);
}

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
  issue_tile<4>(ks, t_begin, kv0, kv0 + NT * KSTR, wave, lane);
  wait_vm_all();
  __syncthreads();
  for (int tile = t_begin; tile < t_end; tile += 2) {  // two buffers, unrolled (see tile_pass)
    if (tile + 1 < t_end) issue_tile<4>(ks, tile + 1, kv1, kv1 + NT * KSTR, wave, lane);
    bool over = compute_tile16<MODE>(kv0, kv0, qf, st, sc2, lane, koff, voff, rm, tile,
                                     tile_needs_mask(tile, rm.nc, rm.nkeys), two_term);
    if (MODE == kLazy && over && lane == 0) flag[0] = 1;
    wait_vm_all();
    __syncthreads();
    if (MODE == kLazy && flag[0]) return true;
    if (tile + 1 >= t_end) break;
    if (tile + 2 < t_end) issue_tile<4>(ks, tile + 2, kv0, kv0 + NT * KSTR, wave, lane);
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
// Workspace: fp32 m and l [B*Hkv][splits][64], then fp32 O [B*Hkv][splits]
// [64][512] normalised by its own l (a convex combination of value rows).
// ---------------------------------------------------------------------------
struct WsLayout {
  float* m;
  float* l;
  float* o;
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
  w.o = (float*)p;
  return w;
}

__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(DecodeArgs a, int tps, int max_splits) {
  __shared__ __attribute__((aligned(16))) char kv0_s[NT * KSTR + NT * VSTR];
  __shared__ __attribute__((aligned(16))) char kv1_s[NT * KSTR + NT * VSTR];
  __shared__ int flag_s[2];

  const int split = blockIdx.x, b = blockIdx.y, kvh = blockIdx.z;
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
  ks.rstride = (size_t)a.hkv * D * sizeof(bf16);
  const size_t head_off = (size_t)kvh * D * sizeof(bf16);
  ks.comp_k = (const char*)a.kc + (size_t)a.cu_blocks[b] * ks.rstride + head_off;
  ks.comp_v = (const char*)a.vc + (size_t)a.cu_blocks[b] * ks.rstride + head_off;
  ks.raw_k = (const char*)a.kw + (size_t)b * a.ring * ks.rstride + head_off;
  ks.raw_v = (const char*)a.vw + (size_t)b * a.ring * ks.rstride + head_off;
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
  const float inv = 1.f / l_tot;
  float* po = w.o + prow * D + 4 * (lane >> 4);
#pragma unroll
  for (int ct = 0; ct < CTILES16; ++ct) *(f32x4*)(po + 16 * ct) = st.o[ct] * inv;
}

// Merge of the split partials: O = sum_s 2^(m_s - M) l_s O_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s, splits taken in order (deterministic).  One workgroup
// of 256 threads merges kMergeRows heads of one (sequence, KV head); each
// thread owns 8 columns of one head and issues its split loads independently.
constexpr int kMergeRows = 4;

__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int tps, int max_splits) {
  const int unit = blockIdx.y;  // b * Hkv + kvh
  const int b = unit / a.hkv, kvh = unit % a.hkv;
  const int r = blockIdx.x * kMergeRows + (threadIdx.x >> 6);  // head within the KV group
  const int c = (threadIdx.x & 63) * 8;
  const int L = a.seqlens[b];
  const int nkeys = L / kBlock + min(a.window, L);
  const int nsplit = ((nkeys + NT - 1) / NT + tps - 1) / tps;
  const WsLayout w = ws_layout(a.ws, a.batch, a.hkv, max_splits);
  const float* mrow = w.m + (size_t)unit * max_splits * G + r;
  const float* lrow = w.l + (size_t)unit * max_splits * G + r;
  const float* orow = w.o + ((size_t)unit * max_splits * G + r) * D + c;
  float M = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) M = fmaxf(M, mrow[sp * G]);
  float den = 0.f;
  f32x4 n0 = {}, n1 = {};
#pragma unroll 4
  for (int sp = 0; sp < nsplit; ++sp) {
    const float wgt = __builtin_amdgcn_exp2f(mrow[sp * G] - M) * lrow[sp * G];
    den += wgt;
    const float* op = orow + (size_t)sp * G * D;
    n0 += wgt * *(const f32x4*)op;
    n1 += wgt * *(const f32x4*)(op + 4);
  }
  const float rden = 1.f / den;
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (bf16)(n0[i] * rden);
    v[4 + i] = (bf16)(n1[i] * rden);
  }
  *(bf16x8*)((bf16*)a.o + ((size_t)b * a.hq + kvh * G + r) * D + c) = v;
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.max_seqlen + 1) / 2), a.batch, a.hkv);
  prefill_bf16_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

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
         units * p.max_splits * G * D * sizeof(float);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  const DecodePlan p = decode_plan(a.batch, a.hkv, a.max_blocks, a.window);
  decode_bf16_kernel<<<dim3(p.max_splits, a.batch, a.hkv), 256, 0, s>>>(a, p.tiles_per_split,
                                                                      p.max_splits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<<<dim3(G / kMergeRows, a.batch * a.hkv), 256, 0, s>>>(a, p.tiles_per_split,
                                                                          p.max_splits);
  return hipGetLastError();
}

}  // namespace hca
