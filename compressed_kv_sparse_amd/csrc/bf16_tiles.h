// Device-side building blocks shared by the bf16 attention kernels (prefill
// and decode) for 512-dim heads and 64 query heads per KV head on CDNA4
// matrix cores.  Internal to libhca.
//
// What the kernels compute (release blog "ERNIE 5.5 Flash Base", section
// 2.1, HCA paragraph; Zhidx article, section "1. Latent-Gated Sparse
// Attention"): each query attends, under one softmax scaled by 1/sqrt(d), to
// the complete compressed entries of its sequence (block j visible once
// 128(j+1) <= t+1) followed by the raw window max(0, t-W+1) .. t.  The model
// card gives the 512-dim heads; the Zhidx article the 64 query heads.
//
// Keys are processed in tiles of 32 that stream through LDS with direct
// buffer->LDS 16-byte loads (one 1 KiB key row per wave instruction).  A
// workgroup's key list is "slots": slot kappa < nc is compressed entry
// kappa, slot kappa >= nc a raw row.  K rows sit in LDS with a 1040-byte
// stride and V rows with 1088 bytes, so the 16-byte K fragment reads and
// the transposed 8-byte V reads hit distinct banks.
#pragma once

#include "hca_internal.h"

namespace hca {
namespace {

constexpr int D = 512;           // head dim of the matrix-core path
constexpr int G = 64;            // query heads per KV head
constexpr int NT = 32;           // keys per tile
constexpr int KSTR = 1040;       // LDS bytes per K row (1024 + 16 pad)
constexpr int VSTR = 1088;       // LDS bytes per V row (1024 + 64 pad)
constexpr int KTILE = NT * KSTR;  // bytes of one K tile in LDS
constexpr int VTILE = NT * VSTR;  // bytes of one V tile in LDS
constexpr float kHeadroom = 32.f;  // max score growth over the reference, log2 units

// Workgroups whose key list is at most this long carry softmax weights as
// two bf16 terms.
constexpr int kTwoTermKeys = 64;

// Softmax schedule of one pass over the key tiles.
//  kLazy: a row fixes its reference max m at the first tile where it sees a
//         key and uses exp2(s - m) from then on (weights <= 2^32 as long as
//         no later score exceeds m by more than kHeadroom); a pass that sees
//         a larger score is abandoned.
//  kMaxOnly: scores and the exact row max only.
//  kFixed: weights exp2(s - m) <= 1 with m exact.
// softmax(x) = exp(x - c) / sum exp(x - c) for any c, so every schedule gives
// the same result up to rounding; the accumulators never need rescaling.
enum Mode { kLazy = 0, kMaxOnly = 1, kFixed = 2 };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Where the keys of one workgroup come from.  Slot kappa < nc is compressed
// entry kappa of the sequence; slot kappa >= nc is raw position
// lo + (kappa - nc), stored at that row of the raw rows, or at row
// (lo + kappa - nc) % ring when ring > 0 (decode ring buffer).  The rows are
// read through buffer resources (base = the sequence's first row of the KV
// head, size = its rows): a row outside them reads as zero, never faults.
struct KeySource {
  __amdgpu_buffer_rsrc_t comp_k, comp_v, raw_k, raw_v;
  int rstride;     // bytes between consecutive rows (Hkv * D * 2)
  int nc, nkeys, ring;
  int raw0;        // row of the oldest raw key: lo, or lo % ring in a ring
};

// A buffer resource over `bytes` bytes from `base` (raw, untyped access;
// the fourth word is the gfx9 default data format).  The record size is 32
// bits: larger ranges are clamped (the host limits the rows a kernel
// addresses to offsets below 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const unsigned n = bytes > 0xffffffffull ? 0xffffffffu : (unsigned)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Which slots a row (one query position t) may see: compressed slots
// [0, nvis_c) and raw slots [r0, r1] (its window; r1 <= nkeys - 1).  nc and
// nkeys describe the workgroup's whole key list.
struct RowMask {
  int nc, nkeys, nvis_c, r0, r1;
  __device__ __forceinline__ bool valid(int kappa) const {
    return kappa < nvis_c || (unsigned)(kappa - r0) <= (unsigned)(r1 - r0);
  }
};

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

// Issue the direct global->LDS loads of key tile `tile` (K rows into kbuf
// when DO_K, V rows into vbuf when DO_V): NW wavefronts share the 32 rows;
// one instruction moves one 1 KiB row (lane l: bytes 16l .. 16l+15).  The
// row of slot kappa is a compressed entry, a raw row, or a raw row one ring
// length back; slots past the end re-read the last key (finite data, masked
// later).  Buffer loads rather than global ones: with a global->LDS load in
// flight the compiler waits for every outstanding LDS read before each use
// of one, which would serialise the fragment reads of the tile math.
// CPOL is the loads' cache policy: 0, or kStreamed for rows that no other
// workgroup reads again (the non-temporal hint keeps them from displacing
// reused lines in L2).
constexpr int kStreamed = 2;  // cache-policy bit of a non-temporal load
template <int NW, bool DO_K = true, bool DO_V = true, int CPOL = 0>
__device__ __forceinline__ void issue_tile(const KeySource& ks, int tile, char HCA_LDS* kbuf,
                                           char HCA_LDS* vbuf, int wave, int lane) {
  constexpr int RPW = NT / NW;
  const int rs = ks.rstride;
  const int wrap_from = ks.ring ? ks.nc - ks.raw0 + ks.ring : 0x7fffffff;  // first slot past the ring end
  const int a0 = tile * NT;
  const int kk0 = wave * RPW;
  const int vo = lane * 16;
  // Common case: all 32 slots lie in one region and inside the key list, so
  // the rows are consecutive from one uniform first row.
  const bool inside = a0 + NT <= ks.nkeys;
  const bool all_comp = a0 + NT <= ks.nc;
  const bool all_raw = a0 >= ks.nc && (a0 + NT <= wrap_from || a0 >= wrap_from);
  if (inside && (all_comp || all_raw)) {
    const int row0 = all_comp ? a0 + kk0 : a0 + kk0 - ks.nc + ks.raw0 - (a0 >= wrap_from ? ks.ring : 0);
    const __amdgpu_buffer_rsrc_t rk = all_comp ? ks.comp_k : ks.raw_k;
    const __amdgpu_buffer_rsrc_t rv = all_comp ? ks.comp_v : ks.raw_v;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      // the row offset goes into the lane offset: the range check covers it
      const int off = (row0 + r) * rs + vo;
      if (DO_K)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (void HCA_LDS*)(kbuf + (kk0 + r) * KSTR), 16, off, 0, 0, CPOL);
      if (DO_V)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (void HCA_LDS*)(vbuf + (kk0 + r) * VSTR), 16, off, 0, 0, CPOL);
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int kk = kk0 + r;
    const int kappa = min(a0 + kk, ks.nkeys - 1);
    const bool comp = kappa < ks.nc;
    const int row = comp ? kappa : kappa - ks.nc + ks.raw0 - (kappa >= wrap_from ? ks.ring : 0);
    const int off = row * rs + vo;
    if (DO_K)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(comp ? ks.comp_k : ks.raw_k, (void HCA_LDS*)(kbuf + kk * KSTR), 16,
                                               off, 0, 0, CPOL);
    if (DO_V)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(comp ? ks.comp_v : ks.raw_v, (void HCA_LDS*)(vbuf + kk * VSTR), 16,
                                               off, 0, 0, CPOL);
  }
}

__device__ __forceinline__ bf16x8 lds_k_frag(const char HCA_LDS* p) {
  return *(const bf16x8 HCA_LDS*)p;
}

// A fragment of V^T for one (32-column tile, 16-key step) of the 32x32x16
// product: two transposed 8-byte reads, keys {16k2 + 4h + j} and
// {16k2 + 8 + 4h + j}, j < 4, h = l/32.
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

__device__ __forceinline__ bool tile_needs_mask(int tile, int nc, int nkeys) {
  // slots that can be invisible to a row: entry nc-1 (row t0 when the second
  // position completes a block), raw slot nc (oldest window key of the later
  // row), the last slot (newest key, invisible to the earlier row) and the tail
  const int a = tile * NT, b = a + NT;
  return (a <= nc && b > nc - 1) || b >= nkeys;
}

}  // namespace
}  // namespace hca
