// Internal declarations shared by the HIP translation units of libhca.
// Not part of the public ABI (include/hca.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hca {

// Tokens pooled into one compressed entry (release blog, section 2.1, HCA
// paragraph: one cached entry per 128 tokens).
constexpr int kBlock = 128;

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define HCA_LDS __attribute__((address_space(3)))

// log2(e): exp(x) == exp2(x * log2(e)); folded into the score scale so the
// softmax runs on the hardware base-2 exponential.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// float -> bf16 conversion rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Element type for a dtype code.
template <int DT> struct dtype_of;
template <> struct dtype_of<0> { typedef float type; };
template <> struct dtype_of<1> { typedef bf16 type; };

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files, called from hca_api.hip after the
// arguments were validated).  All return the hipError_t of the launch.
// ---------------------------------------------------------------------------
struct CompressArgs {
  int batch, total_blocks, hkv, d;
  const int* cu_seqlens;
  const int* cu_blocks;
  const void* x[2];  // K, V (x[1] may be null)
  void* xc[2];       // Kc, Vc
  const float* w;
  // chunk mode only: position of each sequence's first new row, the raw
  // rings [B, ring_cap, Hkv, d] and the most blocks one sequence completes
  const int* pos0;
  const void* ring[2];
  int ring_cap, max_new;
};
hipError_t launch_compress(int dtype, const CompressArgs& a, hipStream_t s);
hipError_t launch_compress_chunk(int dtype, const CompressArgs& a, hipStream_t s);

struct PrefillArgs {
  int batch, max_seqlen, hq, hkv, d, window;
  float scale;
  const int* cu_seqlens;
  const int* cu_blocks;
  const void* q;
  const void* k;
  const void* v;
  const void* kc;
  const void* vc;
  void* o;
  // Chunks of longer sequences: query row i of sequence b sits at position
  // pos0[b] + i (pos0 NULL: 0).  The raw rows of sequence b start at row
  // cu_seqlens[b] + b * halo of k / v and hold positions pos0[b] - halo
  // onward (halo raw rows precede each chunk; 0 for whole sequences).
  const int* pos0;
  int halo;
  // Optional epilogue (bf16 path): per-head gate logits [N, Hq] fp32 and a
  // cross-head low-rank mixing U, V [Hkv, 64, mix_rank] fp32, mix_rank <= 32
  // (NULL: none).
  const float* gate;
  const float* mix_u;
  const float* mix_v;
  int mix_rank;
  // Optional (bf16 path): per-row log-sum-exp of the scaled scores [N, Hq]
  // fp32, natural log, for the backward (NULL: not written).
  float* lse;
};
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);

// Chunk support (chunk.hip).  Rows: cu_seqlens [B+1] counts the new rows
// of each sequence, pos0 [B] their first position; rings [B, ring_cap, Hkv,
// d] hold position s in slot s % ring_cap.
struct ChunkRowsArgs {
  int batch, max_rows, row_elems, elem_bytes, ring_cap, halo;
  const int* cu_seqlens;
  const int* pos0;
  const void* x[2];   // new K, V rows [N, Hkv, d]
  void* ring[2];      // raw rings (read by the staging copy, written by the append)
  void* stage[2];     // staged K, V rows (see PrefillArgs)
};
// Copy the halo rows (from the rings) and the new rows of every sequence
// into the staging buffers.
hipError_t launch_stage_chunk(const ChunkRowsArgs& a, hipStream_t s);
// Write the last min(n, ring_cap) new rows of every sequence into its ring.
hipError_t launch_ring_append(const ChunkRowsArgs& a, hipStream_t s);

struct DecodeArgs {
  int batch, max_blocks, hq, hkv, d, window, ring;
  float scale;
  const int* seqlens;
  const int* cu_blocks;
  const void* q;
  const void* kc;
  const void* vc;
  const void* kw;
  const void* vw;
  void* o;
  void* ws;
  // Optional epilogue (bf16 path), as in PrefillArgs: gate logits [B, Hq]
  // fp32, mixing U, V [Hkv, 64, mix_rank] fp32 (NULL: none).
  const float* gate;
  const float* mix_u;
  const float* mix_v;
  int mix_rank;
};
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// Split plan of the bf16 decode kernel: tiles of 32 keys, `tiles_per_split`
// tiles per workgroup, `max_splits` workgroups per (sequence, KV head).
struct DecodePlan {
  int tiles_per_split;
  int max_splits;
};
DecodePlan decode_plan(int batch, int hkv, int max_blocks, int window);
size_t decode_workspace_bytes_bf16(int batch, int hkv, int max_blocks, int window);

// Backward of the bf16 prefill (backward_bf16.hip).  Inputs as in the
// forward plus the pooling logits w [Hkv, 128], the forward output o, its
// lse [N, Hq] and dout [N, Hq, d]; outputs dq [N, Hq, d], dk, dv [N, Hkv, d]
// (bf16) and dw [Hkv, 128] (fp32).  The workspace pointers below ws are
// carved by the launcher.
struct BackwardArgs {
  int batch, max_seqlen, total_tokens, total_blocks, hq, hkv, d, window;
  float scale;
  const int* cu_seqlens;
  const int* cu_blocks;
  const void* q;
  const void* k;
  const void* v;
  const void* kc;
  const void* vc;
  const void* o;
  const void* dout;
  const float* w;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dw;
  void* ws;
  // set by the launcher
  float* delta;    // dO . O per row [N, Hq]
  float* part_k;   // per-item partials of the key gradients [B, Hkv, items, 64, d]
  float* part_v;
  float* gbuf;     // per entry terms of the pooling-logit gradient [total_blocks, Hkv, 128]
};
// Work split of the dK/dV kernel: raw tiles of 64 rows, each over nsr runs
// of prr positions; compressed tiles of 64 entries, each over nsc runs of
// pch positions; items = raw_tiles * nsr + comp_tiles * nsc.
struct BackwardPlan {
  int raw_tiles, nsr, prr, comp_tiles, nsc, pch, items;
};
BackwardPlan backward_plan(int batch, int hkv, int max_seqlen, int window);
size_t backward_workspace_bytes(int batch, int hq, int hkv, int total_tokens, int total_blocks, int max_seqlen,
                                int window);
hipError_t launch_backward_bf16(BackwardArgs a, hipStream_t s);

// Sparse-attention decode of the full-context layers (dsa.hip): 64 query
// heads and one shared key/value head of width 256, an int8 indexer of
// width 128.  Sequence b has seqlens[b] cached rows starting at row
// cu_rows[b] of k, v [rows, 256] and ki [rows, 128]; its query sits at the
// last position.  The workspace pointers below ws are carved by the launcher.
struct DsaArgs {
  int batch, max_seqlen, topk;
  float scale;
  const int* seqlens;
  const int* cu_rows;
  const void* q;           // [B, 64, 256] bf16
  const signed char* qi;   // [B, 128]
  const void* k;
  const void* v;
  const signed char* ki;
  void* o;                 // [B, 64, 256] bf16
  int* sel;                // [B, topk] selected positions, increasing, -1 padded
  void* ws;
  // set by the launcher
  unsigned* keys;          // [B, max_seqlen] score + 2^21
  unsigned* hist;          // [B, 2049] histogram of key >> 11
  unsigned* lohist;        // [B, 2048] histogram of key & 2047 inside the selected hi bin
  unsigned* chunk_cnt;     // [B, chunks, 2] keys above the threshold, ties at it
  unsigned* thr;           // [B, 2] threshold key, ties to take
  float* part_m;           // [B, nsplit, 64]
  float* part_l;
  bf16* part_o;            // [B, nsplit, 64, 256]
};
size_t dsa_workspace_bytes(int batch, int max_seqlen, int topk);
hipError_t launch_dsa_decode(DsaArgs a, hipStream_t s);

// Measurement probes (probe.hip): a streaming read of `bytes` bytes, a
// matrix-core loop and LDS read loops (mode 0: 16-byte reads, 1: transposed
// 8-byte reads).  Each writes 4 values per workgroup to `sink` (the MFMA
// probe first writes its clock readings to sink[0..3]).
hipError_t launch_probe_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t s);
// The LDS stream reads whole 48 KiB tiles: the bytes it reads of `bytes`.
size_t probe_stream_lds_bytes(size_t bytes);
hipError_t launch_probe_stream_lds(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t s);
hipError_t launch_probe_mfma(int iters, int grid, float* sink, hipStream_t s);
hipError_t launch_probe_lds(int mode, int iters, int grid, unsigned* sink, hipStream_t s);

}  // namespace hca
