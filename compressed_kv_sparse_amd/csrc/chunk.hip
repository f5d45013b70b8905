// Raw-row movement for serving with a cache (release blog "ERNIE 5.5 Flash
// Base", section 2.1, HCA paragraph: a layer keeps one compressed entry per
// 128 tokens plus a short window of recent raw tokens, so the raw part of a
// sequence's cache is a ring of its last ring_cap positions).
//
//   stage_chunk_kernel: before attending a chunk of new rows at positions
//     p0 .. p0+n-1, lay out per sequence the halo (the `halo` positions
//     before p0, read from the ring) followed by the new rows, so that the
//     attention kernels see one contiguous run of raw rows per sequence.
//   ring_append_kernel: after the chunk, write its last min(n, ring_cap)
//     rows into the ring (position s -> slot s % ring_cap).
//
// Both copy whole rows (Hkv x d elements) with 16-byte vector accesses, one
// wavefront per row.  HBM-bound and small next to the attention they serve.
#include "hca_internal.h"

namespace hca {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void copy_row(char* dst, const char* src, size_t bytes, int lane) {
  for (size_t i = (size_t)lane * 16; i < bytes; i += 64 * 16)
    *(u32x4*)(dst + i) = *(const u32x4*)(src + i);
}

// Grid (ceil((halo + max_rows) / 4), B), 256 threads: wavefront w of block x
// fills staged row r = 4x + w of sequence b, i.e. position p0 - halo + r.
__global__ __launch_bounds__(256) void stage_chunk_kernel(ChunkRowsArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int start = a.cu_seqlens[b];
  const int n = a.cu_seqlens[b + 1] - start;
  if (r >= a.halo + n) return;
  const int p0 = a.pos0[b];
  const int pos = p0 - a.halo + r;
  if (pos < 0) return;  // before the sequence start: never read
  const size_t row_bytes = (size_t)a.row_elems * a.elem_bytes;
  const bool is_new = pos >= p0;
  const size_t src_row = is_new ? (size_t)start + (pos - p0) : (size_t)b * a.ring_cap + pos % a.ring_cap;
  const size_t dst_row = (size_t)start + (size_t)b * a.halo + r;
  for (int which = 0; which < 2; ++which) {
    if (!a.x[which]) continue;
    const char* src = (const char*)(is_new ? a.x[which] : a.ring[which]) + src_row * row_bytes;
    copy_row((char*)a.stage[which] + dst_row * row_bytes, src, row_bytes, lane);
  }
}

// Grid (ceil(min(max_rows, ring_cap) / 4), B), 256 threads: wavefront w of
// block x writes the (4x + w)-th of the last min(n, ring_cap) new rows.
__global__ __launch_bounds__(256) void ring_append_kernel(ChunkRowsArgs a) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int x = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int start = a.cu_seqlens[b];
  const int n = a.cu_seqlens[b + 1] - start;
  const int m = min(n, a.ring_cap);
  if (x >= m) return;
  const int i = n - m + x;           // new row index
  const int pos = a.pos0[b] + i;     // its position
  const size_t row_bytes = (size_t)a.row_elems * a.elem_bytes;
  const size_t src_row = (size_t)start + i;
  const size_t dst_row = (size_t)b * a.ring_cap + pos % a.ring_cap;
  for (int which = 0; which < 2; ++which) {
    if (!a.x[which]) continue;
    copy_row((char*)a.ring[which] + dst_row * row_bytes, (const char*)a.x[which] + src_row * row_bytes,
             row_bytes, lane);
  }
}

}  // namespace

hipError_t launch_stage_chunk(const ChunkRowsArgs& a, hipStream_t s) {
  const unsigned gx = (unsigned)((a.halo + a.max_rows + 3) / 4);
  stage_chunk_kernel<<<dim3(gx, a.batch), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_ring_append(const ChunkRowsArgs& a, hipStream_t s) {
  const int rows = a.max_rows < a.ring_cap ? a.max_rows : a.ring_cap;
  ring_append_kernel<<<dim3((unsigned)((rows + 3) / 4), a.batch), 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace hca
