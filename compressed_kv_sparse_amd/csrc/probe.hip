// Measurement probes: what this part reaches on plain streams of work, so
// that the hot-path kernels' fractions can be read against measured ceilings
// as well as against the published ones (8 TB/s HBM, 2.5 PFLOP/s dense bf16).
// None of this is the method; the benchmark times these kernels in the same
// run as the hot path.
//
//  * stream read: every byte of a buffer read once with 16-byte
//    non-temporal loads, four in flight per thread.
//  * stream through LDS: every byte read once by direct buffer->LDS loads
//    (one 1 KiB row per wave instruction, the attention kernels' tile path),
//    48 KiB tiles with two in flight per workgroup, one workgroup per CU.
//  * matrix-core loop: v_mfma_f32_32x32x16_bf16 on register operands, four
//    independent accumulators per wavefront; one wavefront of the first
//    workgroup also reads the shader-clock and fixed-rate (100 MHz) counters
//    around its loop, which gives the clock the loop ran at.
//  * LDS reads: 16-byte reads (one 1 KiB row per instruction) or the
//    transposed 8-byte reads (ds_read_b64_tr_b16) in the lane pattern the
//    attention kernels use for V^T fragments (1088-byte rows).
#include "bf16_tiles.h"

namespace hca {
namespace {

typedef unsigned u32x4_p __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_stream_read_kernel(const u32x4_p* p, size_t n16, unsigned* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  unsigned x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4_p a = __builtin_nontemporal_load(p + i);
    const u32x4_p b = __builtin_nontemporal_load(p + i + stride);
    const u32x4_p c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4_p d = __builtin_nontemporal_load(p + i + 3 * stride);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^
         d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4_p a = __builtin_nontemporal_load(p + i);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = x;
}

// sink layout: [0, 4) clock counters of the timed wavefront (shader clock
// start/end as two 32-bit halves each would overflow; stored as floats of
// the differences: shader cycles, fixed-rate ticks), then one float per
// wavefront (the accumulators' sum, so the work is not removed).
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (bf16)(0.001f * (float)((lane + j) & 7));
    b[j] = (bf16)(0.001f * (float)((lane * 3 + j) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const bool timed = blockIdx.x == 0 && threadIdx.x < 64;
  unsigned long long t0 = 0, r0 = 0;
  if (timed) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  if (timed) {
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
    if (lane == 0) {
      sink[0] = (float)(t1 - t0);
      sink[1] = (float)(r1 - r0);
    }
  }
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) sink[4 + blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

constexpr int kDmaTile = 49152;  // bytes per tile of the LDS stream (48 rows of 1 KiB)
constexpr int kDmaDepth = 2;     // tiles in flight per workgroup

// Workgroup g streams tiles g, g + grid, ... of the buffer through
// kDmaDepth + 1 LDS slots.  Loads issued past the workgroup's last tile use
// an empty range (they read zeros without touching memory), so that every
// wait keeps the same count.
__global__ __launch_bounds__(256, 1) void probe_stream_lds_kernel(const char* src, size_t ntiles, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char buf[(kDmaDepth + 1) * kDmaTile];
  constexpr int kRows = kDmaTile / 1024 / 4;  // rows per wavefront per tile
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t grid = gridDim.x;
  const size_t mine = ntiles > blockIdx.x ? (ntiles - blockIdx.x + grid - 1) / grid : 0;
  auto issue = [&](size_t it) {
    const bool ok = it < mine;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(src) + (ok ? (blockIdx.x + it * grid) * kDmaTile : 0), (short)0, ok ? kDmaTile : 0,
        0x00020000);
    char HCA_LDS* dst = (char HCA_LDS*)buf + (it % (kDmaDepth + 1)) * kDmaTile;
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
      const int row = wave * kRows + rr;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void HCA_LDS*)(dst + row * 1024), 16, row * 1024 + lane * 16, 0,
                                               0, kStreamed);
    }
  };
#pragma unroll
  for (int it = 0; it < kDmaDepth; ++it) issue(it);
  unsigned x = 0;
  for (size_t it = 0; it < mine; ++it) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kDmaDepth - 1) * kRows) : "memory");  // tile `it` has landed
    __syncthreads();  // ... in every wavefront; the slot of tile it - 1 is free
    issue(it + kDmaDepth);
    x ^= *(const unsigned HCA_LDS*)((const char HCA_LDS*)buf + (it % (kDmaDepth + 1)) * kDmaTile + threadIdx.x * 4);
  }
  wait_vm_all();
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) sink[blockIdx.x * 4 + wave] = x;
}

constexpr int kProbeRow = 1088;            // bytes per LDS row (the V tile stride)
constexpr int kProbeRows = 32;             // one 32-key tile
constexpr int kProbeBytes = kProbeRows * kProbeRow;

__global__ __launch_bounds__(256) void probe_lds_kernel(int mode, int iters, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char buf[kProbeBytes];
  for (int o = threadIdx.x * 16; o < kProbeBytes; o += 256 * 16)
    *(u32x4_p HCA_LDS*)((char HCA_LDS*)buf + o) = u32x4_p{(unsigned)o, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  char HCA_LDS* base = (char HCA_LDS*)buf;
  unsigned x = 0;
  if (mode == 0) {
    // one 1 KiB row per instruction: lane l reads bytes 16l .. 16l+15 of row r
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const u32x4_p v = *(const u32x4_p HCA_LDS*)(base + ((r + 8 * wave + it) & 31) * kProbeRow + lane * 16);
        x ^= v[0] ^ v[3];
      }
    }
  } else {
    // V^T fragment reads: rows 4(l/32) + (l%16)/4, columns 16((l/16)%2) + 4(l%4)
    const int off = (4 * (lane >> 5) + ((lane & 15) >> 2)) * kProbeRow + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int tile = (f + 2 * wave + it) & 7;
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 HCA_LDS*)(base + off + (tile & 1) * 8 * kProbeRow + (tile >> 1) * 64));
        x ^= (unsigned)(unsigned short)v[0] ^ ((unsigned)(unsigned short)v[3] << 16);
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) sink[blockIdx.x * 4 + wave] = x;
}

}  // namespace

hipError_t launch_probe_stream_read(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t s) {
  probe_stream_read_kernel<<<grid, 256, 0, s>>>((const u32x4_p*)buf, bytes / 16, sink);
  return hipGetLastError();
}

size_t probe_stream_lds_bytes(size_t bytes) { return bytes / kDmaTile * kDmaTile; }

hipError_t launch_probe_stream_lds(const void* buf, size_t bytes, unsigned* sink, int grid, hipStream_t s) {
  probe_stream_lds_kernel<<<grid, 256, 0, s>>>((const char*)buf, bytes / kDmaTile, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int grid, float* sink, hipStream_t s) {
  probe_mfma_kernel<<<grid, 256, 0, s>>>(iters, sink);
  return hipGetLastError();
}

hipError_t launch_probe_lds(int mode, int iters, int grid, unsigned* sink, hipStream_t s) {
  probe_lds_kernel<<<grid, 256, 0, s>>>(mode, iters, sink);
  return hipGetLastError();
}

}  // namespace hca
