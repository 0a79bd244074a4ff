// Measurement aids (libwanpeak.so): the sustained bf16 MFMA rate and the
// streaming copy, read and write bandwidths of the chip, against which the library's kernels
// are also quoted. Not part of the attention path.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../../include/wanpeak.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = WANPEAK_MFMA_THREADS;
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;   // 16-byte vectors per thread: 16 KiB per workgroup
static_assert(kCopyThreads * kCopyUnroll * 16 == WANPEAK_STREAM_BLOCK_BYTES, "stream block size");

// Four independent accumulator chains per wave keep the MFMA pipe busy; two
// workgroups per CU give each SIMD two waves.
__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(const bf16x8* operands, float* out,
                                                             int iters) {
  const bf16x8 a = operands[threadIdx.x];
  const bf16x8 b = operands[kThreads + threadIdx.x];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) s += (c0[v] + c1[v]) + (c2[v] + c3[v]);
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Each workgroup copies kCopyUnroll * kCopyThreads consecutive vectors: all
// loads first, then all stores, bypassing the caches' retention policy.
__global__ __launch_bounds__(kCopyThreads) void copy_kernel(u32x4* __restrict__ dst,
                                                            const u32x4* __restrict__ src,
                                                            size_t n) {
  const size_t base = (size_t)blockIdx.x * kCopyThreads * kCopyUnroll;
  const size_t i = base + threadIdx.x;
  u32x4 v[kCopyUnroll];
  if (base + kCopyThreads * kCopyUnroll <= n) {   // every workgroup but a ragged last one
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kCopyThreads);
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * kCopyThreads);
    return;
  }
  for (int u = 0; u < kCopyUnroll; ++u)
    if (i + u * kCopyThreads < n)
      __builtin_nontemporal_store(__builtin_nontemporal_load(src + i + u * kCopyThreads),
                                  dst + i + u * kCopyThreads);
}

// Read-only stream: each thread folds its vectors into one word by XOR and
// the workgroup's XOR goes to out[blockIdx.x] (one 4-byte store per 16 KiB
// read), so the loads cannot be removed and the result can be checked.
__global__ __launch_bounds__(kCopyThreads) void read_kernel(uint32_t* __restrict__ out,
                                                            const u32x4* __restrict__ src,
                                                            size_t n) {
  __shared__ uint32_t part[kCopyThreads / 64];
  const size_t base = (size_t)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x;
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const size_t i = base + (size_t)u * kCopyThreads;
    if (i < n) {
      const u32x4 v = __builtin_nontemporal_load(src + i);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kCopyThreads / 64; ++w) r ^= part[w];
    out[blockIdx.x] = r;
  }
}

// Write-only stream: every 4-byte word of dst[0, n) set to `value`.
__global__ __launch_bounds__(kCopyThreads) void fill_kernel(u32x4* __restrict__ dst, size_t n,
                                                            uint32_t value) {
  const size_t base = (size_t)blockIdx.x * kCopyThreads * kCopyUnroll + threadIdx.x;
  const u32x4 v = {value, value, value, value};
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const size_t i = base + (size_t)u * kCopyThreads;
    if (i < n) __builtin_nontemporal_store(v, dst + i);
  }
}

}  // namespace

extern "C" {

int wanpeak_mfma_bf16_loop(const void* operands, float* out, int blocks, int iters,
                           hipStream_t stream) {
  if (!operands || !out || blocks < 1 || blocks > 65536 || iters < 1) return 1;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const bf16x8*>(operands), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int wanpeak_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src || (bytes & 15u)) return 1;
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  if ((d | s) & 15u) return 1;
  if (bytes == 0) return 0;
  if (d < s + bytes && s < d + bytes) return 1;
  const size_t n = bytes / 16;
  const size_t per_block = (size_t)kCopyThreads * kCopyUnroll;
  const size_t blocks = (n + per_block - 1) / per_block;
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int wanpeak_read(uint32_t* out, const void* src, size_t bytes, hipStream_t stream) {
  if (!out || !src || (bytes & 15u)) return 1;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return 1;
  if (bytes == 0) return 0;
  const size_t n = bytes / 16;
  const size_t blocks = (bytes + WANPEAK_STREAM_BLOCK_BYTES - 1) / WANPEAK_STREAM_BLOCK_BYTES;
  if (blocks > 0x7fffffffu) return 1;
  const uintptr_t o = reinterpret_cast<uintptr_t>(out), s = reinterpret_cast<uintptr_t>(src);
  if (o < s + bytes && s < o + blocks * 4) return 1;
  hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream, out,
                     static_cast<const u32x4*>(src), n);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int wanpeak_fill(void* dst, size_t bytes, uint32_t value, hipStream_t stream) {
  if (!dst || (bytes & 15u) || (reinterpret_cast<uintptr_t>(dst) & 15u)) return 1;
  if (bytes == 0) return 0;
  const size_t n = bytes / 16;
  const size_t blocks = (bytes + WANPEAK_STREAM_BLOCK_BYTES - 1) / WANPEAK_STREAM_BLOCK_BYTES;
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     static_cast<u32x4*>(dst), n, value);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
