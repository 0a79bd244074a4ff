// Projection GEMM y = x W^T + b on bf16 MFMA (gfx950): the q/k/v/o Linear
// layers around the attention calls ("Wan2.2 code walkthrough", WanModel
// snippet: nn.Linear weights are [out, in]).
//
// Both operands are read along K (x rows and W rows are K-contiguous), so the
// product is computed transposed, Y^T tile = W_tile X_tile^T, on
// v_mfma_f32_32x32x16_bf16 with W as the A operand and x as the B operand.
// In the accumulator each lane then owns one token row and runs of 4
// consecutive output features, which it stores as one 8-byte bf16 vector.
//
// Work layout:
//  * One workgroup computes a 256 (tokens) x 256 (features) tile with 8
//    wavefronts (2 along tokens x 4 along features, 128 x 64 each: 8
//    accumulator tiles of 32 x 32 per wave, two waves per SIMD).
//  * K advances in steps of 64 through a double-buffered LDS stage (x and W
//    tiles, 32 KiB each). The global loads of step k+1 are issued before the
//    MFMAs of step k and written to the other LDS buffer after them: one
//    barrier per step.
//  * Each 16-byte chunk c of tile row r is stored at chunk c ^ ((r / 2) % 8),
//    so the 16 rows read together at one logical chunk by half a wave fall
//    into 16 different 16-byte bank groups.
//  * Rows past M or N fall outside the buffer resource and read as zero;
//    chunks past K get an offset outside it and read as zero too.
//  * Tiles are walked in bands of 4 token tiles (all feature tiles of a band
//    before the next band), and workgroup ids are remapped so that each XCD
//    takes a contiguous run of the band: the band's x rows and the weight
//    tiles in flight are shared through the L2 and the last-level cache.
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int kBM = 256;                 // token rows per workgroup
constexpr int kBN = 256;                 // output features per workgroup
constexpr int kBK = 64;                  // K per LDS stage
constexpr int kThreads = 512;
constexpr int kRowBytes = kBK * 2;       // 128
constexpr int kTileBytes = kBM * kRowBytes;  // 32 KiB (x and W tiles are the same size)
constexpr int kLoads = kTileBytes / 16 / kThreads;  // 16-byte loads per thread per tile: 4
constexpr int kGroupM = 4;               // token tiles per band
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ int chunk_phys(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ bf16x8 lds_read16(const char* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * kTileBytes];
  char* const Ws = smem;                    // W tiles, buffers 0 and 1
  char* const Xs = smem + 2 * kTileBytes;   // x tiles, buffers 0 and 1

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;       // token half: rows 128 wm ..
  const int wn = wave >> 1;      // feature quarter: 64 wn ..
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  const int nM = (a.M + kBM - 1) / kBM;
  const int nN = (a.N + kBN - 1) / kBN;
  const uint32_t t = xcd_remap(blockIdx.x, (uint32_t)nM * nN);
  const int band = t / (kGroupM * nN);
  const int in_band = t % (kGroupM * nN);
  const int band_m = min(kGroupM, nM - band * kGroupM);
  const int m0 = (band * kGroupM + in_band % band_m) * kBM;
  const int n0 = (in_band / band_m) * kBN;

  const uint32_t row_x = (uint32_t)a.ld_x * 2, row_w = (uint32_t)a.ld_w * 2;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint16_t*>(a.x) + (int64_t)m0 * a.ld_x), (short)0,
      (int)(min(kBM, a.M - m0) * row_x), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const uint16_t*>(a.w) + (int64_t)n0 * a.ld_w), (short)0,
      (int)(min(kBN, a.N - n0) * row_w), kRsrcWord3);

  // Thread tid loads chunk c = tid % 8 of tile rows tid / 8 + 64 i.
  const int lr = tid >> 3, lc = tid & 7;
  uint32_t vo_x[kLoads], vo_w[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    vo_x[i] = (lr + 64 * i) * row_x + lc * 16;
    vo_w[i] = (lr + 64 * i) * row_w + lc * 16;
  }
  const int st_off = lr * kRowBytes + (chunk_phys(lr, lc) << 4);  // + 64 i rows
  u32x4 xreg[kLoads], wreg[kLoads];
  auto load = [&](int kt) {
    const uint32_t so = (uint32_t)kt * kRowBytes;
    const uint32_t oor = (kt * kBK + lc * 8 >= a.K) ? kOutOfRange : 0u;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      xreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, vo_x[i] + oor, so, 0);
      wreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, vo_w[i] + oor, so, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      *reinterpret_cast<u32x4*>(Xs + buf * kTileBytes + st_off + i * 64 * kRowBytes) = xreg[i];
      *reinterpret_cast<u32x4*>(Ws + buf * kTileBytes + st_off + i * 64 * kRowBytes) = wreg[i];
    }
  };

  // Fragment read offsets: lane reads row (base + r32), logical chunk
  // 2 kk + hf of k-step kk; the 32-row sub-tiles are immediate offsets.
  const int sw = (r32 >> 1) & 7;
  const int xa = (wm * 128 + r32) * kRowBytes;
  const int wa = (wn * 64 + r32) * kRowBytes;
  int ch[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) ch[kk] = ((2 * kk + hf) ^ sw) << 4;

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nK = (a.K + kBK - 1) / kBK;
  load(0);
  store(0);
  __syncthreads();

  for (int kt = 0; kt < nK; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nK) load(kt + 1);
    const char* wb = Ws + buf * kTileBytes + wa;
    const char* xb = Xs + buf * kTileBytes + xa;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 wf[2], xf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) wf[i] = lds_read16(wb + ch[kk] + i * 32 * kRowBytes);
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[j] = lds_read16(xb + ch[kk] + j * 32 * kRowBytes);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nK) store(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: acc[i][j][4 g + e] is y[m][n + e] for token m = tile row
  // 128 wm + 32 j + r32 and feature n = 64 wn + 32 i + 8 g + 4 hf.
  uint16_t* const y = static_cast<uint16_t*>(a.y);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * 64 + i * 32 + g * 8 + hf * 4;
      if (n >= a.N) continue;
      f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
      if (a.bias) b = *reinterpret_cast<const f32x4*>(a.bias + n);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 128 + j * 32 + r32;
        if (m >= a.M) continue;
        f32x4 v = {acc[i][j][4 * g] + b[0], acc[i][j][4 * g + 1] + b[1],
                   acc[i][j][4 * g + 2] + b[2], acc[i][j][4 * g + 3] + b[3]};
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 o = __builtin_convertvector(v, bf16x4);
        *reinterpret_cast<u32x2*>(y + (int64_t)m * a.ld_y + n) = __builtin_bit_cast(u32x2, o);
      }
    }
  }
}

hipError_t launch_linear(const LinearArgs& a, hipStream_t s) {
  const int64_t nM = (a.M + kBM - 1) / kBM, nN = (a.N + kBN - 1) / kBN;
  const int64_t total = nM * nN;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(linear_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wan
