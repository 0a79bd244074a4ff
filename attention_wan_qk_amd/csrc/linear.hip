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
//    tiles, 32 KiB each). The tiles of step k+1 are moved by buffer loads
//    whose destination is the LDS (no register staging), issued with the
//    MFMAs of the first two of step k's four 16-deep k-steps into the other
//    buffer; each wave waits for its own loads before the step's barrier,
//    which publishes them: one barrier per step. The two buffers are reached through restrict pointers of an
//    inlined step function, so the compiler can tell that the loads in
//    flight do not write what the step's LDS reads read, and places no wait
//    before those reads.
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
constexpr int kLoads = kTileBytes / 16 / kThreads;  // 1 KiB loads per wave per tile: 4
constexpr int kLoadGroups = 2;          // the next stage's loads go out with the first 2 k-steps
constexpr int kGroupM = 4;               // token tiles per band
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ int chunk_phys(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ bf16x8 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const lds_bf16x8*>(p);
}

// One K step: the loads of the next stage go to (xn, wn) while the MFMAs read
// the current stage (xc, wc). The four LDS pointers are restrict parameters of
// an inlined function, so the compiler knows the loads in flight do not write
// what the reads below read and needs no wait before them.
template <typename Dma, typename Mma>
__device__ __forceinline__ void k_step(int kt, bool more, const lds_char* __restrict__ xc,
                                       const lds_char* __restrict__ wc, lds_char* __restrict__ xn,
                                       lds_char* __restrict__ wn, Dma& dma, Mma& mma) {
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    if (more && kk < kLoadGroups) dma(kt + 1, xn, wn, kk);
    mma(xc, wc, kk);
    __builtin_amdgcn_sched_barrier(0);   // keep each group of loads with its k-step
  }
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void linear_kernel(LinearArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_w0[kTileBytes], smem_w1[kTileBytes],
      smem_x0[kTileBytes], smem_x1[kTileBytes];
  lds_char* const W0 = (lds_char*)smem_w0;
  lds_char* const W1 = (lds_char*)smem_w1;
  lds_char* const X0 = (lds_char*)smem_x0;
  lds_char* const X1 = (lds_char*)smem_x1;

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

  // Tile loads go straight into LDS (buffer loads with the LDS as
  // destination): load i of wave w fills tile rows 8 (4 w + i) .. +7, lane l
  // writing physical chunk l % 8 of row + l / 8, so it fetches the logical
  // chunk that belongs there.
  uint32_t vo_x[kLoads], vo_w[kLoads], lch[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    lch[i] = chunk_phys(r, lane & 7);
    vo_x[i] = r * row_x + lch[i] * 16;
    vo_w[i] = r * row_w + lch[i] * 16;
  }
  // group g < kLoadGroups issues loads i with i / (kLoads / kLoadGroups) == g;
  // group -1 issues all of them.
  auto dma = [&](int kt, lds_char* __restrict__ xd, lds_char* __restrict__ wd, int group) {
    const uint32_t so = (uint32_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      if (group >= 0 && i / (kLoads / kLoadGroups) != group) continue;
      const uint32_t oor = (kt * kBK + (int)lch[i] * 8 >= a.K) ? kOutOfRange : 0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(xd + (4 * wave + i) * 1024), 16,
                                               vo_x[i] + oor, so, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(wd + (4 * wave + i) * 1024), 16,
                                               vo_w[i] + oor, so, 0, 0);
    }
  };
  auto barrier = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Fragment read offsets: lane reads row (base + r32), logical chunk
  // 2 kk + hf of k-step kk; the 32-row sub-tiles are immediate offsets.
  const int sw = (r32 >> 1) & 7;
  const int nK = (a.K + kBK - 1) / kBK;
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

  // MFMAs of k-step kk (16 of the stage's 64 K values).
  auto mma = [&](const lds_char* __restrict__ xc, const lds_char* __restrict__ wc, int kk) {
    const lds_char* wb = wc + wa;
    const lds_char* xb = xc + xa;
    {
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
  };
  dma(0, X0, W0, -1);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  barrier();

  for (int kt = 0; kt < nK; kt += 2) {
    k_step(kt, kt + 1 < nK, X0, W0, X1, W1, dma, mma);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's tile loads have landed
    barrier();
    if (kt + 1 < nK) {
      k_step(kt + 1, kt + 2 < nK, X1, W1, X0, W0, dma, mma);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      barrier();
    }
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
