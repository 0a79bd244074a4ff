// Projection GEMM y = x W^T + b on bf16 MFMA (gfx950): the q/k/v/o Linear
// layers around the attention calls ("Wan2.2 code walkthrough", WanModel
// snippet: nn.Linear weights are [out, in]).
//
// Both operands are read along K (x rows and W rows are K-contiguous), so the
// product is computed transposed, Y^T tile = W_tile X_tile^T, on
// v_mfma_f32_16x16x32_bf16 with W as the A operand and x as the B operand
// (in a pure loop this MFMA sustains ~12% more than v_mfma_f32_32x32x16_bf16
// on gfx950). In the accumulator each lane then owns one token row and runs
// of 4 consecutive output features.
//
// Work layout:
//  * One workgroup computes a 256 (tokens) x 256 (features) tile with 8
//    wavefronts (2 along tokens x 4 along features, 128 x 64 each: 32
//    accumulator tiles of 16 x 16 per wave, two waves per SIMD).
//  * K advances in steps of 64 through a double-buffered LDS stage (x and W
//    tiles, 32 KiB each). The tiles of step k+1 are moved into the other
//    buffer by buffer loads whose destination is the LDS (no register
//    staging); each wave waits for its own loads before the step's barrier,
//    which publishes them: one barrier per step. A wave stalls while its
//    loads queue for the compute unit's load path (~64 bytes per cycle), so
//    waves 0-3 issue theirs before the step's first 32-deep k-step and waves
//    4-7 before its second: the two waves of each SIMD stall at different
//    times and the MFMA pipe keeps running on the other one. The two
//    buffers are reached through restrict pointers of an inlined step
//    function, so the compiler can tell that the loads in flight do not write
//    what the step's LDS reads read, and places no wait before those reads.
//  * Inside a k-step the LDS operand reads run a few fragments ahead of the
//    MFMAs that use them (scheduling groups), instead of all before the first.
//  * Each 16-byte chunk c of tile row r is stored at chunk c ^ ((r / 2) % 8),
//    so the 16 rows read together at one logical chunk by a quarter of a
//    wave fall into 16 different 16-byte bank groups.
//  * The finished 256 x 256 tile goes out through the LDS (see the epilogue):
//    whole 128-byte row segments per store.
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
constexpr int kGroupM = 4;               // token tiles per band
constexpr int kReadAhead = 7;            // LDS fragment reads issued ahead of the MFMAs
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ int chunk_phys(int r, int c) { return c ^ ((r >> 1) & 7); }

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ bf16x8 lds_read16(const lds_char* p) {
  return *reinterpret_cast<const lds_bf16x8*>(p);
}

// One K step: the loads of the next stage go to (xn, wn) while the MFMAs read
// the current stage (xc, wc); this wave issues them before k-step lg. The four
// LDS pointers are restrict parameters of
// an inlined function, so the compiler knows the loads in flight do not write
// what the reads below read and needs no wait before them.
template <typename Dma, typename Mma>
__device__ __forceinline__ void k_step(int kt, bool more, int lg, const lds_char* __restrict__ xc,
                                       const lds_char* __restrict__ wc, lds_char* __restrict__ xn,
                                       lds_char* __restrict__ wn, Dma& dma, Mma& mma) {
#pragma unroll
  for (int kk = 0; kk < kBK / 32; ++kk) {
    if (more && kk == lg) dma(kt + 1, xn, wn);
    mma(xc, wc, kk);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads with their k-step
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
  auto dma = [&](int kt, lds_char* __restrict__ xd, lds_char* __restrict__ wd) {
    const uint32_t so = (uint32_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
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

  // Fragment read offsets (v_mfma_f32_16x16x32_bf16): lane l reads row
  // (base + l % 16), logical chunk 4 kk + l / 16 of k-step kk (32 of the
  // stage's K values); the 16-row sub-tiles are immediate offsets, and the
  // swizzle of a row depends only on its index within 16.
  const int r16 = lane & 15, q4 = lane >> 4;
  const int sw = (r16 >> 1) & 7;
  const int nK = (a.K + kBK - 1) / kBK;
  const int xa = (wm * 128 + r16) * kRowBytes;
  const int wa = (wn * 64 + r16) * kRowBytes;
  int ch[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) ch[kk] = ((4 * kk + q4) ^ sw) << 4;

  // acc[f][t][e]: feature 16 f + 4 q4 + e, token 16 t + r16 of the wave's block
  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[i][j][v] = 0.0f;

  // MFMAs of k-step kk (32 of the stage's 64 K values). The 12 fragments are
  // read in the order the MFMAs first use them (W row block 0, the 8 x row
  // blocks, W row blocks 1-3), kReadAhead of them before the first MFMA and
  // then one after each MFMA, so that an MFMA waits only for its own operands
  // (all 12 reads before the first MFMA made every k-step wait for the last).
  auto mma = [&](const lds_char* __restrict__ xc, const lds_char* __restrict__ wc, int kk) {
    const lds_char* wb = wc + wa;
    const lds_char* xb = xc + xa;
    bf16x8 wf[4], xf[8];
    wf[0] = lds_read16(wb + ch[kk]);
#pragma unroll
    for (int j = 0; j < 8; ++j) xf[j] = lds_read16(xb + ch[kk] + j * 16 * kRowBytes);
#pragma unroll
    for (int i = 1; i < 4; ++i) wf[i] = lds_read16(wb + ch[kk] + i * 16 * kRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, kReadAhead, 0);
#pragma unroll
    for (int r = 0; r < 12 - kReadAhead; ++r) {
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 32 - (12 - kReadAhead), 0);
  };
  dma(0, X0, W0);
  // Wait for everything here, the kernel-argument scalar loads included: with
  // one of them possibly in flight at the loop head (scalar loads complete out
  // of order), the compiler's first operand wait of every k-step would be for
  // all LDS reads, not just the first MFMA's.
  __builtin_amdgcn_s_waitcnt(0);
  barrier();

  // Waves 0-3 issue a stage's loads before its first k-step, waves 4-7 before
  // its second: the two waves of a SIMD stall on load issue at different
  // times, and the other one keeps the MFMA pipe busy meanwhile.
  const int lg = __builtin_amdgcn_readfirstlane(wave) >> 2;
  for (int kt = 0; kt < nK; kt += 2) {
    k_step(kt, kt + 1 < nK, lg, X0, W0, X1, W1, dma, mma);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // this wave's tile loads have landed
    barrier();
    if (kt + 1 < nK) {
      k_step(kt + 1, kt + 2 < nK, lg, X1, W1, X0, W0, dma, mma);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      barrier();
    }
  }

  // Epilogue: acc[i][j][e] is y[m][n + e] for token m = tile row
  // 128 wm + 16 j + r16 and feature n = 64 wn + 16 i + 4 q4. Each wave
  // stages its 128 x 64 block (bias added, bf16) in the LDS array of its
  // feature quarter (the K loop ended with a barrier, so every stage is free)
  // and stores it back as whole 128-byte row segments: written from the
  // registers directly, each store covered 32 rows with 16 bytes, and the
  // partial lines cost about three times the output's bytes in HBM writes.
  // Row r of a quarter keeps 16-byte chunk c at c ^ (r % 8).
  lds_char* const stage = wn == 0 ? W0 : wn == 1 ? W1 : wn == 2 ? X0 : X1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nq = i * 16 + q4 * 4;   // feature inside the quarter
    const int n = n0 + wn * 64 + nq;
    f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
    if (a.bias && n < a.N) b = *reinterpret_cast<const f32x4*>(a.bias + n);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = wm * 128 + j * 16 + r16;
      f32x4 v = acc[i][j] + b;
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      const bf16x4 o = __builtin_convertvector(v, bf16x4);
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
          stage + r * kRowBytes + (((nq >> 3) ^ (r & 7)) << 4) + 8 * ((nq >> 2) & 1)) =
          __builtin_bit_cast(u32x2, o);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's block is staged
  uint16_t* const y = static_cast<uint16_t*>(a.y);
  const int c = lane & 7;
  const int n = n0 + wn * 64 + c * 8;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = wm * 128 + k * 8 + (lane >> 3);
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        stage + r * kRowBytes + ((c ^ (r & 7)) << 4));
    const int m = m0 + r;
    if (m < a.M && n < a.N) *reinterpret_cast<u32x4*>(y + (int64_t)m * a.ld_y + n) = v;
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
