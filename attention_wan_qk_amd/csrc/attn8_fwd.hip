// 8-bit softmax self-attention forward on gfx950 ("论文专题讲解：Wan2.1",
// inference-optimisation table, row "8-bit FlashAttention": INT8 for
// S = Q K^T, FP8 for O = P V, FP32 accumulation across key blocks).
//
// Inputs are the outputs of the quantisation kernel: INT8 q and k with one
// fp32 scale per (batch, head, 64 tokens), FP8 E4M3 v stored transposed per
// 64-key block with power-of-two scales per (channel, 32 keys).
//
// Same work layout as the bf16 kernel (256 query rows per workgroup, 8
// waves of 32 rows, ping-pong between a GEMM phase and a softmax phase,
// online softmax in log2 units with a lazy rescale, K/V tiles loaded into
// LDS by the four waves of group 0), with these differences:
//  * S^T = K Q^T on v_mfma_i32_32x32x32_i8 (exact integer dot products). The
//    accumulator starts at the bit pattern of 2^23 + 2^22, so each result,
//    read as fp32, is 12582912 + S exactly (|S| <= 127^2 * 128 < 2^22) and
//    needs no conversion: t = fma(X, mult, C) with mult = sq sk scale log2 e
//    (truncated to 22 significant bits, so 12582912 mult is exact) and
//    C = -12582912 mult - m folds the offset away.
//  * The key rows of a 32-key block enter the MFMA in the order
//    sigma(8g + 4h + r) = 16h + 4g + r, so that half h of the wave holds
//    keys 16h .. 16h+15 of each block: exactly the k-slots the FP8 product
//    expects from that half (bytes 0-15: first 32-key block, 16-31: second).
//  * The running maximum m is an integer (log2 units): P = 2^(t - m) is then
//    the exact-maximum P times a power of two, so its E4M3 rounding does not
//    depend on when m was last raised, and the rescale factor 2^(m - m') is
//    exact. The tile maximum is only formed on a row's first tile and when a
//    lane's sum of its 32 weights passes 448, E4M3's largest value (which
//    any weight above 448 causes); then m is raised to ceil(max) - 7 if the
//    maximum passes m + 8, and the tile's weights are formed and converted
//    again. So every converted weight is at most 448, and m trails the
//    exact-maximum offset by at most 3.
//  * O^T += V^T P^T on v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands:
//    V^T fragments straight from the transposed tile, P from the softmax
//    registers (v_cvt_pk_fp8_f32, round to nearest even), the V block scales
//    applied by the MFMA itself (one E8M0 byte per lane, selected by op_sel).
//  * The softmax denominator l sums the unrounded fp32 weights (the FP8
//    rounding belongs to the operand of the P V product only); each lane
//    keeps four partial sums, combined across the two half-waves at the end.
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int kWaves = 8;
constexpr int kBM = 32 * kWaves;             // query rows per workgroup
constexpr int kBN = 64;                      // keys per tile (= one q/k scale block)
constexpr int kHD = 128;
constexpr int kKTile = kBN * kHD;            // 8 KiB of INT8 keys
constexpr int kVTile = kHD * kBN;            // 8 KiB of FP8 values (transposed)
constexpr int kSTile = 256;                  // E8M0 scale bytes per tile
constexpr int kMaxBlocks = 4096;             // key-block scales kept in LDS (L <= 262144)
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerWave = kKTile / 1024 / (kWaves / 2);   // group-0 waves
constexpr float kRescaleThreshold = 8.0f;
constexpr float kSumLimit = 448.0f;          // per-lane tile sum of P that forces the tile max
constexpr float kBias = 12582912.0f;         // 2^23 + 2^22
constexpr int kBiasBits = 0x4B400000;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kWaitLoads = 0x0F70;           // s_waitcnt vmcnt(0)
constexpr int kSgMfma = 0x008, kSgDsRead = 0x100;

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

template <int N>
struct Int {
  static constexpr int value = N;
};

// Barrier between phases without a memory fence (see the bf16 kernel): the
// only LDS writes in the loop are group 0's buffer loads, awaited before the
// barrier that publishes them.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// INT8 K tile (64 rows of 128 bytes): chunk c of row r at c ^ gk(r); the 16
// rows read together ({0-7, 16-23} or {8-15, 24-31} of a 32-key block after
// the sigma order) fall into 16 different 16-byte bank groups.
__device__ __forceinline__ int gk(int r) { return ((r >> 1) & 3) | (((r >> 4) & 1) << 2); }
// FP8 V^T tile (128 rows of 64 bytes): chunk c of row d at c ^ ((d / 4) % 4).
__device__ __forceinline__ int gv(int d) { return (d >> 2) & 3; }
// MFMA row i of a 32-key block -> key inside the block.
__device__ __forceinline__ int sigma(int i) {
  return (((i >> 2) & 1) << 4) | (((i >> 3) & 3) << 2) | (i & 3);
}

}  // namespace

__global__ __launch_bounds__(kThreads, 1) void attn8_fwd_kernel(Attn8Args a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kKTile + 2 * kVTile + 2 * kSTile];
  __shared__ float skl[kMaxBlocks];             // k scales of this (batch, head)
  char* const Ks = smem;
  char* const Vs = smem + 2 * kKTile;
  char* const Ss = smem + 2 * kKTile + 2 * kVTile;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int group = wave / (kWaves / 2);
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  const int nQ = (a.L + kBM - 1) / kBM;
  const int nB = (a.L + kBN - 1) / kBN;          // 64-token blocks per (batch, head)
  const uint32_t total = (uint32_t)a.B * a.H * nQ;
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int qt = logical % nQ;
  const int bh = logical / nQ;
  const int b = bh / a.H;
  const int h = bh % a.H;

  int kv_len = a.L;
  if (a.k_lens) kv_len = min(max(a.k_lens[b], 0), a.L);
  const int nT = (kv_len + kBN - 1) / kBN;

  const int8_t* kq = a.k8 + (int64_t)bh * nB * kKTile;
  const uint8_t* vq = a.v8 + (int64_t)bh * nB * kVTile;
  const uint8_t* sv = a.v_scale + (int64_t)bh * nB * kSTile;
  const float* sk = a.k_scale + (int64_t)bh * nB;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)kq, (short)0, nB * kKTile, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)vq, (short)0, nB * kVTile, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)sv, (short)0, nB * kSTile, kRsrcWord3);

  // Group-0 loads: K load i of wave w fills tile rows 8(2w + i) .. +7 (lane l:
  // row + l / 8, physical chunk l % 8); V load i fills rows 16(2w + i) .. +15
  // (lane l: row + l / 4, physical chunk l % 4); wave 0 also moves the 256
  // scale bytes (4 per lane).
  uint32_t vo_k[kLoadsPerWave], vo_v[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; ++i) {
    const int rk_row = ((wave & 3) * kLoadsPerWave + i) * 8 + (lane >> 3);
    vo_k[i] = rk_row * kHD + (((lane & 7) ^ gk(rk_row)) << 4);
    const int rv_row = ((wave & 3) * kLoadsPerWave + i) * 16 + (lane >> 2);
    vo_v[i] = rv_row * kBN + (((lane & 3) ^ gv(rv_row)) << 4);
  }
  auto dma_k = [&](int t, int slot) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (lds_void*)(Ks + slot * kKTile + ((wave & 3) * kLoadsPerWave + i) * 1024), 16,
          vo_k[i], t * kKTile, 0, 0);
  };
  auto dma_v = [&](int t, int slot) {   // values and their scale bytes
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rv, (lds_void*)(Vs + slot * kVTile + ((wave & 3) * kLoadsPerWave + i) * 1024), 16,
          vo_v[i], t * kVTile, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(Ss + slot * kSTile), 4, lane * 4,
                                               t * kSTile, 0, 0);
  };

  // Q fragments (B operand of S^T = K Q^T): lane holds q8[row][32 ds + 16 hf ..].
  const int qrow = qt * kBM + wave * 32 + r32;
  const int qr = min(qrow, a.L - 1);
  i32x4 qf[4];
  {
    const int8_t* qp = a.q8 + ((int64_t)bh * nB + qr / kBN) * kKTile + (qr % kBN) * kHD + 16 * hf;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[ds] = *reinterpret_cast<const i32x4*>(qp + 32 * ds);
  }
  const float sq = a.q_scale[(int64_t)bh * nB + min(qt * kBM + wave * 32, a.L - 1) / kBN];

  if (nT > 0 && group == 0) dma_k(0, 0);
  for (int i = tid; i < nT; i += kThreads) skl[i] = sk[i];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // LDS read offsets inside a tile.
  int ka[4];                                  // K row sigma-ordered, chunk 2 ds + hf
  {
    const int row = sigma(r32);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) ka[ds] = row * kHD + (((2 * ds + hf) ^ gk(row)) << 4);
  }
  int va_lo, va_hi;                           // V^T row r32 (+ 32 db), chunks hf and 2 + hf
  va_lo = r32 * kBN + ((hf ^ gv(r32)) << 4);
  va_hi = r32 * kBN + (((2 + hf) ^ gv(r32)) << 4);

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.f;
  float m_used = -INFINITY;
  float ls[4] = {0.f, 0.f, 0.f, 0.f};         // partial row sums of the unrounded P
  i32x16 s[2];
  i32x8 pq;                                   // P of the tile as 32 E4M3 bytes

  auto gemm = [&](auto ksc, int jj) {
    constexpr int KS = decltype(ksc)::value;
    if (jj >= 1 && jj <= nT) {
      const char* Vt = Vs + (1 - KS) * kVTile;
      const int sc = *reinterpret_cast<const int*>(Ss + (1 - KS) * kSTile + lane * 4);
      i32x4 vlo[4], vhi[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        vlo[db] = *reinterpret_cast<const i32x4*>(Vt + va_lo + 32 * db * kBN);
        vhi[db] = *reinterpret_cast<const i32x4*>(Vt + va_hi + 32 * db * kBN);
      }
#define WAN_PV(DB)                                                                           \
  {                                                                                          \
    const i32x8 va = __builtin_shufflevector(vlo[DB], vhi[DB], 0, 1, 2, 3, 4, 5, 6, 7);       \
    oacc[DB] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pq, oacc[DB], 0, 0, DB, sc, \
                                                               0, 127);                      \
  }
      WAN_PV(0) WAN_PV(1) WAN_PV(2) WAN_PV(3)
#undef WAN_PV
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 2, 0);
    }
    if (jj < nT) {
      const char* Kt = Ks + KS * kKTile;
      i32x4 kf[8];
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          kf[ds * 2 + kb] = *reinterpret_cast<const i32x4*>(Kt + ka[ds] + kb * 32 * kHD);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = kBiasBits;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[ds * 2 + kb], qf[ds], s[kb], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSgMfma, 4, 0);
    }
  };

  auto softmax = [&](int jj) {
    if (jj < 0 || jj >= nT) return;
    // mult is floored at 1e-30 (an all-zero q or k block) so that masked
    // keys (-inf) still give t = -inf, and truncated to 22 significant bits
    // so that 12582912 * mult is exact in fp32: t is then S mult - m rounded
    // once, as if S had been converted.
    float mult = fmaxf((sq * skl[jj]) * a.scale_log2, 1e-30f);
    mult = __uint_as_float(__float_as_uint(mult) & 0xFFFFFFFCu);
    float x[32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[kb * 16 + v] = __int_as_float(s[kb][v]);
    const bool edge = (jj + 1) * kBN > kv_len;
    if (edge) {   // keys past k_len (last tile only): kb 32 + 16 hf + v
#pragma unroll
      for (int e = 0; e < 32; ++e)
        if (jj * kBN + (e >> 4) * 32 + 16 * hf + (e & 15) >= kv_len) x[e] = -INFINITY;
    }
    // P = 2^(t - m): per-lane partial sums of the fp32 values, and their E4M3
    // codes (a weight above 448 converts to NaN; the sum check below then
    // sends the tile through the exact path, which converts it again)
    float sg[4];
    auto exps = [&]() __attribute__((always_inline)) {
      const float cc = -(kBias * mult) - m_used;
#pragma unroll
      for (int q4 = 0; q4 < 8; ++q4) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(x[4 * q4 + e], mult, cc));
          // each partial sum starts at its first weight (no addition to 0)
          sg[e] = q4 == 0 ? p[e] : sg[e] + p[e];
        }
        const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        pq[q4] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
      }
    };
    // The range's first tile forms the row maxima. On a later tile a row whose
    // maximum is still -inf would get weights of inf or NaN, which the sum
    // check below sends through the exact path as well.
    bool exact = jj == 0;
    if (!exact) {
      exps();
      const float big = fmaxf(fmaxf(sg[0], sg[1]), fmaxf(sg[2], sg[3]));
      exact = __any(!(big <= kSumLimit));
    }
    if (exact) {
      float mx = fmaxf(x[0], x[1]);
#pragma unroll
      for (int e = 2; e < 32; ++e) mx = fmaxf(mx, x[e]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float mt = (mx - kBias) * mult;   // row maximum in log2 units (exact offset)
      if (__any(mt > m_used + kRescaleThreshold)) {
        const float mn = fmaxf(m_used, ceilf(mt) - 7.0f);
        const float alpha = mn == m_used ? 1.0f : __builtin_amdgcn_exp2f(m_used - mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) ls[i] *= alpha;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha;
        m_used = mn;
      }
      exps();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) ls[i] += sg[i];
  };

  // As in the bf16 kernel: tile j's K and tile j-1's V (with its scale
  // bytes) stay in LDS for intervals 2j and 2j+1; group 0 loads K(j+1) and
  // V(j) right after its GEMM phase of interval 2j into the slots of K(j-1)
  // and V(j-2) and waits for them at the end of interval 2j+1.
  const int nIntervals = 2 * nT + 2;
  for (int i = 0; i < nIntervals; i += 4) {
    const int j0 = i >> 1;
    if (group == 0) {
      gemm(Int<0>{}, j0);
      if (j0 < nT) {
        if (j0 + 1 < nT) dma_k(j0 + 1, 1);
        dma_v(j0, 0);
      }
    } else softmax(j0 - 1);
    phase_barrier();
    if (group == 0) {
      softmax(j0);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
    } else gemm(Int<0>{}, j0);
    phase_barrier();
    const int j1 = j0 + 1;
    if (group == 0) {
      gemm(Int<1>{}, j1);
      if (j1 < nT) {
        if (j1 + 1 < nT) dma_k(j1 + 1, 0);
        dma_v(j1, 1);
      }
    } else softmax(j0);
    phase_barrier();
    if (group == 0) {
      softmax(j1);
      __builtin_amdgcn_s_waitcnt(kWaitLoads);
    } else gemm(Int<1>{}, j1);
    phase_barrier();
  }

  float lsum = (ls[0] + ls[1]) + (ls[2] + ls[3]);
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                     false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (qrow < a.L) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((int64_t)b * a.L + qrow) * a.ld_o + h * kHD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 xo = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv,
                    oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 y = __builtin_convertvector(xo, bf16x4);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * hf) = __builtin_bit_cast(u32x2, y);
      }
    if (a.lse && hf == 0) {
      a.lse[((int64_t)b * a.H + h) * a.L + qrow] =
          lsum > 0.f ? m_used * 0.6931471805599453f + logf(lsum) : -INFINITY;
    }
  }
}

hipError_t launch_attn8_fwd(const Attn8Args& a, hipStream_t s) {
  const int nQ = (a.L + kBM - 1) / kBM;
  const int64_t total = (int64_t)a.B * a.H * nQ;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn8_fwd_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wan
