// Quantisation of q, k and v for the 8-bit attention ("论文专题讲解：Wan2.1",
// inference-optimisation table, row "8-bit FlashAttention": INT8 for
// S = Q K^T, FP8 for O = P V).
//
// One workgroup per (batch, head, block of 64 tokens), four wavefronts:
//  * q and k: symmetric INT8 with one fp32 scale per block, amax / 127;
//    code = round_half_even(x * (127 / amax)) computed in fp32 (IEEE
//    division and product), clamped to +-127. Stored block-major per head,
//    64 rows of D bytes, so the attention kernel moves a key tile with
//    contiguous 1 KiB loads.
//  * v: FP8 E4M3 with a power-of-two (E8M0) scale per (channel, 32 keys),
//    the OCP microscaling recipe: X = 2^(floor(log2 amax) - 8), element =
//    E4M3(clamp(v / X, +-448)) rounded to nearest even. Stored transposed
//    per block (D rows of 64 key bytes), the A-operand layout of the P V
//    product, with the scale bytes ordered as the MFMA reads them.
//  * Rows past L are quantised as zeros, and so are key and value rows at or
//    past k_lens[b]: padding takes no part in attention, so it must not set
//    the block scales of the valid keys (nor carry an inf or NaN into them).
//    Query rows are all quantised.
// Memory-bound: 2 + 2 + 2 bytes read and 1 + 1 + 1 written per element of
// q, k and v.
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int kBlock = 64;        // tokens per block
constexpr int kHD = 128;          // head size
constexpr int kThreads = 256;

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  const int wave = threadIdx.x >> 6;
  __syncthreads();                      // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// INT8 quantisation of one 64 x 128 block of q or k; thread t covers the
// 16-byte chunk t % 16 of rows t / 16 + 16 i.
__device__ void quant_int8(int8_t* out, float* scale, const uint16_t* in, int64_t ld, int rows,
                           float* red) {
  const int t = threadIdx.x;
  const int c = t & 15;
  float x[4][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 4) + 16 * i;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < rows) w = load_stream(in + (int64_t)r * ld + 8 * c);
    unpack8(w, x[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
  }
  amax = block_max(amax, red);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (t >> 4) + 16 * i;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = fminf(fmaxf(__builtin_rintf(x[i][e] * inv), -127.0f), 127.0f);
      const uint32_t b = (uint32_t)((int)q & 0xff);
      if (e < 4) lo |= b << (8 * e);
      else hi |= b << (8 * (e - 4));
    }
    const u32x2 v = {lo, hi};
    *reinterpret_cast<u32x2*>(out + r * kHD + 8 * c) = v;
  }
  if (t == 0) *scale = amax > 0.0f ? amax / 127.0f : 0.0f;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void quant8_kernel(Quant8Args a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[kBlock * kHD];
  __shared__ float red[4];

  const int nT = (a.L + kBlock - 1) / kBlock;
  const int blk = blockIdx.x % nT;
  const int bh = blockIdx.x / nT;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int rows = min(kBlock, a.L - blk * kBlock);
  int kv_len = a.L;
  if (a.k_lens) kv_len = min(max(a.k_lens[b], 0), a.L);
  const int rows_kv = max(0, min(rows, kv_len - blk * kBlock));   // valid key rows of the block
  const int64_t tok0 = (int64_t)b * a.L + (int64_t)blk * kBlock;
  const int64_t tile = (int64_t)bh * nT + blk;   // [B][H][nT]

  quant_int8(a.q8 + tile * kBlock * kHD, a.q_scale + tile,
             static_cast<const uint16_t*>(a.q) + tok0 * a.ld_q + h * kHD, a.ld_q, rows, red);
  quant_int8(a.k8 + tile * kBlock * kHD, a.k_scale + tile,
             static_cast<const uint16_t*>(a.k) + tok0 * a.ld_k + h * kHD, a.ld_k, rows_kv, red);

  // v: stage the block in LDS, then thread t owns channel t % 128 of key
  // half t / 128 (32 keys).
  const int t = threadIdx.x;
  {
    const uint16_t* vin = static_cast<const uint16_t*>(a.v) + tok0 * a.ld_v + h * kHD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (t >> 4) + 16 * i;
      u32x4 w = {0u, 0u, 0u, 0u};
      if (r < rows_kv) w = load_stream(vin + (int64_t)r * a.ld_v + 8 * (t & 15));
      *reinterpret_cast<u32x4*>(vt + r * kHD + 8 * (t & 15)) = w;
    }
  }
  __syncthreads();
  const int ch = t & (kHD - 1), half = t >> 7;
  float x[32];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    x[j] = __uint_as_float((uint32_t)vt[(half * 32 + j) * kHD + ch] << 16);
    amax = fmaxf(amax, fabsf(x[j]));
  }
  int ex = -127;                                      // E8M0 byte 0 for an all-zero block
  if (amax > 0.0f) ex = max(__builtin_amdgcn_frexp_expf(amax) - 1 - 8, -127);
  uint32_t packed[8];
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    float s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      s[e] = fminf(fmaxf(__builtin_ldexpf(x[j + e], -ex), -448.0f), 448.0f);
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], w, true);
    packed[j / 4] = w;
  }
  uint8_t* vout = a.v8 + tile * kBlock * kHD + ch * kBlock + half * 32;
  *reinterpret_cast<u32x4*>(vout) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  *reinterpret_cast<u32x4*>(vout + 16) = u32x4{packed[4], packed[5], packed[6], packed[7]};
  // scale bytes: [half][channel % 32][channel / 32]
  a.v_scale[tile * 256 + half * 128 + (ch & 31) * 4 + (ch >> 5)] = (uint8_t)(ex + 127);
}

hipError_t launch_quant8(const Quant8Args& a, hipStream_t s) {
  const int64_t nT = (a.L + kBlock - 1) / kBlock;
  const int64_t total = (int64_t)a.B * a.H * nT;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quant8_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wan
