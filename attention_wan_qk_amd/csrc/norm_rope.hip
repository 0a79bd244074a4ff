// Fused q/k RMSNorm + 3D RoPE over the (t, h, w) latent-patch grid.
//
// Follows the self-attention path of the WanAttentionBlock on the "Wan2.2
// code walkthrough" page (q/k RMSNorm, then rope_apply on q and k; V is not
// rotated) and its 3D RoPE snippet: the d/2 frequencies of a head are split
// [c - 2(c//3), c//3, c//3] between t, h and w (22/21/21 pairs for d = 128),
// broadcast over the flattened (f, h, w) grid (w fastest) and applied as a
// complex multiply on interleaved (re, im) pairs. Readings: one standard RoPE
// ladder theta^(-2j/D_a) per axis, positions from 0, RMSNorm over the full
// H*d token row unless WAN_NORM_PER_HEAD.
//
// Memory-bound: one wavefront owns one token row (q and k), streams it as
// 16-byte vectors held in registers, reduces the sum of squares across the
// wave and writes the rotated row back; the fp32 gain of the next 8-channel
// chunk is requested before the current chunk is written. Every lane works
// on the same 4 pairs of every head it touches (its chunks are lane + 64 i
// and a head is 16 chunks), so its 4 (cos, sin) pairs are computed once per
// token.
#include "wan_device.h"
#include "wan_internal.h"
#include "../../include/wanattn.h"

namespace wan {

template <int NCH>
__device__ __forceinline__ void norm_rope_one(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
    const float* __restrict__ gain, int lane, int nchunk, float inv_c,
    float eps, bool norm, bool per_head, bool rope, const float* cs,
    const float* sn) {
  u32x4 v[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    if (c < nchunk) v[i] = load_stream(src + 8 * c);
    else v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  float scale[NCH];
  if (norm) {
    float ss[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      float f[8];
      unpack8(v[i], f);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(f[e], f[e], s);
      ss[i] = s;
    }
    if (per_head) {
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        scale[i] = 1.0f / sqrtf(group16_sum(ss[i]) * (1.0f / 128.0f) + eps);
    } else {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) s += ss[i];
      const float r = 1.0f / sqrtf(wave_sum(s) * inv_c + eps);
#pragma unroll
      for (int i = 0; i < NCH; ++i) scale[i] = r;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NCH; ++i) scale[i] = 1.0f;
  }
  // The gain of chunk i + 1 is requested before chunk i is written, so the
  // L2 latency of the gain vectors is not paid chunk by chunk. Without a gain
  // (or without the norm) the factor is 1.
  const bool use_gain = norm && gain;
  auto load_gain = [&](int c, float* g) __attribute__((always_inline)) {
    if (use_gain && c < nchunk) {
      const f32x4 g0 = *reinterpret_cast<const f32x4*>(gain + 8 * c);
      const f32x4 g1 = *reinterpret_cast<const f32x4*>(gain + 8 * c + 4);
      g[0] = g0[0]; g[1] = g0[1]; g[2] = g0[2]; g[3] = g0[3];
      g[4] = g1[0]; g[5] = g1[1]; g[6] = g1[2]; g[7] = g1[3];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = 1.0f;
    }
  };
  float g_n[8];
  load_gain(lane, g_n);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = g_n[e];
    if (i + 1 < NCH) load_gain(c + kWave, g_n);
    if (c < nchunk) {
      float f[8];
      unpack8(v[i], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= scale[i] * g[e];
      if (rope) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float re = f[2 * p], im = f[2 * p + 1];
          f[2 * p] = re * cs[p] - im * sn[p];
          f[2 * p + 1] = re * sn[p] + im * cs[p];
        }
      }
      store_stream(dst + 8 * c, pack8(f));
    }
  }
}

template <int NCH>
__global__ __launch_bounds__(256) void norm_rope_kernel(NormRopeArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const bool norm = a.flags & WAN_NORM;
  const bool rope = a.flags & WAN_ROPE;
  const bool per_head = a.flags & WAN_NORM_PER_HEAD;
  const int C = a.H * a.D;
  const int nchunk = C >> 3;

  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (rope) {
    const int n = (int)(row % a.L);
    const int hw = a.grid_h * a.grid_w;
    const int pos_t = n / hw, pos_h = (n / a.grid_w) % a.grid_h, pos_w = n % a.grid_w;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // Pair j of the head: t owns 22 pairs, h and w 21 each (d = 128).
      const int j = 4 * (lane & 15) + p;
      int pos, jl, na;
      if (j < 22) { pos = pos_t; jl = j; na = 22; }
      else if (j < 43) { pos = pos_h; jl = j - 22; na = 21; }
      else { pos = pos_w; jl = j - 43; na = 21; }
      // omega = theta^(-2 jl / (2 na)); angle = pos * omega.
      const float omega = exp2f(-(float)jl * a.log2_theta / (float)na);
      sincosf((float)pos * omega, &sn[p], &cs[p]);
    }
  }
  const float inv_c = 1.0f / (float)C;
  if (a.q)
    norm_rope_one<NCH>(static_cast<const uint16_t*>(a.q) + row * a.ld_in,
                       static_cast<uint16_t*>(a.q_out) + row * a.ld_out,
                       a.gain_q, lane, nchunk, inv_c, a.eps, norm, per_head,
                       rope, cs, sn);
  if (a.k)
    norm_rope_one<NCH>(static_cast<const uint16_t*>(a.k) + row * a.ld_in,
                       static_cast<uint16_t*>(a.k_out) + row * a.ld_out,
                       a.gain_k, lane, nchunk, inv_c, a.eps, norm, per_head,
                       rope, cs, sn);
}

template <int NCH>
static hipError_t launch_nch(const NormRopeArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  hipLaunchKernelGGL(norm_rope_kernel<NCH>, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s) {
  const int nch = (a.H * a.D / 8 + kWave - 1) / kWave;
  switch (nch) {
    case 1: return launch_nch<1>(a, s);
    case 2: return launch_nch<2>(a, s);
    case 3: return launch_nch<3>(a, s);
    case 4: return launch_nch<4>(a, s);
    case 5: return launch_nch<5>(a, s);
    case 6: return launch_nch<6>(a, s);
    case 7: return launch_nch<7>(a, s);
    case 8: return launch_nch<8>(a, s);
    case 9: return launch_nch<9>(a, s);
    case 10: return launch_nch<10>(a, s);
    case 11: return launch_nch<11>(a, s);
    case 12: return launch_nch<12>(a, s);
    case 13: return launch_nch<13>(a, s);
    case 14: return launch_nch<14>(a, s);
    case 15: return launch_nch<15>(a, s);
    case 16: return launch_nch<16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wan
