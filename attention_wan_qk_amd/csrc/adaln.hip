// Residual update + AdaLN-modulated LayerNorm, one wavefront per token row.
//
// Follows the WanAttentionBlock snippet of the "Wan2.2 code walkthrough"
// page: norm1(x).float() * (1 + e[1]) + e[0] (modulated fp32 LayerNorm),
// x = x + y * e[2] (gated residual) and x = x + cross_attn(norm3(x), ...)
// (ungated residual, norm3 being the same LayerNorm with an affine).
//
// Memory-bound: the row is read once as 16-byte vectors, kept in registers,
// reduced twice across the wave (mean, then the centred sum of squares) and
// written once per output. The kernel is specialised on whether there is a
// residual input (without one the row stays packed bf16 and is widened on
// each pass, which halves its registers) and on whether the normalised output
// is wanted (without it there is nothing to reduce).
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
}

template <int NCH, bool kY, bool kH>
__global__ __launch_bounds__(256) void adaln_kernel(AdaLNArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int nchunk = a.C >> 3;
  const int64_t b = row / a.L, l = row % a.L;
  const int64_t moff = b * a.mod_stride_b + l * a.mod_stride_l;
  const float* gate = a.gate ? a.gate + moff : nullptr;
  const float* shift = a.shift ? a.shift + moff : nullptr;
  const float* scale = a.scale ? a.scale + moff : nullptr;
  const uint16_t* x = static_cast<const uint16_t*>(a.x) + row * a.C;
  const uint16_t* y = kY ? static_cast<const uint16_t*>(a.y) + row * a.C : nullptr;
  uint16_t* xo = a.x_out ? static_cast<uint16_t*>(a.x_out) + row * a.C : nullptr;
  uint16_t* ho = kH ? static_cast<uint16_t*>(a.h_out) + row * a.C : nullptr;

  u32x4 xv[NCH], yv[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    const bool in = c < nchunk;
    xv[i] = in ? load_stream(x + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    if (kY) yv[i] = in ? load_stream(y + 8 * c) : u32x4{0u, 0u, 0u, 0u};
  }

  // r = x + gate * y in fp32 (the residual row); without y it is x itself.
  float r[kY ? NCH : 1][8];
  auto row_vals = [&](int i, float* f) __attribute__((always_inline)) {
    if (kY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = r[kY ? i : 0][e];
    } else {
      unpack8(xv[i], f);
    }
  };
  if (kY) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
      float xf[8], yf[8];
      unpack8(xv[i], xf);
      unpack8(yv[i], yf);
      if (gate && c < nchunk) {
        float g[8];
        load8f(gate + 8 * c, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) r[kY ? i : 0][e] = fmaf(g[e], yf[e], xf[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) r[kY ? i : 0][e] = xf[e] + yf[e];
      }
    }
  }

  float mean = 0.f, rstd = 0.f;
  if (kH) {
    const float inv_c = 1.0f / (float)a.C;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      float f[8];
      row_vals(i, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += f[e];
    }
    mean = wave_sum(sum) * inv_c;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (lane + kWave * i < nchunk) {
        float f[8];
        row_vals(i, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = f[e] - mean;
          sq = fmaf(d, d, sq);
        }
      }
    }
    rstd = 1.0f / sqrtf(wave_sum(sq) * inv_c + a.eps);
  }
  // Keep the modulation loads below the reductions: hoisting them would hold
  // two more rows of registers and cut occupancy.
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    if (c >= nchunk) continue;
    float f[8];
    row_vals(i, f);
    if (xo) store_stream(xo + 8 * c, kY ? pack8(f) : xv[i]);
    if (kH) {
      float sc[8], sh[8], hv[8];
      if (scale) load8f(scale + 8 * c, sc);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sc[e] = 0.f;
      }
      if (shift) load8f(shift + 8 * c, sh);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) sh[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = fmaf((f[e] - mean) * rstd, 1.0f + sc[e], sh[e]);
      store_stream(ho + 8 * c, pack8(hv));
    }
    __builtin_amdgcn_sched_barrier(0);   // one chunk's modulation vectors live at a time
  }
}

template <int NCH>
static hipError_t launch_nch(const AdaLNArgs& a, hipStream_t s) {
  const unsigned blocks = (unsigned)((a.rows + 3) / 4);
  const bool y = a.y != nullptr, h = a.h_out != nullptr;
  if (y && h) hipLaunchKernelGGL((adaln_kernel<NCH, true, true>), dim3(blocks), dim3(256), 0, s, a);
  else if (y) hipLaunchKernelGGL((adaln_kernel<NCH, true, false>), dim3(blocks), dim3(256), 0, s, a);
  else if (h) hipLaunchKernelGGL((adaln_kernel<NCH, false, true>), dim3(blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((adaln_kernel<NCH, false, false>), dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_adaln(const AdaLNArgs& a, hipStream_t s) {
  const int nch = (a.C / 8 + kWave - 1) / kWave;
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
