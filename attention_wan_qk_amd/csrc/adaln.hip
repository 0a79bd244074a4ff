// Residual update + AdaLN-modulated LayerNorm, one wavefront per R token rows.
//
// Follows the WanAttentionBlock snippet of the "Wan2.2 code walkthrough"
// page: norm1(x).float() * (1 + e[1]) + e[0] (modulated fp32 LayerNorm),
// x = x + y * e[2] (gated residual) and x = x + cross_attn(norm3(x), ...)
// (ungated residual, norm3 being the same LayerNorm with an affine).
//
// Memory-bound: each row is read once as 16-byte vectors, kept in registers,
// reduced twice across the wave (mean, then the centred sum of squares) and
// written once per output. The fp32 modulation vectors (shift, scale, gate)
// cost 4 bytes per channel each, more than the row itself, and come from L2:
// a wave that owns R consecutive rows of one sample loads them once for all
// R rows, and the vectors of the next 8-channel chunk are requested before
// the current chunk is used, so their L2 latency is not paid chunk by chunk.
// The kernel is specialised on whether there is a residual input (without one
// the row stays packed bf16 and is widened on each pass, which halves its
// registers) and on whether the normalised output is wanted (without it there
// is nothing to reduce).
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

// Rows per wavefront: two without a residual input (its rows stay packed and
// are small), one with it (its fp32 residual rows already fill the registers).
constexpr int kRowsNoY = 2;
constexpr int kRowsY = 1;

__device__ __forceinline__ void load8f(const float* p, float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
}

// The packed rows are widened again on every pass over them: an empty asm
// that claims to modify them keeps the compiler from holding the widened
// fp32 copies (twice the registers) from one pass to the next.
template <int R, int NCH>
__device__ __forceinline__ void launder_rows(u32x4 (&v)[R][NCH]) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < NCH; ++i) asm volatile("" : "+v"(v[r][i]));
}

template <int NCH, int R, bool kY, bool kH>
__global__ __launch_bounds__(256) void adaln_kernel(AdaLNArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (row0 >= a.rows) return;
  const int nchunk = a.C >> 3;
  int64_t moff[R];
  bool valid[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = min(row0 + r, a.rows - 1);
    valid[r] = row0 + r < a.rows;
    moff[r] = (row / a.L) * a.mod_stride_b + (row % a.L) * a.mod_stride_l;
  }
  // one set of modulation vectors serves every row of the wave
  bool shared = true;
#pragma unroll
  for (int r = 1; r < R; ++r) shared = shared && moff[r] == moff[0];

  const uint16_t* x = static_cast<const uint16_t*>(a.x) + row0 * a.C;
  const uint16_t* y = kY ? static_cast<const uint16_t*>(a.y) + row0 * a.C : nullptr;
  uint16_t* xo = a.x_out ? static_cast<uint16_t*>(a.x_out) + row0 * a.C : nullptr;
  uint16_t* ho = kH ? static_cast<uint16_t*>(a.h_out) + row0 * a.C : nullptr;

  u32x4 xv[R][NCH], yv[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
      const bool in = c < nchunk && valid[r];
      xv[r][i] = in ? load_stream(x + (int64_t)r * a.C + 8 * c) : u32x4{0u, 0u, 0u, 0u};
      if (kY) yv[r][i] = in ? load_stream(y + (int64_t)r * a.C + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }

  // res = x + gate * y in fp32 (the residual row); without y it is x itself.
  float res[kY ? R : 1][kY ? NCH : 1][8];
  auto row_vals = [&](int r, int i, float* f) __attribute__((always_inline)) {
    if (kY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = res[kY ? r : 0][kY ? i : 0][e];
    } else {
      unpack8(xv[r][i], f);
    }
  };
  // An fp32 modulation vector (8 channels of chunk c), zero where absent.
  auto load_mod8 = [&](const float* base, int64_t off, int c, float* v) __attribute__((always_inline)) {
    if (base && c < nchunk) load8f(base + off + 8 * c, v);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
  };
  if (kY) {
    // the gate of chunk i + 1 is in flight while chunk i is combined
    float g_n[8];
    load_mod8(a.gate, moff[0], lane, g_n);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = lane + kWave * i;
      float g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = g_n[e];
      if (i + 1 < NCH) load_mod8(a.gate, moff[0], c + kWave, g_n);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r > 0 && !shared) load_mod8(a.gate, moff[r], c, g);
        float xf[8], yf[8];
        unpack8(xv[r][i], xf);
        unpack8(yv[r][i], yf);
        if (a.gate) {
#pragma unroll
          for (int e = 0; e < 8; ++e) res[kY ? r : 0][kY ? i : 0][e] = fmaf(g[e], yf[e], xf[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) res[kY ? r : 0][kY ? i : 0][e] = xf[e] + yf[e];
        }
      }
    }
  }

  float mean[R], rstd[R];
  if (kH) {
    const float inv_c = 1.0f / (float)a.C;
    float sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sum[r] = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        float f[8];
        row_vals(r, i, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[r] += f[e];
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) mean[r] = wave_sum(sum[r]) * inv_c;
    float sq[R];
    if (!kY) launder_rows(xv);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sq[r] = 0.f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        if (lane + kWave * i < nchunk) {
          float f[8];
          row_vals(r, i, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float d = f[e] - mean[r];
            sq[r] = fmaf(d, d, sq[r]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) rstd[r] = 1.0f / sqrtf(wave_sum(sq[r]) * inv_c + a.eps);
  }
  // Keep the modulation loads below the reductions: hoisting them would hold
  // more rows of registers and cut occupancy.
  __builtin_amdgcn_sched_barrier(0);
  if (!kY) launder_rows(xv);

  // the modulation of chunk i + 1 is in flight while chunk i is written
  float sc_n[8], sh_n[8];
  if (kH) {
    load_mod8(a.scale, moff[0], lane, sc_n);
    load_mod8(a.shift, moff[0], lane, sh_n);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = lane + kWave * i;
    float sc[8], sh[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sc[e] = sc_n[e];
      sh[e] = sh_n[e];
    }
    if (kH && i + 1 < NCH) {
      load_mod8(a.scale, moff[0], c + kWave, sc_n);
      load_mod8(a.shift, moff[0], c + kWave, sh_n);
    }
    if (c < nchunk) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!valid[r]) continue;
        float f[8];
        row_vals(r, i, f);
        if (xo) store_stream(xo + (int64_t)r * a.C + 8 * c, kY ? pack8(f) : xv[r][i]);
        if (kH) {
          if (r > 0 && !shared) {
            load_mod8(a.scale, moff[r], c, sc);
            load_mod8(a.shift, moff[r], c, sh);
          }
          float hv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) hv[e] = fmaf((f[e] - mean[r]) * rstd[r], 1.0f + sc[e], sh[e]);
          store_stream(ho + (int64_t)r * a.C + 8 * c, pack8(hv));
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // two chunks' modulation vectors live at a time
  }
}

template <int NCH>
static hipError_t launch_nch(const AdaLNArgs& a, hipStream_t s) {
  const bool y = a.y != nullptr, h = a.h_out != nullptr;
  constexpr int RY = kRowsY, RN = kRowsNoY;
  const unsigned by = (unsigned)((a.rows + 4 * RY - 1) / (4 * RY));
  const unsigned bn = (unsigned)((a.rows + 4 * RN - 1) / (4 * RN));
  if (y && h) hipLaunchKernelGGL((adaln_kernel<NCH, RY, true, true>), dim3(by), dim3(256), 0, s, a);
  else if (y) hipLaunchKernelGGL((adaln_kernel<NCH, RY, true, false>), dim3(by), dim3(256), 0, s, a);
  else if (h) hipLaunchKernelGGL((adaln_kernel<NCH, RN, false, true>), dim3(bn), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((adaln_kernel<NCH, RN, false, false>), dim3(bn), dim3(256), 0, s, a);
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
