// Softmax attention forward on bf16 MFMA (gfx950), used for both the full
// self-attention over all video tokens and the cross-attention to text.
//
// Follows the self-attention call of the "Wan2.2 code walkthrough" page,
// flash_attention(q, k, v, k_lens, window_size = (-1, -1)): global window,
// no causal mask, keys at or past k_lens[b] excluded. The L x L score matrix
// is never stored: each workgroup owns 128 query rows of one (batch, head)
// and streams the keys in tiles of 64 with a running (online) softmax.
//
// Layout of the work (per workgroup: 4 wavefronts x 32 query rows):
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16. K (A operand, keys x dims) is
//    read from LDS; Q (B operand) stays in registers for the whole loop. In
//    the accumulator each lane owns one query row (lane % 32) and 16 keys, so
//    the row max needs one exchange with the other half-wave and the row sum
//    none until the end.
//  * O^T += V^T P^T on the same MFMA. P comes straight from the score
//    registers (converted to bf16); V^T is read from the row-major V tile with
//    ds_read_b64_tr_b16, whose key order is chosen to match P's.
//  * The running max is in log2 units of the scaled scores; it is only moved
//    (and O, l rescaled) when some row's tile max exceeds it by more than 8,
//    so the exponentials stay <= 2^8 and the rescale is rare.
//  * K/V tiles are double-buffered in LDS (XOR-swizzled 16-byte chunks for
//    conflict-free MFMA operand reads); the next tile's global loads are
//    issued before the current tile's math.
//  * Workgroup ids are remapped so that each XCD works through consecutive
//    query tiles of the same (batch, head) and shares its K/V in its L2.
#include "wan_device.h"
#include "wan_internal.h"

namespace wan {

namespace {

constexpr int kBM = 128;        // query rows per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr int kHD = 128;        // head size
constexpr int kRowBytes = kHD * 2;
constexpr int kTileBytes = kBN * kRowBytes;  // 16 KiB
constexpr int kThreads = 256;
constexpr float kRescaleThreshold = 8.0f;    // log2 units

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 lds_read16(const char* base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

__device__ __forceinline__ s16x4 lds_read_tr(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
}

// Byte offset of 16-byte chunk `ch` of key row `key` in the K tile. The
// chunk index is XORed with key % 16 so that 16 consecutive keys reading the
// same logical chunk hit 16 different bank groups.
__device__ __forceinline__ uint32_t k_off(int key, int ch) {
  return (uint32_t)(key * kRowBytes + ((ch ^ (key & 15)) << 4));
}
// V tile: the transposed reads touch 4 consecutive keys x 4 consecutive
// chunks per half-wave, so the chunk is XORed with 4 * (key % 4).
__device__ __forceinline__ uint32_t v_off(int key, int ch) {
  return (uint32_t)(key * kRowBytes + ((ch ^ ((key & 3) << 2)) << 4));
}

}  // namespace

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2][2][kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r32 = lane & 31;
  const int hf = lane >> 5;

  const int nQ = (a.Lq + kBM - 1) / kBM;
  const uint32_t total = (uint32_t)a.B * a.H * nQ;
  const uint32_t logical = xcd_remap(blockIdx.x, total);
  const int qt = logical % nQ;
  const int bh = logical / nQ;
  const int h = bh % a.H;
  const int b = bh / a.H;

  int kv_len = a.Lk;
  if (a.k_lens) kv_len = min(max(a.k_lens[b], 0), a.Lk);

  const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (int64_t)b * a.Lq * a.ld_q + h * kHD;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k) + (int64_t)b * a.Lk * a.ld_k + h * kHD;
  const uint16_t* vg = static_cast<const uint16_t*>(a.v) + (int64_t)b * a.Lk * a.ld_v + h * kHD;

  // Q fragment: B operand of S^T = K Q^T, lane holds Q[row][16c + 8hf .. +8].
  const int qrow = qt * kBM + wave * 32 + r32;
  bf16x8 qf[8];
  if (qrow < a.Lq) {
    const uint16_t* qr = qg + (int64_t)qrow * a.ld_q + 8 * hf;
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qr + 16 * c);
  } else {
#pragma unroll
    for (int c = 0; c < 8; ++c) qf[c] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 oacc[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[d][v] = 0.f;
  float m_used = -INFINITY;
  float lsum = 0.f;

  const int nT = (kv_len + kBN - 1) / kBN;

  // Tile staging: thread tid moves 16-byte chunks tid + 256 i (i < 4) of the
  // 64 x 16 chunk tile; rows past kv_len are zero-filled (P is exactly 0
  // there, and 0 * 0 keeps O finite).
  u32x4 kreg[4], vreg[4];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int key = t * kBN + (idx >> 4);
      const int ch = idx & 15;
      if (key < kv_len) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kg + (int64_t)key * a.ld_k + 8 * ch);
        vreg[i] = *reinterpret_cast<const u32x4*>(vg + (int64_t)key * a.ld_v + 8 * ch);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto swrite = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + kThreads * i;
      const int key = idx >> 4;
      const int ch = idx & 15;
      *reinterpret_cast<u32x4*>(&smem[buf][0][k_off(key, ch)]) = kreg[i];
      *reinterpret_cast<u32x4*>(&smem[buf][1][v_off(key, ch)]) = vreg[i];
    }
  };

  if (nT > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();

  // Per-lane constants of the transposed V read (this lane as a source lane
  // of ds_read_b64_tr_b16: group g = lane / 16, key step e4, dim quad q4).
  const int g16 = lane >> 4;
  const int e4 = (lane & 15) >> 2;
  const int q4 = lane & 3;
  const int vkey_base = 4 * (g16 >> 1) + e4;
  const int vbyte_base = 32 * (g16 & 1) + 8 * q4;

  for (int t = 0; t < nT; ++t) {
    const int buf = t & 1;
    if (t + 1 < nT) gload(t + 1);

    // ---- S^T = K Q^T for 64 keys: two 32-key blocks x 8 dim steps.
    const char* Kt = smem[buf][0];
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = lds_read16(Kt, k_off(kb * 32 + r32, 2 * c + hf));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }

    // ---- mask keys past kv_len (last tile only)
    if ((t + 1) * kBN > kv_len) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = t * kBN + kb * 32 + 8 * (v >> 2) + 4 * hf + (v & 3);
          if (key >= kv_len) s[kb][v] = -INFINITY;
        }
    }

    // ---- online softmax (log2 domain)
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mt = mx * a.scale_log2;
    if (__any(mt > m_used + kRescaleThreshold)) {
      const float mn = fmaxf(m_used, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
      lsum *= alpha;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[d][v] *= alpha;
      m_used = mn;
    }
    bf16x8 pf[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[kc >> 1][8 * (kc & 1) + e], a.scale_log2, -m_used));
        lsum += p[e];
      }
      f32x8 pv = {p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]};
      pf[kc] = __builtin_convertvector(pv, bf16x8);
    }

    // ---- O^T += V^T P^T: 4 dim blocks x 4 key chunks of 16.
    const char* Vt = smem[buf][1];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int key0 = 32 * (kc >> 1) + 16 * (kc & 1) + vkey_base;
        const int byte = 64 * db + vbyte_base;
        const uint32_t o0 = v_off(key0, byte >> 4) + (byte & 15);
        const uint32_t o1 = v_off(key0 + 8, byte >> 4) + (byte & 15);
        const s16x4 lo = lds_read_tr(Vt, o0);
        const s16x4 hi = lds_read_tr(Vt, o1);
        const s16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, cat), pf[kc], oacc[db], 0, 0, 0);
      }
    }

    if (t + 1 < nT) swrite(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: combine the two half-waves' partial sums, normalise, store.
  const float ltot = lsum + __shfl_xor(lsum, 32, 64);
  if (qrow < a.Lq) {
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;
    uint16_t* orow = static_cast<uint16_t*>(a.o) + ((int64_t)b * a.Lq + qrow) * a.ld_o + h * kHD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        f32x4 x = {oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv,
                   oacc[db][4 * a4 + 2] * inv, oacc[db][4 * a4 + 3] * inv};
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        const bf16x4 y = __builtin_convertvector(x, bf16x4);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * a4 + 4 * hf) = __builtin_bit_cast(u32x2, y);
      }
    if (a.lse && hf == 0) {
      a.lse[((int64_t)b * a.H + h) * a.Lq + qrow] =
          ltot > 0.f ? m_used * 0.6931471805599453f + logf(ltot) : -INFINITY;
    }
  }
}

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
  const int nQ = (a.Lq + kBM - 1) / kBM;
  const int64_t total = (int64_t)a.B * a.H * nQ;
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)total), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace wan
