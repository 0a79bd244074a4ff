// Internal launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace wan {

struct NormRopeArgs {
  void* q_out;
  void* k_out;
  const void* q;
  const void* k;
  const float* gain_q;
  const float* gain_k;
  int64_t rows;    // B * L token rows
  int L, H, D;
  int grid_f, grid_h, grid_w;
  int64_t ld_in, ld_out;  // elements between consecutive token rows
  float eps;
  float log2_theta;
  unsigned flags;
};

struct AdaLNArgs {
  void* x_out;
  void* h_out;
  const void* x;
  const void* y;
  const float* gate;
  const float* shift;
  const float* scale;
  int64_t rows;    // B * L
  int L, C;
  int64_t mod_stride_b, mod_stride_l;
  float eps;
};

struct AttnArgs {
  void* o;
  float* lse;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* k_lens;
  int B, Lq, Lk, H;
  int64_t ld_q, ld_k, ld_v, ld_o;
  float scale_log2;   // softmax scale * log2(e)
  int q_offset;       // chunk-causal only: global position of query row 0
  int chunk_len;      // chunk-causal only: tokens per chunk (>= 1)
};

struct LinearArgs {
  void* y;
  const void* x;
  const void* w;
  const float* bias;
  int M, N, K;
  int64_t ld_x, ld_w, ld_y;
};

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s);
hipError_t launch_adaln(const AdaLNArgs& a, hipStream_t s);
// kind: 0 self-attention, 1 cross-attention, 2 chunk-causal self-attention.
hipError_t launch_attn_fwd(const AttnArgs& a, int kind, hipStream_t s);
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);

}  // namespace wan
