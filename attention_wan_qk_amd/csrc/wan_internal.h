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

struct Quant8Args {
  int8_t* q8;
  int8_t* k8;
  uint8_t* v8;
  float* q_scale;
  float* k_scale;
  uint8_t* v_scale;
  const void* q;
  const void* k;
  const void* v;
  int B, L, H;
  int64_t ld_q, ld_k, ld_v;
};

struct Attn8Args {
  void* o;
  float* lse;
  const int8_t* q8;
  const int8_t* k8;
  const uint8_t* v8;
  const float* q_scale;
  const float* k_scale;
  const uint8_t* v_scale;
  const int32_t* k_lens;
  int B, L, H;
  int64_t ld_o;
  float scale_log2;   // softmax scale * log2(e), fp32
};

hipError_t launch_norm_rope(const NormRopeArgs& a, hipStream_t s);
hipError_t launch_adaln(const AdaLNArgs& a, hipStream_t s);
// kind: 0 self-attention, 1 cross-attention, 2 chunk-causal self-attention.
hipError_t launch_attn_fwd(const AttnArgs& a, int kind, hipStream_t s);
hipError_t launch_linear(const LinearArgs& a, hipStream_t s);
hipError_t launch_quant8(const Quant8Args& a, hipStream_t s);
hipError_t launch_attn8_fwd(const Attn8Args& a, hipStream_t s);

}  // namespace wan
