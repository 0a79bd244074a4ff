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
  // Self-attention only: when part is not NULL, work items n_full and later
  // are split into n_split key ranges whose partial results go to part and
  // are combined by a second kernel (see plan_self_attn_split).
  float* part;
  uint32_t n_full;
  int n_split;
};

// Self-attention work items are 256 query rows of one (batch, head); keys are
// streamed in tiles of 64.
constexpr int kAttnRows = 256;
constexpr int kAttnKeys = 64;
// Floats of one key-split partial result: O [256][128] unnormalised, then
// the running maximum m [256] (log2 units) and the sum l [256].
constexpr uint64_t kAttnPartFloats = (uint64_t)kAttnRows * 128 + 2 * kAttnRows;

// Key split of the last round of self-attention work items. With `items`
// items of `n_tiles` key tiles each and one item per CU at a time, the last
// items % cus items would run on a partly idle chip; when they are at most
// half of it, each is split into n_split key ranges instead (up to one per
// idle CU), whose partial results need `bytes` of workspace. n_split = 1:
// no split.
struct AttnSplit {
  uint32_t n_full;
  int n_split;
  uint64_t bytes;
};

inline AttnSplit plan_self_attn_split(int64_t items, int n_tiles, int cus) {
  AttnSplit none{(uint32_t)items, 1, 0};
  if (cus <= 0 || n_tiles < 32 || items <= 0) return none;
  const int64_t tail = items % cus;
  if (tail == 0 || 2 * tail > cus) return none;
  int64_t split = cus / tail;
  if (split > n_tiles) split = n_tiles;
  if (split < 2) return none;
  return AttnSplit{(uint32_t)(items - tail), (int)split,
                   (uint64_t)(tail * split) * kAttnPartFloats * 4};
}

// Compute units of the current device (cached per device).
hipError_t device_cu_count(int* n);
// Device address and size of the library's static scratch array on the
// current device (looked up once per device).
hipError_t device_scratch(void** p, uint64_t* bytes);

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
  const int32_t* k_lens;   // device [B] or NULL: key/value rows at or past it are zero
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
