// C ABI of libwanattn: host-side argument checks, then one kernel launch per
// call. Nothing is enqueued unless every check passes.
#include <math.h>
#include <stdint.h>

#include "../../include/wanattn.h"
#include "wan_internal.h"

namespace {

constexpr int kHeadDim = 128;
constexpr int kMaxC = 8192;
constexpr int kMaxGrid = 1024;  // length of the precomputed RoPE table on the pages

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte range [lo, hi) touched by a token-major tensor.
struct Range {
  uintptr_t lo, hi;
};

Range span_bf16(const void* p, int64_t rows, int64_t ld, int64_t width) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return {lo, lo + (uintptr_t)(((rows - 1) * ld + width) * 2)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Outputs may be exactly an input (in place, same stride); any other overlap
// is rejected.
bool bad_alias(const void* out, Range ro, int64_t ld_out, const void* in, Range ri,
               int64_t ld_in) {
  if (!out || !in) return false;
  if (out == in) return ld_out != ld_in;
  return overlap(ro, ri);
}

// Two token-major tensors of `rows` rows and C columns either touch disjoint
// byte ranges, or are column slices of the same rows (same stride, start
// offsets at least C apart and both inside one row).
bool slices_disjoint(const void* a, int64_t ld_a, const void* b, int64_t ld_b, int64_t rows,
                     int64_t C) {
  if (!overlap(span_bf16(a, rows, ld_a, C), span_bf16(b, rows, ld_b, C))) return true;
  if (ld_a != ld_b) return false;
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  const uintptr_t d = pa > pb ? pa - pb : pb - pa;
  return d >= (uintptr_t)(2 * C) && d <= (uintptr_t)(2 * (ld_a - C));
}

wanStatus_t from_hip(hipError_t e) {
  return e == hipSuccess ? WAN_SUCCESS : WAN_ERROR_LAUNCH;
}

// Shared checks of the two attention calls.
wanStatus_t check_attn(void* o, const float* lse, const void* q, const void* k,
                       const void* v, int B, int Lq, int Lk, int H, int D,
                       int64_t& ld_q, int64_t& ld_k, int64_t& ld_v, int64_t& ld_o,
                       float softmax_scale) {
  if (B < 0 || Lq < 0 || Lk < 1 || H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
  if (D != kHeadDim) return WAN_ERROR_NOT_SUPPORTED;
  if (!o || !q || !k || !v) return WAN_ERROR_INVALID_VALUE;
  if (!aligned16(o) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return WAN_ERROR_INVALID_VALUE;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return WAN_ERROR_INVALID_VALUE;
  const int64_t C = (int64_t)H * D;
  if (C > (int64_t)1 << 24) return WAN_ERROR_NOT_SUPPORTED;
  int64_t* lds[4] = {&ld_q, &ld_k, &ld_v, &ld_o};
  for (int64_t* ld : lds) {
    if (*ld == 0) *ld = C;
    if (*ld < C || (*ld & 7)) return WAN_ERROR_INVALID_VALUE;
  }
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return WAN_ERROR_INVALID_VALUE;
  const int64_t rq = (int64_t)B * Lq, rk = (int64_t)B * Lk;
  const Range ro = span_bf16(o, rq, ld_o, C);
  if (overlap(ro, span_bf16(q, rq, ld_q, C)) || overlap(ro, span_bf16(k, rk, ld_k, C)) ||
      overlap(ro, span_bf16(v, rk, ld_v, C)))
    return WAN_ERROR_INVALID_VALUE;
  if (lse) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(lse);
    const Range rl{lo, lo + (uintptr_t)((int64_t)B * H * Lq * 4)};
    if (overlap(rl, ro) || overlap(rl, span_bf16(q, rq, ld_q, C)) ||
        overlap(rl, span_bf16(k, rk, ld_k, C)) || overlap(rl, span_bf16(v, rk, ld_v, C)))
      return WAN_ERROR_INVALID_VALUE;
  }
  if ((int64_t)B * H * ((Lq + 127) / 128) > 0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;
  // K/V of one (batch, head) are addressed with 32-bit byte offsets.
  if ((int64_t)Lk * (ld_k > ld_v ? ld_k : ld_v) * 2 > (int64_t)0xffffffff)
    return WAN_ERROR_NOT_SUPPORTED;
  return WAN_SUCCESS;
}

}  // namespace

extern "C" {

const char* wan_status_string(wanStatus_t status) {
  switch (status) {
    case WAN_SUCCESS: return "WAN_SUCCESS";
    case WAN_ERROR_INVALID_VALUE: return "WAN_ERROR_INVALID_VALUE";
    case WAN_ERROR_NOT_SUPPORTED: return "WAN_ERROR_NOT_SUPPORTED";
    case WAN_ERROR_LAUNCH: return "WAN_ERROR_LAUNCH";
  }
  return "WAN_ERROR_UNKNOWN";
}

int wan_version(void) { return 100; }  // 0.1.0

wanStatus_t wan_qk_norm_rope3d(void* q_out, void* k_out, const void* q, const void* k,
                               const float* gain_q, const float* gain_k, int B, int L,
                               int H, int D, int grid_f, int grid_h, int grid_w,
                               int64_t ld_in, int64_t ld_out, float eps, float rope_theta,
                               unsigned flags, hipStream_t stream) {
  if (B < 0 || L < 0 || H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
  if (D != kHeadDim) return WAN_ERROR_NOT_SUPPORTED;
  const int64_t C = (int64_t)H * D;
  if (C > kMaxC) return WAN_ERROR_NOT_SUPPORTED;
  if (flags & ~(WAN_NORM | WAN_ROPE | WAN_NORM_PER_HEAD)) return WAN_ERROR_INVALID_VALUE;
  if ((flags & WAN_NORM_PER_HEAD) && !(flags & WAN_NORM)) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * L == 0) return WAN_SUCCESS;
  if (!q && !k) return WAN_ERROR_INVALID_VALUE;
  if ((q == nullptr) != (q_out == nullptr) || (k == nullptr) != (k_out == nullptr))
    return WAN_ERROR_INVALID_VALUE;
  const void* ptrs[4] = {q_out, k_out, q, k};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return WAN_ERROR_INVALID_VALUE;
  if ((gain_q && !aligned16(gain_q)) || (gain_k && !aligned16(gain_k)))
    return WAN_ERROR_INVALID_VALUE;
  if (ld_in == 0) ld_in = C;
  if (ld_out == 0) ld_out = C;
  if (ld_in < C || ld_out < C || (ld_in & 7) || (ld_out & 7)) return WAN_ERROR_INVALID_VALUE;
  if (!(eps >= 0.f) || isinf(eps)) return WAN_ERROR_INVALID_VALUE;
  if (flags & WAN_ROPE) {
    if (grid_f < 1 || grid_h < 1 || grid_w < 1 || grid_f > kMaxGrid || grid_h > kMaxGrid ||
        grid_w > kMaxGrid)
      return WAN_ERROR_INVALID_VALUE;
    if ((int64_t)grid_f * grid_h * grid_w != L) return WAN_ERROR_INVALID_VALUE;
    if (!(rope_theta > 1.f) || isinf(rope_theta)) return WAN_ERROR_INVALID_VALUE;
  }
  const int64_t rows = (int64_t)B * L;
  if (rows / 4 + 1 > 0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;
  // Outputs may equal their own input (in place, same stride). Otherwise an
  // output may share bytes with another tensor only as a disjoint column
  // slice of the same rows (q/k slices of one fused projection buffer).
  struct T {
    const void* p;
    int64_t ld;
  };
  const T outs[2] = {{q_out, ld_out}, {k_out, ld_out}};
  const T ins[2] = {{q, ld_in}, {k, ld_in}};
  if (q_out && k_out && !slices_disjoint(q_out, ld_out, k_out, ld_out, rows, C))
    return WAN_ERROR_INVALID_VALUE;
  for (int i = 0; i < 2; ++i) {
    if (!outs[i].p) continue;
    for (int j = 0; j < 2; ++j) {
      if (!ins[j].p) continue;
      if (i == j && outs[i].p == ins[j].p) {
        if (outs[i].ld != ins[j].ld) return WAN_ERROR_INVALID_VALUE;
        continue;
      }
      if (!slices_disjoint(outs[i].p, outs[i].ld, ins[j].p, ins[j].ld, rows, C))
        return WAN_ERROR_INVALID_VALUE;
    }
  }

  wan::NormRopeArgs a;
  a.q_out = q_out;
  a.k_out = k_out;
  a.q = q;
  a.k = k;
  a.gain_q = gain_q;
  a.gain_k = gain_k;
  a.rows = rows;
  a.L = L;
  a.H = H;
  a.D = D;
  a.grid_f = grid_f;
  a.grid_h = grid_h;
  a.grid_w = grid_w;
  a.ld_in = ld_in;
  a.ld_out = ld_out;
  a.eps = eps;
  a.log2_theta = (flags & WAN_ROPE) ? log2f(rope_theta) : 0.f;
  a.flags = flags;
  return from_hip(wan::launch_norm_rope(a, stream));
}

}  // extern "C"

namespace {

// Key split of a self-attention call on the current device (no split if the
// device cannot be queried).
wan::AttnSplit self_attn_split(int B, int L, int H) {
  int cus = 0;
  if (wan::device_cu_count(&cus) != hipSuccess) cus = 0;
  const int64_t items = (int64_t)B * H * ((L + wan::kAttnRows - 1) / wan::kAttnRows);
  return wan::plan_self_attn_split(items, (L + wan::kAttnKeys - 1) / wan::kAttnKeys, cus);
}

// Self-attention with the argument checks of check_attn; `part` (NULL: no
// split) receives the key-split partial results planned by `split`.
wanStatus_t self_attn(void* o, float* lse, const void* q, const void* k, const void* v,
                      const int32_t* k_lens, int B, int L, int H, int64_t ld_q, int64_t ld_k,
                      int64_t ld_v, int64_t ld_o, float softmax_scale, float* part,
                      const wan::AttnSplit& split, hipStream_t stream) {
  wan::AttnArgs a{};
  a.o = o;
  a.lse = lse;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_lens = k_lens;
  a.B = B;
  a.Lq = L;
  a.Lk = L;
  a.H = H;
  a.ld_q = ld_q;
  a.ld_k = ld_k;
  a.ld_v = ld_v;
  a.ld_o = ld_o;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)kHeadDim);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.q_offset = 0;
  a.chunk_len = 0;
  a.part = part;
  a.n_full = split.n_full;
  a.n_split = split.n_split;
  return from_hip(wan::launch_attn_fwd(a, 0, stream));
}

}  // namespace

extern "C" {

wanStatus_t wan_self_attn_fwd(void* o, float* lse, const void* q, const void* k, const void* v,
                              const int32_t* k_lens, int B, int L, int H, int D, int64_t ld_q,
                              int64_t ld_k, int64_t ld_v, int64_t ld_o, float softmax_scale,
                              hipStream_t stream) {
  if (B < 0 || L < 0) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * L == 0) {
    if (H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
    return D == kHeadDim ? WAN_SUCCESS : WAN_ERROR_NOT_SUPPORTED;
  }
  wanStatus_t st = check_attn(o, lse, q, k, v, B, L, L, H, D, ld_q, ld_k, ld_v, ld_o,
                              softmax_scale);
  if (st != WAN_SUCCESS) return st;
  const wan::AttnSplit none{(uint32_t)((int64_t)B * H * ((L + wan::kAttnRows - 1) / wan::kAttnRows)),
                            1, 0};
  return self_attn(o, lse, q, k, v, k_lens, B, L, H, ld_q, ld_k, ld_v, ld_o, softmax_scale,
                   nullptr, none, stream);
}

size_t wan_self_attn_workspace_size(int B, int L, int H, int D) {
  if (B < 1 || L < 1 || H < 1 || D != kHeadDim) return 0;
  return (size_t)self_attn_split(B, L, H).bytes;
}

wanStatus_t wan_self_attn_fwd_ws(void* o, float* lse, const void* q, const void* k,
                                 const void* v, const int32_t* k_lens, int B, int L, int H,
                                 int D, int64_t ld_q, int64_t ld_k, int64_t ld_v, int64_t ld_o,
                                 float softmax_scale, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (B < 0 || L < 0) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * L == 0) {
    if (H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
    return D == kHeadDim ? WAN_SUCCESS : WAN_ERROR_NOT_SUPPORTED;
  }
  wanStatus_t st = check_attn(o, lse, q, k, v, B, L, L, H, D, ld_q, ld_k, ld_v, ld_o,
                              softmax_scale);
  if (st != WAN_SUCCESS) return st;
  const wan::AttnSplit split = self_attn_split(B, L, H);
  float* part = nullptr;
  if (split.bytes > 0) {
    if (!workspace || !aligned16(workspace) || workspace_bytes < split.bytes)
      return WAN_ERROR_INVALID_VALUE;
    const int64_t C = (int64_t)H * D, rows = (int64_t)B * L;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(workspace);
    const Range rw{lo, lo + (uintptr_t)split.bytes};
    if (overlap(rw, span_bf16(o, rows, ld_o, C)) || overlap(rw, span_bf16(q, rows, ld_q, C)) ||
        overlap(rw, span_bf16(k, rows, ld_k, C)) || overlap(rw, span_bf16(v, rows, ld_v, C)))
      return WAN_ERROR_INVALID_VALUE;
    if (lse) {
      const uintptr_t ll = reinterpret_cast<uintptr_t>(lse);
      if (overlap(rw, Range{ll, ll + (uintptr_t)((int64_t)B * H * L * 4)}))
        return WAN_ERROR_INVALID_VALUE;
    }
    part = static_cast<float*>(workspace);
  }
  return self_attn(o, lse, q, k, v, k_lens, B, L, H, ld_q, ld_k, ld_v, ld_o, softmax_scale,
                   part, split, stream);
}

wanStatus_t wan_self_attn_fwd_noalloc(void* o, float* lse, const void* q, const void* k,
                                      const void* v, const int32_t* k_lens, int B, int L, int H,
                                      int D, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                      int64_t ld_o, float softmax_scale, hipStream_t stream) {
  if (B < 0 || L < 0) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * L == 0) {
    if (H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
    return D == kHeadDim ? WAN_SUCCESS : WAN_ERROR_NOT_SUPPORTED;
  }
  wanStatus_t st = check_attn(o, lse, q, k, v, B, L, L, H, D, ld_q, ld_k, ld_v, ld_o,
                              softmax_scale);
  if (st != WAN_SUCCESS) return st;
  const wan::AttnSplit split = self_attn_split(B, L, H);
  float* part = nullptr;
  if (split.bytes > 0) {
    void* p = nullptr;
    uint64_t bytes = 0;
    if (wan::device_scratch(&p, &bytes) != hipSuccess) return WAN_ERROR_LAUNCH;
    if (split.bytes > bytes) return WAN_ERROR_NOT_SUPPORTED;
    part = static_cast<float*>(p);
  }
  return self_attn(o, lse, q, k, v, k_lens, B, L, H, ld_q, ld_k, ld_v, ld_o, softmax_scale,
                   part, split, stream);
}

wanStatus_t wan_cross_attn_fwd(void* o, const void* q, const void* k, const void* v,
                               const int32_t* context_lens, int B, int Lq, int Lk, int H, int D,
                               int64_t ld_q, int64_t ld_kv, int64_t ld_o, float softmax_scale,
                               hipStream_t stream) {
  if (B < 0 || Lq < 0 || Lk < 1) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * Lq == 0) {
    if (H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
    return D == kHeadDim ? WAN_SUCCESS : WAN_ERROR_NOT_SUPPORTED;
  }
  int64_t ld_k = ld_kv, ld_v = ld_kv;
  wanStatus_t st = check_attn(o, nullptr, q, k, v, B, Lq, Lk, H, D, ld_q, ld_k, ld_v, ld_o,
                              softmax_scale);
  if (st != WAN_SUCCESS) return st;
  wan::AttnArgs a{};
  a.o = o;
  a.lse = nullptr;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_lens = context_lens;
  a.B = B;
  a.Lq = Lq;
  a.Lk = Lk;
  a.H = H;
  a.ld_q = ld_q;
  a.ld_k = ld_k;
  a.ld_v = ld_v;
  a.ld_o = ld_o;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.q_offset = 0;
  a.chunk_len = 0;
  return from_hip(wan::launch_attn_fwd(a, 1, stream));
}

wanStatus_t wan_chunk_causal_attn_fwd(void* o, float* lse, const void* q, const void* k,
                                      const void* v, const int32_t* k_lens, int B, int Lq,
                                      int Lk, int H, int D, int q_offset, int chunk_len,
                                      int64_t ld_q, int64_t ld_k, int64_t ld_v, int64_t ld_o,
                                      float softmax_scale, hipStream_t stream) {
  if (B < 0 || Lq < 0 || Lk < 1 || q_offset < 0 || chunk_len < 1) return WAN_ERROR_INVALID_VALUE;
  if ((int64_t)B * Lq == 0) {
    if (H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
    return D == kHeadDim ? WAN_SUCCESS : WAN_ERROR_NOT_SUPPORTED;
  }
  wanStatus_t st = check_attn(o, lse, q, k, v, B, Lq, Lk, H, D, ld_q, ld_k, ld_v, ld_o,
                              softmax_scale);
  if (st != WAN_SUCCESS) return st;
  wan::AttnArgs a{};
  a.o = o;
  a.lse = lse;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_lens = k_lens;
  a.B = B;
  a.Lq = Lq;
  a.Lk = Lk;
  a.H = H;
  a.ld_q = ld_q;
  a.ld_k = ld_k;
  a.ld_v = ld_v;
  a.ld_o = ld_o;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  a.q_offset = q_offset;
  a.chunk_len = chunk_len;
  return from_hip(wan::launch_attn_fwd(a, 2, stream));
}

wanStatus_t wan_adaln_modulate_gate(void* x_out, void* h_out, const void* x, const void* y,
                                    const float* gate, const float* shift, const float* scale,
                                    int B, int L, int C, int64_t mod_stride_b,
                                    int64_t mod_stride_l, float eps, hipStream_t stream) {
  if (B < 0 || L < 0 || C < 1) return WAN_ERROR_INVALID_VALUE;
  if (C & 7) return WAN_ERROR_INVALID_VALUE;
  if (C > kMaxC) return WAN_ERROR_NOT_SUPPORTED;
  if ((int64_t)B * L == 0) return WAN_SUCCESS;
  if (!x || (!x_out && !h_out)) return WAN_ERROR_INVALID_VALUE;
  const void* ptrs[7] = {x_out, h_out, x, y, gate, shift, scale};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return WAN_ERROR_INVALID_VALUE;
  if (mod_stride_b == 0) mod_stride_b = C;
  if (mod_stride_b < 0 || mod_stride_l < 0 || (mod_stride_b & 3) || (mod_stride_l & 3))
    return WAN_ERROR_INVALID_VALUE;
  if (!(eps >= 0.f) || isinf(eps)) return WAN_ERROR_INVALID_VALUE;
  const int64_t rows = (int64_t)B * L;
  if (rows / 4 + 1 > 0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;
  const Range rx = span_bf16(x, rows, C, C);
  const Range ry = y ? span_bf16(y, rows, C, C) : Range{0, 0};
  const Range rxo = x_out ? span_bf16(x_out, rows, C, C) : Range{0, 0};
  const Range rho = h_out ? span_bf16(h_out, rows, C, C) : Range{0, 0};
  if (x_out && h_out && overlap(rxo, rho)) return WAN_ERROR_INVALID_VALUE;
  if (bad_alias(x_out, rxo, C, x, rx, C) || bad_alias(x_out, rxo, C, y, ry, C) ||
      bad_alias(h_out, rho, C, x, rx, C) || bad_alias(h_out, rho, C, y, ry, C))
    return WAN_ERROR_INVALID_VALUE;

  wan::AdaLNArgs a;
  a.x_out = x_out;
  a.h_out = h_out;
  a.x = x;
  a.y = y;
  a.gate = y ? gate : nullptr;
  a.shift = shift;
  a.scale = scale;
  a.rows = rows;
  a.L = L;
  a.C = C;
  a.mod_stride_b = mod_stride_b;
  a.mod_stride_l = mod_stride_l;
  a.eps = eps;
  return from_hip(wan::launch_adaln(a, stream));
}

wanStatus_t wan_linear_fwd(void* y, const void* x, const void* w, const float* bias, int M,
                          int N, int K, int64_t ld_x, int64_t ld_w, int64_t ld_y,
                          hipStream_t stream) {
  if (M < 0 || N < 1 || K < 1) return WAN_ERROR_INVALID_VALUE;
  if (M == 0) return WAN_SUCCESS;
  if (!y || !x || !w) return WAN_ERROR_INVALID_VALUE;
  if (!aligned16(y) || !aligned16(x) || !aligned16(w) || (bias && !aligned16(bias)))
    return WAN_ERROR_INVALID_VALUE;
  if ((N & 7) || (K & 7)) return WAN_ERROR_INVALID_VALUE;
  if (ld_x == 0) ld_x = K;
  if (ld_w == 0) ld_w = K;
  if (ld_y == 0) ld_y = N;
  if (ld_x < K || ld_w < K || ld_y < N || ((ld_x | ld_w | ld_y) & 7))
    return WAN_ERROR_INVALID_VALUE;
  // 256 rows of x or W must fit one 32-bit buffer range.
  if (256 * (ld_x > ld_w ? ld_x : ld_w) * 2 > (int64_t)0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;
  const Range ry = span_bf16(y, M, ld_y, N);
  if (overlap(ry, span_bf16(x, M, ld_x, K)) || overlap(ry, span_bf16(w, N, ld_w, K)))
    return WAN_ERROR_INVALID_VALUE;
  if (bias) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(bias);
    if (overlap(ry, Range{lo, lo + (uintptr_t)N * 4})) return WAN_ERROR_INVALID_VALUE;
  }
  wan::LinearArgs a{y, x, w, bias, M, N, K, ld_x, ld_w, ld_y};
  return from_hip(wan::launch_linear(a, stream));
}

wanStatus_t wan_quantize_qkv_8bit(int8_t* q8, int8_t* k8, uint8_t* v8, float* q_scale,
                                  float* k_scale, uint8_t* v_scale, const void* q, const void* k,
                                  const void* v, const int32_t* k_lens, int B, int L, int H,
                                  int D, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                  hipStream_t stream) {
  if (B < 0 || L < 0 || H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
  if (D != kHeadDim) return WAN_ERROR_NOT_SUPPORTED;
  if ((int64_t)B * L == 0) return WAN_SUCCESS;
  const void* ptrs[9] = {q8, k8, v8, q_scale, k_scale, v_scale, q, k, v};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return WAN_ERROR_INVALID_VALUE;
  const int64_t C = (int64_t)H * D;
  if (C > (int64_t)1 << 24) return WAN_ERROR_NOT_SUPPORTED;
  int64_t* lds[3] = {&ld_q, &ld_k, &ld_v};
  for (int64_t* ld : lds) {
    if (*ld == 0) *ld = C;
    if (*ld < C || (*ld & 7)) return WAN_ERROR_INVALID_VALUE;
  }
  // outputs: codes B*H*nT*64*D bytes each, scales B*H*nT floats / B*H*nT*256 bytes
  const int64_t nT = (L + 63) / 64, tiles = (int64_t)B * H * nT;
  if (tiles > 0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;   // one workgroup per block
  const Range outs[6] = {
      {reinterpret_cast<uintptr_t>(q8), reinterpret_cast<uintptr_t>(q8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(k8), reinterpret_cast<uintptr_t>(k8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(v8), reinterpret_cast<uintptr_t>(v8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(q_scale), reinterpret_cast<uintptr_t>(q_scale) + (uintptr_t)(tiles * 4)},
      {reinterpret_cast<uintptr_t>(k_scale), reinterpret_cast<uintptr_t>(k_scale) + (uintptr_t)(tiles * 4)},
      {reinterpret_cast<uintptr_t>(v_scale), reinterpret_cast<uintptr_t>(v_scale) + (uintptr_t)(tiles * 256)}};
  const int64_t rows = (int64_t)B * L;
  const Range ins[3] = {span_bf16(q, rows, ld_q, C), span_bf16(k, rows, ld_k, C),
                        span_bf16(v, rows, ld_v, C)};
  for (int i = 0; i < 6; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], ins[j])) return WAN_ERROR_INVALID_VALUE;
    for (int j = i + 1; j < 6; ++j)
      if (overlap(outs[i], outs[j])) return WAN_ERROR_INVALID_VALUE;
  }
  if (k_lens && (reinterpret_cast<uintptr_t>(k_lens) & 3u)) return WAN_ERROR_INVALID_VALUE;
  wan::Quant8Args a{q8, k8, v8, q_scale, k_scale, v_scale, q, k, v, k_lens,
                    B, L, H, ld_q, ld_k, ld_v};
  return from_hip(wan::launch_quant8(a, stream));
}

wanStatus_t wan_self_attn_fwd_8bit(void* o, float* lse, const int8_t* q8, const int8_t* k8,
                                   const uint8_t* v8, const float* q_scale,
                                   const float* k_scale, const uint8_t* v_scale,
                                   const int32_t* k_lens, int B, int L, int H, int D,
                                   int64_t ld_o, float softmax_scale, hipStream_t stream) {
  if (B < 0 || L < 0 || H < 1 || D < 1) return WAN_ERROR_INVALID_VALUE;
  if (D != kHeadDim) return WAN_ERROR_NOT_SUPPORTED;
  if ((int64_t)B * L == 0) return WAN_SUCCESS;
  const void* ptrs[7] = {o, q8, k8, v8, q_scale, k_scale, v_scale};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return WAN_ERROR_INVALID_VALUE;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return WAN_ERROR_INVALID_VALUE;
  const int64_t C = (int64_t)H * D;
  if (C > (int64_t)1 << 24) return WAN_ERROR_NOT_SUPPORTED;
  if (ld_o == 0) ld_o = C;
  if (ld_o < C || (ld_o & 7)) return WAN_ERROR_INVALID_VALUE;
  if (!(softmax_scale == softmax_scale) || isinf(softmax_scale)) return WAN_ERROR_INVALID_VALUE;
  const int64_t nT = (L + 63) / 64, tiles = (int64_t)B * H * nT;
  if (nT > 4096) return WAN_ERROR_NOT_SUPPORTED;   // key-block scales held in LDS
  if ((int64_t)B * H * ((L + 255) / 256) > 0x7fffffff) return WAN_ERROR_NOT_SUPPORTED;
  const Range ro = span_bf16(o, (int64_t)B * L, ld_o, C);
  const Range ins[6] = {
      {reinterpret_cast<uintptr_t>(q8), reinterpret_cast<uintptr_t>(q8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(k8), reinterpret_cast<uintptr_t>(k8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(v8), reinterpret_cast<uintptr_t>(v8) + (uintptr_t)(tiles * 64 * D)},
      {reinterpret_cast<uintptr_t>(q_scale), reinterpret_cast<uintptr_t>(q_scale) + (uintptr_t)(tiles * 4)},
      {reinterpret_cast<uintptr_t>(k_scale), reinterpret_cast<uintptr_t>(k_scale) + (uintptr_t)(tiles * 4)},
      {reinterpret_cast<uintptr_t>(v_scale), reinterpret_cast<uintptr_t>(v_scale) + (uintptr_t)(tiles * 256)}};
  for (const Range& r : ins)
    if (overlap(ro, r)) return WAN_ERROR_INVALID_VALUE;
  if (lse) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(lse);
    const Range rl{lo, lo + (uintptr_t)((int64_t)B * H * L * 4)};
    if (overlap(rl, ro)) return WAN_ERROR_INVALID_VALUE;
    for (const Range& r : ins)
      if (overlap(rl, r)) return WAN_ERROR_INVALID_VALUE;
  }
  wan::Attn8Args a{};
  a.o = o;
  a.lse = lse;
  a.q8 = q8;
  a.k8 = k8;
  a.v8 = v8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.k_lens = k_lens;
  a.B = B;
  a.L = L;
  a.H = H;
  a.ld_o = ld_o;
  const float sc = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
  a.scale_log2 = sc * 1.4426950408889634f;
  return from_hip(wan::launch_attn8_fwd(a, stream));
}

}  // extern "C"
