/*
 * wanattn: the attention sublayer of a Wan2.1/2.2 DiT block (WanAttentionBlock)
 * on AMD Instinct MI355X (gfx950).
 *
 * The four compute calls follow the block as the "Wan2.2 code walkthrough"
 * page (newtid.com repost) shows it:
 *
 *   y = self_attn(norm1(x) * (1 + e[1]) + e[0], seq_lens, grid_sizes, freqs)
 *         -> q/k RMSNorm, rope_apply(q), rope_apply(k), flash_attention(...)
 *   x = x + y * e[2]
 *   x = x + cross_attn(norm3(x), context, context_lens)
 *
 * and the paper deep dive "论文专题讲解：Wan2.1：开源视频生成系统路线"
 * (section "Video DiT 与 Flow Matching": full spatio-temporal self-attention,
 * cross-attention to the 512-token umT5 text context).
 *
 * wan_linear_fwd computes the q/k/v and output projections between them
 * (bf16 Linear layers); wan_chunk_causal_attn_fwd is the chunk-wise
 * autoregressive variant of the self-attention; wan_quantize_qkv_8bit and
 * wan_self_attn_fwd_8bit are its 8-bit (INT8 / FP8) variant.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every call returns a wanStatus_t. Arguments are checked on the host
 *   before anything is enqueued; on an error nothing is launched.
 * - Tensor pointers are caller-owned DEVICE memory. bf16 tensors are passed
 *   as void* holding IEEE bfloat16 bit patterns and must be 16-byte aligned;
 *   fp32 vectors must be 16-byte aligned too.
 * - The library allocates nothing, frees nothing, keeps no pointer and no
 *   state between calls, and never synchronises: work is enqueued on
 *   `stream` (NULL = the default stream) and device faults surface at the
 *   caller's next synchronisation. Calls are reentrant and thread-safe.
 * - Token-major tensors [B, L, H, D] address element (b, l, h, d) at
 *   ptr[(b * L + l) * ld + h * D + d]; `ld` (elements between consecutive
 *   tokens) may exceed H*D so that slices of a fused buffer can be passed;
 *   ld = 0 means H*D. ld must be a multiple of 8.
 * - D (head size) must be 128; otherwise WAN_ERROR_NOT_SUPPORTED.
 * - A call whose B or L (Lq) is 0 has nothing to do and returns
 *   WAN_SUCCESS without reading any pointer.
 */
#ifndef WANATTN_H_
#define WANATTN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wanStatus {
  WAN_SUCCESS = 0,
  WAN_ERROR_INVALID_VALUE = 1,  /* bad pointer, size, stride, alias or flag */
  WAN_ERROR_NOT_SUPPORTED = 2,  /* valid request outside what is built (D != 128, C too large) */
  WAN_ERROR_LAUNCH = 3          /* the HIP runtime refused the launch */
} wanStatus_t;

/* Flags of wan_qk_norm_rope3d. */
#define WAN_NORM 1u          /* RMSNorm of each token row, times the gain */
#define WAN_ROPE 2u          /* 3D RoPE over the (f, h, w) grid */
#define WAN_NORM_PER_HEAD 4u /* RMSNorm over each head's D channels instead of the H*D row */

/* Static string for a status code. */
const char* wan_status_string(wanStatus_t status);

/* Library version as major * 10000 + minor * 100 + patch. */
int wan_version(void);

/*
 * wan_qk_norm_rope3d: q/k RMSNorm fused with 3D RoPE.
 *
 * Passage: WanAttentionBlock self-attention (q/k RMSNorm, then
 * rope_apply(q, grid_sizes, freqs) and rope_apply(k, ...); V is not rotated)
 * and the 3D RoPE snippet of the "Wan2.2 code walkthrough" page: the
 * d/2 = 64 complex frequencies of a head are split [c - 2(c//3), c//3, c//3]
 * = 22/21/21 between the t, h and w axes, broadcast over the flattened grid
 * (token n = (t*h + y)*w + x, w fastest) and applied as a complex multiply
 * on interleaved (re, im) pairs. "初识wan系列模型" (huan-yin.github.io), "3D RoPE
 * 坐标体系的建立与预计算", gives each token its (t, y, x) coordinates.
 *
 * For each token row r of q (and of k):
 *   WAN_NORM:  r <- r / sqrt(mean(r^2) + eps) * gain   (mean over H*D, or over
 *              each head's D with WAN_NORM_PER_HEAD; gain NULL = 1)
 *   WAN_ROPE:  pair j of every head rotates by pos_a * theta^(-2 j' / D_a),
 *              a = axis of j, j' = index of j inside that axis, D_a = 2 * (pairs
 *              of that axis), pos = (t, y, x) of the token
 * computed in fp32 and stored as bf16 (round to nearest even).
 *
 * q_out, k_out   bf16 [B, L, H, D], row stride ld_out. May equal q / k
 *                (in place; then ld_out must equal ld_in).
 * q, k           bf16 [B, L, H, D], row stride ld_in. Either may be NULL
 *                (then its output must be NULL too), not both.
 * gain_q, gain_k fp32 [H*D] RMSNorm gains, or NULL for 1.
 * grid_f/h/w     latent-patch grid; with WAN_ROPE, f*h*w must equal L and each
 *                of f, h, w must be in [1, 1024].
 * eps            RMSNorm epsilon (>= 0), e.g. 1e-6.
 * rope_theta     RoPE base (> 1), e.g. 10000.
 * flags          any OR of WAN_NORM, WAN_ROPE, WAN_NORM_PER_HEAD (PER_HEAD only
 *                with WAN_NORM).
 * Errors: WAN_ERROR_INVALID_VALUE for NULL/misaligned pointers, bad sizes or
 * strides, partial overlap between an input and an output, bad flags or a
 * grid that does not match L; WAN_ERROR_NOT_SUPPORTED for D != 128 or
 * H*D > 8192.
 */
wanStatus_t wan_qk_norm_rope3d(void* q_out, void* k_out, const void* q,
                               const void* k, const float* gain_q,
                               const float* gain_k, int B, int L, int H, int D,
                               int grid_f, int grid_h, int grid_w,
                               int64_t ld_in, int64_t ld_out, float eps,
                               float rope_theta, unsigned flags,
                               hipStream_t stream);

/*
 * wan_self_attn_fwd: full non-causal softmax self-attention.
 *
 * Passage: WanSelfAttention.forward on the "Wan2.2 code walkthrough" page,
 * flash_attention(q = rope(q), k = rope(k), v, k_lens = seq_lens,
 * window_size = (-1, -1)): a global window and no causal mask, so every video
 * token attends to every token of past, present and future frames.
 *
 * For every (b, h) and query row i:
 *   o[b,i,h,:] = sum_{j < n_b} softmax_j(scale * q_i . k_j) v_j,
 *   n_b = clamp(k_lens[b], 0, L) (k_lens NULL: n_b = L),
 *   lse[b,h,i] = log(sum_{j < n_b} exp(scale * q_i . k_j))  (natural log).
 * n_b = 0 gives o = 0 and lse = -inf. bf16 MFMA products, fp32 accumulation,
 * fp32 running max and sum; o is stored as bf16.
 *
 * o        bf16 [B, L, H, D], row stride ld_o; must not overlap q, k or v.
 * lse      fp32 [B, H, L] or NULL; must not overlap the other tensors.
 * q, k, v  bf16 [B, L, H, D], row strides ld_q, ld_k, ld_v.
 * k_lens   device int32 [B] or NULL. Read on the device, so not checked on
 *          the host: values are clamped to [0, L].
 * softmax_scale  > 0, or <= 0 for 1/sqrt(D).
 * Errors: WAN_ERROR_INVALID_VALUE (NULL/misaligned pointers, bad sizes or
 * strides, o overlapping an input), WAN_ERROR_NOT_SUPPORTED (D != 128, or the
 * keys of one (batch, head) spanning more than 4 GiB: L * max(ld_k, ld_v) * 2
 * bytes, since they are addressed with 32-bit byte offsets).
 */
wanStatus_t wan_self_attn_fwd(void* o, float* lse, const void* q,
                              const void* k, const void* v,
                              const int32_t* k_lens, int B, int L, int H,
                              int D, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                              int64_t ld_o, float softmax_scale,
                              hipStream_t stream);

/*
 * wan_self_attn_workspace_size / wan_self_attn_fwd_ws: wan_self_attn_fwd with
 * a caller-owned workspace, which lets the library even out the last round of
 * work on the current device.
 *
 * Same passage and arithmetic as wan_self_attn_fwd. The call runs one work
 * item (256 query rows of one (batch, head)) per compute unit at a time;
 * when the items of the last round would leave at least half of the device
 * idle, each of them is split into key ranges that run on the idle units,
 * and a second kernel combines their partial results: for ranges s with
 * running maxima m_s, sums l_s and unnormalised outputs O_s,
 *   o = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s,
 * the exact softmax over the union of the ranges (up to fp32 rounding), so o
 * and lse match wan_self_attn_fwd to rounding.
 *
 * wan_self_attn_workspace_size returns the bytes of workspace a call with
 * these sizes needs on the current device (0: no split, the workspace is not
 * used and may be NULL; also 0 for sizes wan_self_attn_fwd would reject).
 * workspace: device memory of at least that many bytes, 16-byte aligned,
 * overlapping no other argument; its contents on entry do not matter and are
 * left undefined. Calls that run at the same time need separate workspaces.
 * Errors: as wan_self_attn_fwd, and WAN_ERROR_INVALID_VALUE for a workspace
 * that is needed and NULL, misaligned, too small or overlapping a tensor.
 */
size_t wan_self_attn_workspace_size(int B, int L, int H, int D);

wanStatus_t wan_self_attn_fwd_ws(void* o, float* lse, const void* q,
                                 const void* k, const void* v,
                                 const int32_t* k_lens, int B, int L, int H,
                                 int D, int64_t ld_q, int64_t ld_k,
                                 int64_t ld_v, int64_t ld_o,
                                 float softmax_scale, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * wan_self_attn_fwd_noalloc: wan_self_attn_fwd_ws without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, arithmetic and errors as wan_self_attn_fwd, same results
 * as wan_self_attn_fwd_ws. The key-split partial results go to a static
 * device array of the library (34 MB, one per device, kept until the process
 * ends; its address is looked up on the first call on each device). The call
 * allocates and frees nothing. Every call on one device shares that array:
 * calls that overlap on one device (other streams, other threads) race and
 * must be serialised by the caller. A split needing more than the array
 * (a device of more than 256 compute units) returns WAN_ERROR_NOT_SUPPORTED;
 * a failed address lookup returns WAN_ERROR_LAUNCH.
 */
wanStatus_t wan_self_attn_fwd_noalloc(void* o, float* lse, const void* q,
                                      const void* k, const void* v,
                                      const int32_t* k_lens, int B, int L,
                                      int H, int D, int64_t ld_q, int64_t ld_k,
                                      int64_t ld_v, int64_t ld_o,
                                      float softmax_scale, hipStream_t stream);

/*
 * wan_cross_attn_fwd: cross-attention of video tokens to text tokens.
 *
 * Passage: cross_attn(norm3(x), context, context_lens) in the WanAttentionBlock
 * snippet of the "Wan2.2 code walkthrough" page; the context is the 512-token
 * umT5 text embedding projected to the model width ("论文专题讲解：Wan2.1",
 * section "Video DiT 与 Flow Matching"). No RoPE.
 *
 * Same arithmetic as wan_self_attn_fwd with Lq query rows and Lk keys:
 *   o[b,i,h,:] = sum_{j < n_b} softmax_j(scale * q_i . k_j) v_j,
 *   n_b = clamp(context_lens[b], 0, Lk) (NULL: Lk); n_b = 0 gives o = 0.
 *
 * o      bf16 [B, Lq, H, D], row stride ld_o; must not overlap q, k or v.
 * q      bf16 [B, Lq, H, D], row stride ld_q.
 * k, v   bf16 [B, Lk, H, D], row stride ld_kv (shared by k and v).
 * context_lens  device int32 [B] or NULL.
 * Errors: as wan_self_attn_fwd; Lk must be >= 1.
 */
wanStatus_t wan_cross_attn_fwd(void* o, const void* q, const void* k,
                               const void* v, const int32_t* context_lens,
                               int B, int Lq, int Lk, int H, int D,
                               int64_t ld_q, int64_t ld_kv, int64_t ld_o,
                               float softmax_scale, hipStream_t stream);

/*
 * wan_chunk_causal_attn_fwd: self-attention under chunk-wise autoregression.
 *
 * Passage: the causalization discussion of the "Wan2.2 code walkthrough" page
 * (turning the bidirectional video denoiser into a world model): the video is
 * generated chunk by chunk, tokens of the chunk being denoised attend to each
 * other and to the chunks already observed or generated (a KV cache), never to
 * later ones.
 *
 * Query row i is the token at global position q_offset + i; key j is at
 * position j; chunk(x) = floor(x / chunk_len). Key j is visible to row i iff
 *   j < n_b  and  chunk(j) <= chunk(q_offset + i),   n_b = clamp(k_lens[b], 0, Lk).
 * o and lse as in wan_self_attn_fwd over the visible keys (no visible key:
 * o = 0, lse = -inf). Tiles of keys no row of a workgroup can see are skipped,
 * so a full causal pass costs about half of full attention.
 * chunk_len >= Lk + q_offset + Lq gives full attention; chunk_len = 1 with
 * q_offset = 0 gives token-causal attention. Typical use: q_offset = Lk - Lq
 * (the newest Lq tokens against cache + themselves), chunk_len = tokens of a
 * chunk of latent frames (frames * h * w).
 *
 * o      bf16 [B, Lq, H, D], row stride ld_o; must not overlap q, k or v.
 * lse    fp32 [B, H, Lq] or NULL.
 * q      bf16 [B, Lq, H, D], row stride ld_q.
 * k, v   bf16 [B, Lk, H, D], row strides ld_k, ld_v.
 * Errors: as wan_self_attn_fwd; Lk >= 1, q_offset >= 0 and chunk_len >= 1
 * are required (WAN_ERROR_INVALID_VALUE otherwise).
 */
wanStatus_t wan_chunk_causal_attn_fwd(void* o, float* lse, const void* q,
                                      const void* k, const void* v,
                                      const int32_t* k_lens, int B, int Lq,
                                      int Lk, int H, int D, int q_offset,
                                      int chunk_len, int64_t ld_q,
                                      int64_t ld_k, int64_t ld_v, int64_t ld_o,
                                      float softmax_scale, hipStream_t stream);

/*
 * wan_adaln_modulate_gate: residual update + AdaLN-modulated LayerNorm.
 *
 * Passage: the WanAttentionBlock snippet of the "Wan2.2 code walkthrough" page:
 * e = (modulation + e).chunk(6) gives shift, scale, gate, shift2, scale2,
 * gate2; norm1(x).float() * (1 + e[1]) + e[0] feeds self-attention;
 * x = x + y * e[2] is the gated residual; x = x + cross_attn(norm3(x), ...)
 * is the ungated one. norm1/norm2 are LayerNorms computed in fp32.
 *
 * Per token row (C channels), in fp32:
 *   r = x + gate * y    (y NULL: r = x; gate NULL: r = x + y)
 *   x_out = bf16(r)                                  (if x_out != NULL)
 *   h_out = bf16((r - mean(r)) / sqrt(var(r) + eps) * (1 + scale) + shift)
 *                                                    (if h_out != NULL)
 * with the population variance and shift/scale NULL meaning 0. h is taken
 * from the unrounded r. norm3 with affine (gamma, beta) is this call with
 * scale = gamma - 1 and shift = beta.
 *
 * x_out, h_out  bf16 [B, L, C] dense; at least one non-NULL; they must not
 *               overlap each other. Either may be the same pointer as x or
 *               y (in place); partial overlaps are rejected.
 * x, y          bf16 [B, L, C] dense; y may be NULL.
 * gate, shift, scale  fp32, element (b, l, c) at ptr[b*mod_stride_b +
 *               l*mod_stride_l + c]: mod_stride_l = 0 broadcasts one vector
 *               per sample over the tokens (per-sample modulation, [B, 6, C]
 *               chunks use mod_stride_b = 6C); mod_stride_l = C or 6C gives
 *               per-token modulation. mod_stride_b = 0 means C.
 * C must be a multiple of 8 and at most 8192.
 */
wanStatus_t wan_adaln_modulate_gate(void* x_out, void* h_out, const void* x,
                                    const void* y, const float* gate,
                                    const float* shift, const float* scale,
                                    int B, int L, int C, int64_t mod_stride_b,
                                    int64_t mod_stride_l, float eps,
                                    hipStream_t stream);

/*
 * wan_linear_fwd: projection y = x W^T + b (a torch nn.Linear in bf16).
 *
 * Passage: the WanModel snippet of the "Wan2.2 code walkthrough" page builds
 * the model from nn.Linear layers (weight [out, in], bias [out]); the q, k, v
 * and o projections of self- and cross-attention are such layers of width
 * dim. "论文专题讲解：Wan2.1", section "大规模训练系统", gives their cost as the
 * alpha * b * s * h^2 term beside attention's beta * b * s^2 * h.
 *
 *   y[m, n] = bf16( sum_k x[m, k] * w[n, k] + bias[n] )
 * with bf16 MFMA products, fp32 accumulation, the bias added in fp32 and one
 * round to nearest even.
 *
 * y     bf16 [M, N], row stride ld_y (e.g. the q, k, v thirds of a fused
 *       [M, 3C] buffer: pass N = 3C with W = [Wq; Wk; Wv], or one slice).
 *       Must not overlap x, w or bias.
 * x     bf16 [M, K], row stride ld_x (tokens: M = B * L).
 * w     bf16 [N, K], row stride ld_w.
 * bias  fp32 [N] or NULL (no bias).
 * N and K must be multiples of 8; ld = 0 means the dense stride.
 * Errors: WAN_ERROR_INVALID_VALUE for NULL/misaligned pointers, bad sizes or
 * strides, y overlapping an input; WAN_ERROR_NOT_SUPPORTED when 256 rows of
 * x or w span more than 2^31 bytes.
 */
wanStatus_t wan_linear_fwd(void* y, const void* x, const void* w,
                           const float* bias, int M, int N, int K,
                           int64_t ld_x, int64_t ld_w, int64_t ld_y,
                           hipStream_t stream);

/*
 * 8-bit self-attention: wan_quantize_qkv_8bit, then wan_self_attn_fwd_8bit.
 *
 * Passage: "论文专题讲解：Wan2.1", inference-optimisation table, row "8-bit
 * FlashAttention": INT8 for S = Q K^T, FP8 for O = P V, FP32 accumulation
 * across key blocks. The table gives no granularity; this library takes:
 *   q, k: symmetric INT8 per (batch, head, block of 64 tokens), fp32 scale
 *         amax / 127, code = round_half_even(x * (127 / amax)) in fp32,
 *         clamped to +-127 (amax = 0: codes and scale 0).
 *   v:    FP8 E4M3 (OCP E4M3FN) per (batch, head, channel, 32 keys) with a
 *         power-of-two scale 2^e, e = floor(log2 amax) - 8 (OCP microscaling;
 *         the scale byte is e + 127, amax = 0 gives byte 0), element =
 *         E4M3(clamp(v / 2^e, +-448)) rounded to nearest even.
 *   Keys and values at or past k_lens[b] are padding: they are quantised as
 *         zeros and left out of their blocks' scales.
 *   P:    E4M3 of 2^(t - m), t the scaled score in log2 units and m an integer
 *         running maximum; the softmax denominator sums the unrounded
 *         2^(t - m) in fp32 (only the operand of the P V product is FP8).
 * Quantised layouts (nT = ceil(L / 64); rows past L are zero):
 *   q8, k8   int8  [B][H][nT][64][D]          (token blocks, row-major)
 *   q_scale, k_scale  fp32 [B][H][nT]
 *   v8       uint8 [B][H][nT][D][64]          (E4M3, each block transposed)
 *   v_scale  uint8 [B][H][nT][2][32][D / 32]  (E8M0: [key half][channel % 32]
 *                                             [channel / 32])
 * All buffers are caller-owned device memory, 16-byte aligned.
 */

/*
 * wan_quantize_qkv_8bit: quantise q, k, v ([B, L, H, D] bf16, row strides
 * ld_q, ld_k, ld_v; ld = 0 means H*D) into the layouts above. Outputs must
 * not overlap each other or the inputs. k_lens: device int32 [B] or NULL
 * (= L), clamped to [0, L]; key and value rows at or past it are never read
 * (they may hold anything, inf and NaN included) and quantise as zeros.
 * Pass the same k_lens to wan_self_attn_fwd_8bit. All query rows are
 * quantised: a non-finite q value spoils the scale of its 64-row block.
 * Errors: WAN_ERROR_INVALID_VALUE for NULL/misaligned pointers, bad sizes or
 * strides, overlaps; WAN_ERROR_NOT_SUPPORTED for D != 128, H*D > 2^24, or
 * B*H*nT > 2^31 - 1 (one workgroup per block).
 */
wanStatus_t wan_quantize_qkv_8bit(int8_t* q8, int8_t* k8, uint8_t* v8,
                                  float* q_scale, float* k_scale,
                                  uint8_t* v_scale, const void* q,
                                  const void* k, const void* v,
                                  const int32_t* k_lens, int B, int L, int H,
                                  int D, int64_t ld_q, int64_t ld_k,
                                  int64_t ld_v, hipStream_t stream);

/*
 * wan_self_attn_fwd_8bit: self-attention of the quantised q over the
 * quantised k, v (all L tokens, keys masked by k_lens as in
 * wan_self_attn_fwd):
 *   S_ij = sum_d q8_id k8_jd (exact), mult = sq_i sk_j scale log2(e),
 *   m_i integer, p_ij = 2^(S_ij mult - m_i), P_ij = E4M3(p_ij),
 *   o_i = sum_j P_ij v_j / sum_j p_ij  (v dequantised),
 *   lse_i = ln 2 (m_i + log2 sum_j p_ij).
 * INT8 MFMA for S, FP8 MFMA with hardware block scales for P V, fp32
 * accumulation; o is stored as bf16.
 * o      bf16 [B, L, H, D], row stride ld_o; must not overlap the inputs.
 * lse    fp32 [B, H, L] or NULL.
 * k_lens device int32 [B] or NULL (clamped to [0, L]).
 * softmax_scale  > 0, or <= 0 for 1/sqrt(D).
 * Errors: WAN_ERROR_INVALID_VALUE (NULL/misaligned pointers, bad sizes,
 * overlaps), WAN_ERROR_NOT_SUPPORTED (D != 128, H*D > 2^24, L > 262144, or
 * more than 2^31 - 1 workgroups: B*H*ceil(L / 256)).
 */
wanStatus_t wan_self_attn_fwd_8bit(void* o, float* lse, const int8_t* q8,
                                   const int8_t* k8, const uint8_t* v8,
                                   const float* q_scale, const float* k_scale,
                                   const uint8_t* v_scale,
                                   const int32_t* k_lens, int B, int L, int H,
                                   int D, int64_t ld_o, float softmax_scale,
                                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WANATTN_H_ */
