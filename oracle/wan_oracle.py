"""float64 CPU oracle for the attention sublayer of a Wan DiT block.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by tests, the smoke
check and the benchmark's CPU-baseline leg, never by the product path.

Sources (the pages this follows; each function names its passage):

* "Wan2.2 code walkthrough" (newtid.com repost of the AUTOHUB article),
  the WanAttentionBlock snippet (norm1 -> modulate -> self_attn -> gated
  residual -> cross_attn(norm3(x)) -> modulated FFN), the 3D RoPE snippet
  (frequency split ``[c - 2(c//3), c//3, c//3]``, broadcast over the (f,h,w)
  grid, complex multiply, ``view_as_real(...).flatten``) and the
  self-attention snippet (RoPE on q and k only, ``k_lens=seq_lens``, global
  window, no causal mask).
* "论文专题讲解：Wan2.1：开源视频生成系统路线" (charles2530.github.io), section
  "Video DiT 与 Flow Matching": full spatio-temporal self-attention plus
  cross-attention to 512 umT5 text tokens.
* "初识wan系列模型" (huan-yin.github.io), "3D RoPE 坐标体系的建立与预计算" and
  "Spatio-Temporal Transformer Blocks 运算流": every token gets (t, y, x)
  coordinates and the head dimension is shared out between the three axes;
  RoPE is a per-token complex multiply applied to Q and K.

Readings taken where the pages are silent (each one is a parameter here):
RoPE base theta = 10000; each axis gets its own standard 1D frequency ladder
theta**(-2j/D_a) over its own D_a = 2 * (its pair count); pairs are
interleaved (2j, 2j+1) = (re, im); positions start at 0; RMSNorm is over the
whole H*d token row with a length-C gain unless ``per_head``; LayerNorm uses
the population variance and no affine; softmax scale defaults to 1/sqrt(d);
keys at or past ``k_len`` are excluded and k_len = 0 gives o = 0,
lse = -inf.

Parity status: every function below is pinned by the CPU tests
(closed forms, invariants, library special cases, brute force). Fidelity to
released Wan weights (theta, ladder, norm axis, eps) cannot be pinned without
weights: those readings are "parity unpinned" against Wan itself.
"""

from __future__ import annotations

import numpy as np

# Largest finite bf16: (2 - 2**-7) * 2**127.
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ----------------------------------------------------------------------------
# bf16 <-> float64
# ----------------------------------------------------------------------------
def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly.

    A bf16 value is the top half of an IEEE-754 binary32 word, so shifting the
    16 bits up and reinterpreting as float32 is exact, as is float32->float64.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Round float64 to the nearest bf16, ties to even; return uint16 bits.

    bf16 keeps 8 significant bits (1 implicit + 7 stored) and binary32's
    exponent range. For |x| in [2**(e-1), 2**e) the spacing of bf16 values is
    2**(e-8) (never below the subnormal spacing 2**-133), so rounding is
    ``rint(x / q) * q`` with q that power of two; ``np.rint`` rounds halves to
    even and the division by a power of two is exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(xf / q) * q
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, r), r)
    r = np.where(finite, r, x)
    f32 = r.astype(np.float32)  # exact: at most 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x) -> np.ndarray:
    """float64 -> nearest bf16 (ties to even) -> float64."""
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def _f64(a) -> np.ndarray:
    """Inputs may be bf16 bit patterns (uint16) or real arrays."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# AdaLN modulation and gated residual
# ----------------------------------------------------------------------------
def layer_norm(r, eps: float) -> np.ndarray:
    """LayerNorm over the last axis without affine: (r - mean) / sqrt(var + eps).

    WanAttentionBlock snippet: norm1/norm2 are LayerNorms evaluated in fp32
    whose output is then modulated; the variance is the population variance
    (mean of squared deviations), the plain definition of LayerNorm.
    """
    r = _f64(r)
    mu = r.mean(axis=-1, keepdims=True)
    var = ((r - mu) ** 2).mean(axis=-1, keepdims=True)
    return (r - mu) / np.sqrt(var + eps)


def _per_row(v, ndim):
    """Modulation vectors are [B, C] (one per sample, broadcast over the
    tokens) or [B, L, C] (one per token)."""
    v = np.asarray(v, dtype=np.float64)
    return v[:, None, :] if v.ndim == 2 and ndim == 3 else v


def adaln_modulate_gate(x, y=None, gate=None, shift=None, scale=None,
                        eps: float = 1e-6):
    """Residual update then modulated LayerNorm of the result.

    WanAttentionBlock snippet: ``x = x + y * e[2]`` (gated residual after
    self-attention), ``x = x + cross_attn(...)`` (ungated residual after
    cross-attention) and ``norm(x) * (1 + e[1]) + e[0]`` (AdaLN modulation with
    scale e[1] and shift e[0]; ``(modulation + e).chunk(6)`` gives the six
    vectors). Here:

        r = x + gate * y      (y absent: r = x; gate absent: r = x + y)
        h = LayerNorm(r) * (1 + scale) + shift   (absent scale/shift = 0)

    x, y: [B, L, C]. gate/shift/scale: [B, C] or [B, L, C]. Returns (r, h).
    """
    x = _f64(x)
    r = x.copy()
    if y is not None:
        y = _f64(y)
        r = r + (y if gate is None else _per_row(gate, x.ndim) * y)
    h = layer_norm(r, eps)
    if scale is not None:
        h = h * (1.0 + _per_row(scale, x.ndim))
    if shift is not None:
        h = h + _per_row(shift, x.ndim)
    return r, h


# ----------------------------------------------------------------------------
# q/k RMSNorm and 3D RoPE
# ----------------------------------------------------------------------------
def rms_norm(x, gain, eps: float, group: int) -> np.ndarray:
    """RMSNorm: each group of ``group`` consecutive channels is divided by
    sqrt(mean(x**2) + eps), then multiplied by ``gain`` (length C, or None).

    WanAttentionBlock / self-attention description: q and k optionally pass
    an RMSNorm before RoPE. group = C (the whole token row) is the reading
    taken for the block-level ``qk_norm``; group = d is the per-head variant.
    """
    x = _f64(x)
    shp = x.shape
    g = x.reshape(shp[:-1] + (shp[-1] // group, group))
    ms = (g * g).mean(axis=-1, keepdims=True)
    y = (g / np.sqrt(ms + eps)).reshape(shp)
    if gain is not None:
        y = y * np.asarray(gain, dtype=np.float64)
    return y


def rope3d_pair_split(d: int):
    """Pairs per axis (t, h, w) for head size d.

    3D RoPE snippet: the d/2 complex frequencies are split as
    ``[c - 2*(c//3), c//3, c//3]`` with c = d/2 (22, 21, 21 for d = 128).
    """
    c = d // 2
    return (c - 2 * (c // 3), c // 3, c // 3)


def rope3d_token_positions(f: int, h: int, w: int) -> np.ndarray:
    """(t, y, x) of every token of an (f, h, w) latent-patch grid, [L, 3].

    Forward snippet: patches are flattened with ``flatten(2)`` over (F, H, W),
    so the token index runs w fastest, then h, then f; the RoPE snippet expands
    the t, h and w frequency rows over exactly that (f, h, w) order.
    """
    n = np.arange(f * h * w, dtype=np.int64)
    return np.stack([n // (h * w), (n // w) % h, n % w], axis=1)


def rope3d_angles(f: int, h: int, w: int, d: int,
                  theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of every (token, pair), [L, d/2], float64.

    Pair j belongs to axis a by the split of ``rope3d_pair_split``; with j'
    its index inside that axis and D_a = 2 * (pairs of axis a), the angle is
    pos_a * theta**(-2 j' / D_a). (Reading: one standard RoPE ladder per
    axis, positions from 0; the pages give the split and the per-axis
    broadcast, not the ladder.)
    """
    pos = rope3d_token_positions(f, h, w).astype(np.float64)
    cols = []
    for a, n_a in enumerate(rope3d_pair_split(d)):
        omega = float(theta) ** (-(2.0 * np.arange(n_a)) / (2.0 * n_a))
        cols.append(np.outer(pos[:, a], omega))
    return np.concatenate(cols, axis=1)


def rope3d_rotate(x, phi) -> np.ndarray:
    """Rotate interleaved pairs of x [..., L, H, d] by phi [L, d/2].

    3D RoPE snippet: ``x_i * freqs_i`` on the complex view of the pairs, then
    ``view_as_real(...).flatten``: pair (2j, 2j+1) = (re, im) becomes
    (re cos - im sin, re sin + im cos).
    """
    x = _f64(x)
    phi = np.asarray(phi, dtype=np.float64)
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def qk_norm_rope3d(x, gain, grid, H: int, eps: float = 1e-6,
                   theta: float = 10000.0, norm: bool = True,
                   rope: bool = True, per_head: bool = False,
                   rows=None) -> np.ndarray:
    """RMSNorm (times gain) then 3D RoPE of one projected tensor.

    x: [B, L, H*d] token-major rows; grid = (f, h, w) with f*h*w = L. With
    ``rows`` given, x holds only those token rows ([B, len(rows), H*d]) and
    rows are their token indices in the grid.
    Self-attention snippet: ``rope_apply(q)`` / ``rope_apply(k)`` after the
    optional q/k RMSNorm; V is never rotated. With norm False the gain is not
    applied (it belongs to the norm).
    """
    x = _f64(x)
    B, R, C = x.shape
    d = C // H
    y = rms_norm(x, gain, eps, d if per_head else C) if norm else x.copy()
    if rope:
        f, hh, ww = grid
        phi = rope3d_angles(f, hh, ww, d, theta)
        assert rows is not None or phi.shape[0] == R
        if rows is not None:
            phi = phi[np.asarray(rows, dtype=np.int64)]
        y = rope3d_rotate(y.reshape(B, R, H, d), phi).reshape(B, R, C)
    return y


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------
def attention(q, k, v, k_len: int, scale: float):
    """Softmax attention of one (batch, head).

    q: [M, d] query rows; k, v: [Lk, d]. Keys with index >= k_len do not
    take part (``k_lens=seq_lens`` in the self-attention snippet,
    ``context_lens`` for cross-attention); there is no causal mask (global
    window). Returns o [M, d] and the natural-log sum-exp lse [M].
    """
    q = _f64(q)
    M, d = q.shape
    n = max(0, min(int(k_len), np.shape(k)[0]))
    if n == 0:
        return np.zeros((M, d)), np.full(M, -np.inf)
    kk = _f64(k[:n])
    vv = _f64(v[:n])
    s = (q @ kk.T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = (p @ vv) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def _mha(q, k, v, H: int, k_lens, scale, rows):
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Lq, C = q.shape
    d = C // H
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, rows.size, C))
    lse = np.zeros((B, H, rows.size))
    for b in range(B):
        kl = k.shape[1] if k_lens is None else int(k_lens[b])
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            ob, lb = attention(q[b, rows, sl], k[b, :, sl], v[b, :, sl], kl,
                               scale)
            o[b, :, sl] = ob
            lse[b, h] = lb
    return o, lse


def self_attention(q, k, v, H: int, k_lens=None, scale=None, rows=None):
    """Full non-causal self-attention over every video token.

    Self-attention snippet: ``flash_attention(q=rope(q), k=rope(k), v,
    k_lens=seq_lens, window_size=(-1, -1))``. q, k, v: [B, L, H*d]
    (bf16 bits or reals); ``rows`` selects query rows (all if None).
    Returns o [B, rows, H*d] and lse [B, H, rows].
    """
    return _mha(q, k, v, H, k_lens, scale, rows)


def cross_attention(q, k, v, H: int, context_lens=None, scale=None,
                    rows=None):
    """Cross-attention of video queries to text keys/values.

    WanAttentionBlock snippet: ``cross_attn(norm3(x), context,
    context_lens)``; the text context is 512 umT5 tokens projected to the
    model width. q: [B, Lq, H*d]; k, v: [B, Lk, H*d]. No RoPE.
    """
    return _mha(q, k, v, H, context_lens, scale, rows)


def chunk_causal_visible(Lq: int, Lk: int, q_offset: int, chunk_len: int,
                         k_len: int, rows=None) -> np.ndarray:
    """Visibility of key j to query i under chunk-wise autoregression, [Lq, Lk].

    "Wan2.2 code walkthrough", the causalization passage (world-action models):
    a video is generated chunk by chunk; tokens of a chunk attend to each other
    and to every earlier (already observed or generated) chunk, never to a
    later one. Query i sits at global position q_offset + i (the newest chunk
    after a cache of earlier keys); key j at position j; chunk(x) =
    floor(x / chunk_len). Key j is visible iff j < k_len and
    chunk(j) <= chunk(q_offset + i). Returns the rows ``rows`` (default all)
    of the [Lq, Lk] matrix.
    """
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    qi = q_offset + rows[:, None]
    kj = np.arange(Lk)[None, :]
    return (kj < k_len) & (kj // chunk_len <= qi // chunk_len)


def chunk_causal_attention(q, k, v, H: int, q_offset: int, chunk_len: int,
                           k_lens=None, scale=None, rows=None):
    """Self-attention with the chunk-causal visibility above, per (b, h).

    q: [B, Lq, H*d] (the newest tokens), k, v: [B, Lk, H*d] (cache + newest).
    Returns o [B, rows, H*d] and lse [B, H, rows]; a row with no visible key
    gets o = 0, lse = -inf.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Lq, C = q.shape
    Lk = k.shape[1]
    d = C // H
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, rows.size, C))
    lse = np.full((B, H, rows.size), -np.inf)
    for b in range(B):
        kl = Lk if k_lens is None else int(k_lens[b])
        vis = chunk_causal_visible(Lq, Lk, q_offset, chunk_len, kl, rows)
        for hh in range(H):
            sl = slice(hh * d, (hh + 1) * d)
            qq = _f64(q[b, rows, sl])
            kk = _f64(k[b, :, sl])
            vv = _f64(v[b, :, sl])
            s = np.where(vis, (qq @ kk.T) * scale, -np.inf)
            m = s.max(axis=1, keepdims=True)
            ok = np.isfinite(m[:, 0])
            p = np.where(vis, np.exp(s - np.where(np.isfinite(m), m, 0.0)), 0.0)
            l = p.sum(axis=1, keepdims=True)
            o[b, ok, sl] = (p[ok] @ vv) / l[ok]
            lse[b, hh, ok] = (m[ok] + np.log(l[ok]))[:, 0]
    return o, lse



# ----------------------------------------------------------------------------
# Projections (the Linear layers around the attention calls)
# ----------------------------------------------------------------------------
def linear(x, w, bias=None) -> np.ndarray:
    """y = x W^T + b, as a torch ``nn.Linear`` computes it.

    "Wan2.2 code walkthrough", the WanModel snippet: the model's projections
    are ``nn.Linear`` layers (weight [out, in], bias [out]); the q, k, v and
    o projections of self- and cross-attention are Linear layers of width
    dim. "论文专题讲解：Wan2.1", section "大规模训练系统": their cost is the
    alpha * b * s * h^2 term next to attention's beta * b * s^2 * h.

    x: [..., K]; w: [N, K]; bias: [N] or None. Returns float64 [..., N].
    """
    y = _f64(x) @ _f64(w).T
    if bias is not None:
        y = y + _f64(bias)
    return y


# ----------------------------------------------------------------------------
# 8-bit attention (the pages' inference speed path)
# ----------------------------------------------------------------------------
# "论文专题讲解：Wan2.1", inference-optimisation table, row "8-bit
# FlashAttention": the scores S = Q K^T are formed from INT8 operands, the
# output O = P V from FP8 operands, and the accumulation across key blocks is
# kept in FP32. That row fixes the formats and nothing else; the readings
# taken (each one on format grounds):
#  * q and k: symmetric INT8 (codes -127..127, one scale per block) over
#    blocks of 64 tokens of one (batch, head); scale = amax / 127 stored as
#    fp32; code = round-half-even of x * (127 / amax), that product formed in
#    fp32 (a quantised code is an integer decided by floating point, so the
#    decision is pinned to one precision).
#  * v: FP8 E4M3 with the OCP microscaling recipe: one power-of-two (E8M0)
#    scale per 32 keys of one channel, 2^(floor(log2 amax) - 8) (8 = the
#    exponent of E4M3's largest binade), elements clamped to +-448 and
#    rounded to nearest even.
#  * Keys at or past k_len are padding: they take no part in attention, so
#    they are also left out of k's and v's block scales and get code 0.
#  * The score of a (query, key) pair is the exact integer dot product of the
#    codes times both block scales and the softmax scale.
#  * P, the FP8 operand of P V, is E4M3 of 2^(t - m): t = the score in log2
#    units, m = ceil(max_j t) - 7 an integer. A power-of-two offset leaves the
#    E4M3 rounding of every normal value that of the weight itself, and this
#    one puts the row maximum in (2^6, 2^7], inside E4M3's normal range
#    [2^-6, 448] with room above it.
#  * The softmax denominator is not an operand of the FP8 product: it sums
#    the unrounded weights 2^(t - m), accumulated in high precision beside
#    the product (float64 here).
# Every step after the quantisation is carried out in float64.
INT8_BLOCK = 64
MX_BLOCK = 32
E4M3_MAX = 448.0
P_OFFSET = 7    # m = ceil(max t) - P_OFFSET


def e4m3_bits_to_f64(bits) -> np.ndarray:
    """Decode OCP FP8 E4M3FN codes (bias 7, no infinities, S.1111.111 = NaN)."""
    b = np.asarray(bits).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -9), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & ((b & 7) == 7), np.nan, mag)
    return s * mag


def f64_to_e4m3_bits(x) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to even mantissa; magnitudes
    past 464 (halfway from 448 to the NaN code; 464 itself ties to 448) and
    NaN give the NaN code (no saturation, as the format conversion does)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.clip(ex - 1, -6, 8)                  # exponent of the binade (subnormals use -6)
    q = np.ldexp(1.0, e - 3)                    # spacing of representable values there
    n = np.rint(a / q)                          # ties to even
    val = n * q
    e2 = np.clip(np.frexp(np.where(val > 0, val, 1.0))[1] - 1, -6, 8)
    normal = val >= 2.0 ** -6
    mant = np.where(normal, np.rint(val / np.ldexp(1.0, e2 - 3)) - 8, np.rint(val / 2.0 ** -9))
    code = np.where(normal, ((e2 + 7) << 3) + mant.astype(np.int64), mant.astype(np.int64))
    code = np.where((a > 464.0) | np.isnan(x), 0x7F, code)
    return (sign | code).astype(np.uint8)


def _valid_rows(B: int, L: int, lens):
    """[B, L] bool: token l of sample b is valid (l < lens[b]; all if lens is None)."""
    if lens is None:
        return np.ones((B, L), dtype=bool)
    n = np.clip(np.asarray(lens, dtype=np.int64).reshape(B), 0, L)
    return np.arange(L)[None, :] < n[:, None]


def quantize_int8_blocks(x, H: int, block: int = INT8_BLOCK, lens=None):
    """Symmetric INT8 per (batch, head, block of ``block`` tokens).

    x: [B, L, H*d]; lens: per-sample valid token count or None (all valid).
    Returns codes int8 [B, H, L, d] and scales float32 [B, H, ceil(L / block)]:
    amax = max |x| over the valid rows of the block, code =
    round_half_even(fp32(x * fp32(127 / amax))) clamped to +-127, scale =
    fp32(amax / 127); rows past the valid count and blocks with amax = 0 get
    code 0 (and scale 0 when the whole block is zero).
    """
    x = _f64(x)
    B, L, C = x.shape
    d = C // H
    nb = -(-L // block)
    valid = _valid_rows(B, L, lens)
    x = np.where(valid[:, :, None], x, 0.0)
    xh = x.reshape(B, L, H, d).transpose(0, 2, 1, 3).astype(np.float32)   # exact (bf16 -> f32)
    codes = np.zeros((B, H, L, d), dtype=np.int8)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    for j in range(nb):
        blk = xh[:, :, j * block:(j + 1) * block]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(1))
        inv = (np.float32(127) / safe).astype(np.float32)
        c = np.rint((blk * inv[:, :, None, None]).astype(np.float32))
        c = np.where(amax[:, :, None, None] > 0, np.clip(c, -127, 127), 0)
        codes[:, :, j * block:(j + 1) * block] = c.astype(np.int8)
        scales[:, :, j] = np.where(amax > 0, (amax / np.float32(127)).astype(np.float32), 0)
    return codes, scales


def quantize_v_mxfp8(v, H: int, block: int = MX_BLOCK, lens=None):
    """FP8 E4M3 per (batch, head, channel, block of ``block`` keys) with a
    power-of-two scale (OCP microscaling): X = 2^(floor(log2 amax) - 8), the
    largest E4M3 binade being 2^8; element = E4M3(clamp(v / X, +-448)).

    v: [B, L, H*d]; lens as in quantize_int8_blocks (rows past it are zero).
    Returns codes uint8 [B, H, L, d], the scale exponents int
    [B, H, ceil(L / block), d] (X = 2^exp; amax = 0 gives exp -127 and zero
    codes) and the dequantised values float64 [B, H, L, d].
    """
    v = _f64(v)
    B, L, C = v.shape
    d = C // H
    nb = -(-L // block)
    v = np.where(_valid_rows(B, L, lens)[:, :, None], v, 0.0)
    vh = v.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    codes = np.zeros((B, H, L, d), dtype=np.uint8)
    exps = np.full((B, H, nb, d), -127, dtype=np.int64)
    deq = np.zeros((B, H, L, d))
    for j in range(nb):
        blk = vh[:, :, j * block:(j + 1) * block]
        amax = np.abs(blk).max(axis=2)                               # [B, H, d]
        _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
        ex = np.where(amax > 0, np.maximum((fe - 1) - 8, -127), -127)
        scaled = np.clip(blk / np.ldexp(1.0, ex)[:, :, None, :], -E4M3_MAX, E4M3_MAX)
        c = f64_to_e4m3_bits(scaled)
        codes[:, :, j * block:(j + 1) * block] = c
        exps[:, :, j] = ex
        deq[:, :, j * block:(j + 1) * block] = (e4m3_bits_to_f64(c)
                                                * np.ldexp(1.0, ex)[:, :, None, :])
    return codes, exps, deq


def attention_8bit(q, k, v, H: int, k_lens=None, scale=None, rows=None, on_head=None):
    """8-bit self-attention as read from the "8-bit FlashAttention" row (see
    the section comment): INT8 scores, FP8 probabilities and values, the rest
    in float64.

    q, k, v: [B, L, H*d]. Per (b, h) and query row i, with n = k_len[b]:
      S_ij = sum_e qc_ie kc_je                   (exact integer dot product)
      s_ij = S_ij * sq_i * sk_j * scale          (scale defaults to 1/sqrt(d))
      t_ij = s_ij * log2(e),  m_i = ceil(max_{j<n} t_ij) - 7
      p_ij = 2^(t_ij - m_i),  P_ij = E4M3(p_ij)  (round to nearest even)
      l_i  = sum_{j<n} p_ij
      o_i  = sum_{j<n} P_ij vdeq_j / l_i
      lse_i = ln 2 * (m_i + log2 l_i)            (= log sum_j exp(s_ij))
    Returns o [B, rows, H*d] and lse [B, H, rows]; n = 0 gives o = 0 and
    lse = -inf. ``on_head(b, h, terms)``, if given, receives each (batch,
    head)'s float64 terms over the selected rows and the n visible keys, a
    dict with t, m, p, P, l, the dequantised values v and ``unit`` (t of one
    unit of S, i.e. sq_i sk_j scale log2 e), for tests that bound what a
    finite-precision evaluation of these steps may change.
    """
    qc, sq = quantize_int8_blocks(q, H)
    kc, sk = quantize_int8_blocks(k, H, lens=k_lens)
    _, _, vdeq = quantize_v_mxfp8(v, H, lens=k_lens)
    B, _, Lq, d = qc.shape
    Lk = kc.shape[2]
    sc = float(scale) if scale is not None and scale > 0 else 1.0 / np.sqrt(d)
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, rows.size, H * d))
    lse = np.full((B, H, rows.size), -np.inf)
    qblk = rows // INT8_BLOCK
    kblk = np.arange(Lk) // INT8_BLOCK
    for b in range(B):
        n = Lk if k_lens is None else max(0, min(int(k_lens[b]), Lk))
        if n == 0:
            continue
        for h in range(H):
            S = qc[b, h, rows].astype(np.float64) @ kc[b, h, :n].astype(np.float64).T
            unit = sq[b, h, qblk].astype(np.float64)[:, None] \
                * sk[b, h, kblk[:n]].astype(np.float64)[None, :] * sc
            s = S * unit
            t = s / np.log(2.0)
            m = np.ceil(t.max(axis=1)) - P_OFFSET
            p = np.exp2(t - m[:, None])
            P = e4m3_bits_to_f64(f64_to_e4m3_bits(p))
            l = p.sum(axis=1)
            o[b, :, h * d:(h + 1) * d] = (P @ vdeq[b, h, :n]) / l[:, None]
            lse[b, h] = np.log(2.0) * (m + np.log2(l))
            if on_head is not None:
                on_head(b, h, {"t": t, "m": m, "p": p, "P": P, "l": l, "v": vdeq[b, h, :n],
                               "unit": unit / np.log(2.0)})
    return o, lse
