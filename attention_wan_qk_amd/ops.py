"""Torch-facing wrappers of the libwanattn C ABI.

Each function only checks tensor metadata, allocates outputs with torch and
passes raw device pointers, sizes, strides and the current HIP stream to the
library. All arithmetic happens in the library's kernels.

The C ABI sees pointers and sizes only, so every shape, stride and length a
kernel relies on is checked here first (ValueError / TypeError), before the
device check and before anything reaches the library.
"""

from __future__ import annotations

import torch

from ._lib import WAN_NORM, WAN_NORM_PER_HEAD, WAN_ROPE, check, lib

HEAD_DIM = 128


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _token_major(t: torch.Tensor, name: str, C: int):
    """bf16 tensor [B, L, C] or [B, L, H, D] whose rows may be a column slice
    of a wider buffer. Returns (B, L, ld)."""
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name}: expected a bf16 tensor, got {t.dtype}")
    if t.dim() == 4:
        B, L, H, D = t.shape
        if H * D != C or t.stride(3) != 1 or t.stride(2) != D:
            raise ValueError(f"{name}: heads must be contiguous [B, L, H, D] with H*D = {C}")
    elif t.dim() == 3:
        B, L, c = t.shape
        if c != C or t.stride(2) != 1:
            raise ValueError(f"{name}: expected [B, L, {C}] with unit channel stride")
    else:
        raise ValueError(f"{name}: expected a 3-D or 4-D tensor")
    ld = t.stride(1) if L > 1 else max(C, t.stride(1))
    if B > 1 and t.stride(0) != L * ld:
        raise ValueError(f"{name}: batch stride must be L * row stride")
    return B, L, ld


def _check_lens(lens, B: int, name: str) -> None:
    """Per-sample lengths: a contiguous int32 tensor of B elements, or None."""
    if lens is None:
        return
    if lens.dtype != torch.int32:
        raise TypeError(f"{name} must be an int32 tensor")
    if lens.numel() != B or not lens.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor of B = {B} lengths")


def _same(name: str, got, want) -> None:
    if tuple(got) != tuple(want):
        raise ValueError(f"{name}: expected (B, L) = {tuple(want)}, got {tuple(got)}")


def _on_device(*ts) -> None:
    """Every tensor (None skipped) is on the same GPU."""
    devs = {t.device for t in ts if t is not None}
    if any(d.type != "cuda" for d in devs) or len(devs) != 1:
        raise TypeError(f"tensors must all be on one CUDA device, got {sorted(map(str, devs))}")


def _channels(t: torch.Tensor) -> int:
    return t.shape[2] * (t.shape[3] if t.dim() == 4 else 1)


def qk_norm_rope3d(q, k, heads: int, grid, gain_q=None, gain_k=None, *, eps: float = 1e-6,
                   theta: float = 10000.0, norm: bool = True, rope: bool = True,
                   per_head: bool = False, q_out=None, k_out=None, inplace: bool = False):
    """RMSNorm (times gain) and 3D RoPE of q and/or k; returns (q_out, k_out)."""
    ref = q if q is not None else k
    C = _channels(ref)
    B, L, ld_in = _token_major(ref, "q" if q is not None else "k", C)
    if q is not None and k is not None:
        Bk, Lk, ldk = _token_major(k, "k", C)
        if (Bk, Lk, ldk) != (B, L, ld_in):
            raise ValueError("q and k must have the same shape and row stride")
    if inplace:
        q_out, k_out = q, k
    else:
        if (q_out is not None and q is None) or (k_out is not None and k is None):
            raise ValueError("an output is given for a missing input")
        if q is not None and q_out is None:
            q_out = torch.empty(B, L, C, dtype=torch.bfloat16, device=ref.device)
        if k is not None and k_out is None:
            k_out = torch.empty(B, L, C, dtype=torch.bfloat16, device=ref.device)
    outs = [(n, t) for n, t in (("q_out", q_out), ("k_out", k_out)) if t is not None]
    ld_out = None
    for n, t in outs:   # one row stride serves both outputs
        Bo, Lo, ldo = _token_major(t, n, C)
        _same(n, (Bo, Lo), (B, L))
        if ld_out is not None and ldo != ld_out:
            raise ValueError("q_out and k_out must share one row stride")
        ld_out = ldo
    for g in (gain_q, gain_k):
        if g is not None and (g.dtype != torch.float32 or g.numel() != C or not g.is_contiguous()):
            raise ValueError("gains must be contiguous fp32 [H*D]")
    if C % heads:
        raise ValueError(f"{C} channels do not split into {heads} heads")
    _on_device(q, k, q_out, k_out, gain_q, gain_k)
    flags = (WAN_NORM if norm else 0) | (WAN_ROPE if rope else 0) | \
        (WAN_NORM_PER_HEAD if per_head else 0)
    f, h, w = grid if grid is not None else (0, 0, 0)
    st = lib().wan_qk_norm_rope3d(_ptr(q_out), _ptr(k_out), _ptr(q), _ptr(k), _ptr(gain_q),
                                  _ptr(gain_k), B, L, heads, C // heads, f, h, w, ld_in,
                                  ld_out, eps, theta, flags, _stream(ref))
    check("wan_qk_norm_rope3d", st)
    return q_out, k_out


def self_attn_fwd(q, k, v, heads: int, k_lens=None, scale: float = 0.0, out=None,
                  return_lse: bool = False):
    """Full non-causal self-attention; returns o (and lse [B, H, L] fp32)."""
    C = _channels(q)
    B, L, ld_q = _token_major(q, "q", C)
    *bl, ld_k = _token_major(k, "k", C)
    _same("k", bl, (B, L))
    *bl, ld_v = _token_major(v, "v", C)
    _same("v", bl, (B, L))
    if out is not None:
        _same("out", _token_major(out, "out", C)[:2], (B, L))
    _check_lens(k_lens, B, "k_lens")
    _on_device(q, k, v, out, k_lens)
    if out is None:
        out = torch.empty(B, L, C, dtype=torch.bfloat16, device=q.device)
    ld_o = _token_major(out, "out", C)[2]
    lse = torch.empty(B, heads, L, dtype=torch.float32, device=q.device) if return_lse else None
    # workspace for the key split of the last round of work (torch's caching
    # allocator keeps it stream-ordered and cheap after the first call)
    with torch.cuda.device(q.device):
        ws_bytes = lib().wan_self_attn_workspace_size(B, L, heads, C // heads)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    st = lib().wan_self_attn_fwd_ws(_ptr(out), _ptr(lse), _ptr(q), _ptr(k), _ptr(v),
                                    _ptr(k_lens), B, L, heads, C // heads, ld_q, ld_k, ld_v,
                                    ld_o, scale, _ptr(ws), ws_bytes, _stream(q))
    check("wan_self_attn_fwd_ws", st)
    return (out, lse) if return_lse else out


def cross_attn_fwd(q, k, v, heads: int, context_lens=None, scale: float = 0.0, out=None):
    """Cross-attention of q [B, Lq, C] to k, v [B, Lk, C]; returns o."""
    C = _channels(q)
    B, Lq, ld_q = _token_major(q, "q", C)
    Bk, Lk, ld_k = _token_major(k, "k", C)
    _same("k", (Bk,), (B,))
    *bl, ld_v = _token_major(v, "v", C)
    _same("v", bl, (B, Lk))
    if ld_k != ld_v:
        raise ValueError("k and v must share one row stride")
    if out is not None:
        _same("out", _token_major(out, "out", C)[:2], (B, Lq))
    _check_lens(context_lens, B, "context_lens")
    _on_device(q, k, v, out, context_lens)
    if out is None:
        out = torch.empty(B, Lq, C, dtype=torch.bfloat16, device=q.device)
    ld_o = _token_major(out, "out", C)[2]
    st = lib().wan_cross_attn_fwd(_ptr(out), _ptr(q), _ptr(k), _ptr(v), _ptr(context_lens), B,
                                  Lq, Lk, heads, C // heads, ld_q, ld_k, ld_o, scale,
                                  _stream(q))
    check("wan_cross_attn_fwd", st)
    return out


def chunk_causal_attn_fwd(q, k, v, heads: int, q_offset: int, chunk_len: int, k_lens=None,
                          scale: float = 0.0, out=None, return_lse: bool = False):
    """Self-attention of q [B, Lq, C] (tokens q_offset ..) over k, v [B, Lk, C]
    where a key is visible iff its chunk is not after the query's chunk."""
    C = _channels(q)
    B, Lq, ld_q = _token_major(q, "q", C)
    Bk, Lk, ld_k = _token_major(k, "k", C)
    _same("k", (Bk,), (B,))
    *bl, ld_v = _token_major(v, "v", C)
    _same("v", bl, (B, Lk))
    if out is not None:
        _same("out", _token_major(out, "out", C)[:2], (B, Lq))
    _check_lens(k_lens, B, "k_lens")
    _on_device(q, k, v, out, k_lens)
    if out is None:
        out = torch.empty(B, Lq, C, dtype=torch.bfloat16, device=q.device)
    ld_o = _token_major(out, "out", C)[2]
    lse = torch.empty(B, heads, Lq, dtype=torch.float32, device=q.device) if return_lse else None
    st = lib().wan_chunk_causal_attn_fwd(_ptr(out), _ptr(lse), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(k_lens), B, Lq, Lk, heads, C // heads, q_offset,
                                         chunk_len, ld_q, ld_k, ld_v, ld_o, scale, _stream(q))
    check("wan_chunk_causal_attn_fwd", st)
    return (out, lse) if return_lse else out


def _mod_strides(vecs, B, L, C):
    strides = None
    for v in vecs:
        if v is None:
            continue
        if v.dtype != torch.float32 or v.stride(-1) != 1:
            raise ValueError("modulation vectors must be fp32 tensors with unit channel stride")
        if v.dim() == 2 and tuple(v.shape) == (B, C):
            s = (v.stride(0) if B > 1 else C, 0)
        elif v.dim() == 3 and tuple(v.shape) == (B, L, C):
            s = (v.stride(0) if B > 1 else L * v.stride(1), v.stride(1) if L > 1 else C)
        else:
            raise ValueError("modulation vectors must be [B, C] or [B, L, C]")
        if strides is not None and s != strides:
            raise ValueError("gate, shift and scale must share one layout")
        strides = s
    return strides or (C, 0)


def adaln_modulate_gate(x, y=None, gate=None, shift=None, scale=None, eps: float = 1e-6, *,
                        want_x: bool = True, want_h: bool = True, x_out=None, h_out=None):
    """r = x + gate*y; returns (bf16(r) or None, bf16(LN(r)*(1+scale)+shift) or None)."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() != 3:
        raise ValueError("x must be a contiguous bf16 [B, L, C] tensor")
    B, L, C = x.shape
    if y is not None and (y.shape != x.shape or y.dtype != x.dtype or not y.is_contiguous()):
        raise ValueError("y must match x")
    for n, t in (("x_out", x_out), ("h_out", h_out)):
        if t is not None and (t.shape != x.shape or t.dtype != x.dtype or not t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous bf16 tensor shaped like x")
    sb, sl = _mod_strides((gate, shift, scale), B, L, C)
    _on_device(x, y, gate, shift, scale, x_out, h_out)
    if want_x and x_out is None:
        x_out = torch.empty_like(x)
    if want_h and h_out is None:
        h_out = torch.empty_like(x)
    st = lib().wan_adaln_modulate_gate(_ptr(x_out), _ptr(h_out), _ptr(x), _ptr(y), _ptr(gate),
                                       _ptr(shift), _ptr(scale), B, L, C, sb, sl, eps,
                                       _stream(x))
    check("wan_adaln_modulate_gate", st)
    return x_out, h_out



def _row_stride(t: torch.Tensor, name: str) -> int:
    """Stride between consecutive rows of t [..., W] whose leading dims
    flatten to equally spaced rows."""
    W = t.shape[-1]
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: expected unit stride in the last dim")
    ld = t.stride(-2) if t.dim() > 1 and t.shape[-2] > 1 else W
    exp = ld
    for d in range(t.dim() - 2, -1, -1):
        if t.shape[d] > 1 and t.stride(d) != exp:
            raise ValueError(f"{name}: rows must be equally spaced")
        exp *= t.shape[d]
    return max(ld, W)


def linear_fwd(x, weight, bias=None, out=None):
    """y = x W^T + b for x [..., K] (rows may be a column slice of a wider
    buffer), weight [N, K] bf16, bias fp32 [N] or None; returns y [..., N]."""
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("x and weight must be bf16 tensors")
    K = x.shape[-1]
    N = weight.shape[0]
    if weight.dim() != 2 or weight.shape[1] != K or weight.stride(1) != 1:
        raise ValueError("weight must be [N, K] with unit column stride")
    lead = x.shape[:-1]
    M = 1
    for n in lead:
        M *= n
    ld_x = _row_stride(x, "x")
    if bias is not None and (bias.dtype != torch.float32 or bias.numel() != N or
                             not bias.is_contiguous()):
        raise ValueError("bias must be contiguous fp32 [N]")
    if out is not None and (tuple(out.shape) != (*lead, N) or out.dtype != torch.bfloat16):
        raise ValueError("out must be bf16 [..., N] matching x")
    _on_device(x, weight, bias, out)
    if out is None:
        out = torch.empty(*lead, N, dtype=torch.bfloat16, device=x.device)
    ld_y = _row_stride(out, "out")
    st = lib().wan_linear_fwd(_ptr(out), _ptr(x), _ptr(weight), _ptr(bias), M, N, K, ld_x,
                              weight.stride(0), ld_y, _stream(x))
    check("wan_linear_fwd", st)
    return out


def quantize_qkv_8bit(q, k, v, heads: int, k_lens=None, out: dict | None = None):
    """INT8 q, k (per 64-token block) and MXFP8 v (per channel and 32 keys) in
    the layouts the 8-bit attention reads, key/value rows at or past k_lens
    quantised as zeros; returns a dict of device tensors (``out``, a dict
    returned by an earlier call of the same shape, is reused)."""
    C = _channels(q)
    B, L, ld_q = _token_major(q, "q", C)
    _, Lk, ld_k = _token_major(k, "k", C)
    _, Lv, ld_v = _token_major(v, "v", C)
    if Lk != L or Lv != L:
        raise ValueError("q, k and v must have the same token count")
    D = C // heads
    nT = (L + 63) // 64
    dev = q.device
    _check_lens(k_lens, B, "k_lens")
    if C % heads:
        raise ValueError(f"{C} channels do not split into {heads} heads")
    _on_device(q, k, v, k_lens)
    if out is not None:
        if (out["B"], out["L"], out["H"], out["D"]) != (B, L, heads, D):
            raise ValueError("out was made for another shape")
        st = lib().wan_quantize_qkv_8bit(_ptr(out["q8"]), _ptr(out["k8"]), _ptr(out["v8"]),
                                         _ptr(out["q_scale"]), _ptr(out["k_scale"]),
                                         _ptr(out["v_scale"]), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(k_lens), B, L, heads, D, ld_q, ld_k, ld_v,
                                         _stream(q))
        check("wan_quantize_qkv_8bit", st)
        return out
    out = {
        "q8": torch.empty(B, heads, nT, 64, D, dtype=torch.int8, device=dev),
        "k8": torch.empty(B, heads, nT, 64, D, dtype=torch.int8, device=dev),
        "v8": torch.empty(B, heads, nT, D, 64, dtype=torch.uint8, device=dev),
        "q_scale": torch.empty(B, heads, nT, dtype=torch.float32, device=dev),
        "k_scale": torch.empty(B, heads, nT, dtype=torch.float32, device=dev),
        "v_scale": torch.empty(B, heads, nT, 2, 32, D // 32, dtype=torch.uint8, device=dev),
        "B": B, "L": L, "H": heads, "D": D,
    }
    st = lib().wan_quantize_qkv_8bit(_ptr(out["q8"]), _ptr(out["k8"]), _ptr(out["v8"]),
                                     _ptr(out["q_scale"]), _ptr(out["k_scale"]),
                                     _ptr(out["v_scale"]), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(k_lens), B, L, heads, D, ld_q, ld_k, ld_v, _stream(q))
    check("wan_quantize_qkv_8bit", st)
    return out


def self_attn_fwd_8bit(qkv8: dict, k_lens=None, scale: float = 0.0, out=None,
                       return_lse: bool = False):
    """Self-attention on the output of quantize_qkv_8bit; returns o (and lse)."""
    B, L, H, D = qkv8["B"], qkv8["L"], qkv8["H"], qkv8["D"]
    dev = qkv8["q8"].device
    if out is not None:
        _same("out", _token_major(out, "out", H * D)[:2], (B, L))
    _check_lens(k_lens, B, "k_lens")
    _on_device(qkv8["q8"], out, k_lens)
    if out is None:
        out = torch.empty(B, L, H * D, dtype=torch.bfloat16, device=dev)
    ld_o = _token_major(out, "out", H * D)[2]
    lse = torch.empty(B, H, L, dtype=torch.float32, device=dev) if return_lse else None
    st = lib().wan_self_attn_fwd_8bit(_ptr(out), _ptr(lse), _ptr(qkv8["q8"]), _ptr(qkv8["k8"]),
                                      _ptr(qkv8["v8"]), _ptr(qkv8["q_scale"]),
                                      _ptr(qkv8["k_scale"]), _ptr(qkv8["v_scale"]), _ptr(k_lens),
                                      B, L, H, D, ld_o, scale, _stream(out))
    check("wan_self_attn_fwd_8bit", st)
    return (out, lse) if return_lse else out
