"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark. Holds no arithmetic of the method: it only draws random tensors.

Recipe (per workload, every tensor from its own seed):
  x, y                 bf16 [B, L, C]   ~ N(0, 1)   (block input, projected attention output)
  q, k, v              bf16 [B, L, C]   ~ N(0, 1)   (same law as x W with W ~ N(0, 1/C))
  text_k, text_v       bf16 [B, Lt, C]  ~ N(0, 1)
  cross_q, cross_y     bf16 [B, L, C]   ~ N(0, 1)
  gain_q, gain_k       fp32 [C]         ~ 1 + 0.1 N(0, 1)
  modulation e         fp32 [B, 6, C]   ~ N(0, 0.1)  (variance 0.1)
  projection weights   bf16 [N, C]      ~ N(0, 1/C)  (q/k/v fused [3C, C], o, cross q, cross
                                                      k/v fused [2C, C], cross o)
  projection biases    fp32 [N]         ~ N(0, 1/C)
  text context         bf16 [B, Lt, C]  ~ N(0, 1)
  image context        bf16 [B, 257, C] ~ N(0, 1)   (image tokens of the I2V decoupled
                                                      cross-attention; count is a reading)
  FFN output           bf16 [B, L, C]   ~ N(0, 1)   (stands in for ffn(h2) at the e5 gate)
Values are drawn in fp32 and rounded to bf16 (nearest even) by torch.
Independent draws per batch entry, so the two CFG halves differ.
"""

from __future__ import annotations

import numpy as np
import torch

TAGS = {
    "x": 1, "y": 2, "q": 3, "k": 4, "v": 5, "text_k": 6, "text_v": 7,
    "cross_q": 8, "cross_y": 9, "gain_q": 10, "gain_k": 11, "mod": 12,
    "gain_cq": 13, "gain_ck": 14, "w_qkv": 15, "b_qkv": 16, "w_o": 17, "b_o": 18,
    "w_cq": 19, "b_cq": 20, "w_ckv": 21, "b_ckv": 22, "w_co": 23, "b_co": 24, "context": 25,
    "img_context": 26, "w_ikv": 27, "b_ikv": 28, "gain_ik": 29, "ffn_out": 30,
    "rows": 99,
}


IMAGE_TOKENS = 257


def seed_of(workload_index: int, tag: str, salt: int = 0) -> int:
    return ((1000 + workload_index) * 1000 + TAGS[tag]) * 7919 + salt


def normal(shape, seed: int, device, std: float = 1.0, mean: float = 0.0,
           dtype=torch.bfloat16) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


def tensor(w, tag: str, device, salt: int = 0) -> torch.Tensor:
    """One named input of workload ``w`` (a ``workloads.Workload``)."""
    B, L, C, Lt = w.batch, w.tokens, w.dim, w.text_len
    s = seed_of(w.index, tag, salt)
    if tag in ("x", "y", "q", "k", "v", "cross_q", "cross_y", "ffn_out"):
        return normal((B, L, C), s, device)
    if tag in ("text_k", "text_v"):
        return normal((B, Lt, C), s, device)
    if tag in ("gain_q", "gain_k", "gain_cq", "gain_ck", "gain_ik"):
        return normal((C,), s, device, std=0.1, mean=1.0, dtype=torch.float32)
    if tag in ("w_qkv", "w_o", "w_cq", "w_ckv", "w_co", "w_ikv"):
        rows = {"w_qkv": 3 * C, "w_ckv": 2 * C, "w_ikv": 2 * C}.get(tag, C)
        return normal((rows, C), s, device, std=C ** -0.5)
    if tag in ("b_qkv", "b_o", "b_cq", "b_ckv", "b_co", "b_ikv"):
        n = {"b_qkv": 3 * C, "b_ckv": 2 * C, "b_ikv": 2 * C}.get(tag, C)
        return normal((n,), s, device, std=C ** -0.5, dtype=torch.float32)
    if tag == "context":
        return normal((B, Lt, C), s, device)
    if tag == "img_context":
        return normal((B, IMAGE_TOKENS, C), s, device)
    if tag == "mod":
        return normal((B, 6, C), s, device, std=0.1 ** 0.5, dtype=torch.float32)
    raise KeyError(tag)


def sample_rows(w, n: int = 256, salt: int = 0) -> np.ndarray:
    """Seeded token rows to check at large shapes, plus the rows where
    indexing mistakes show: first, last, first row of the last partial
    128-row tile, and the 8 corners of the (f, h, w) grid."""
    L = w.tokens
    f, h, ww = w.grid
    rng = np.random.default_rng(seed_of(w.index, "rows", salt))
    rows = set(rng.choice(L, size=min(n, L), replace=False).tolist())
    rows |= {0, L - 1, (L // 128) * 128 if L % 128 else L - 128}
    for t in (0, f - 1):
        for y in (0, h - 1):
            for x in (0, ww - 1):
                rows.add((t * h + y) * ww + x)
    return np.array(sorted(r for r in rows if 0 <= r < L), dtype=np.int64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
