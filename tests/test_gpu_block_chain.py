"""The attention sublayer of a WanAttentionBlock end to end through the C ABI,
projections included, against the same chain computed by the float64 oracle.

Chain (WanAttentionBlock snippet of the "Wan2.2 code walkthrough" page, plus
the I2V decoupled image cross-attention of "论文专题讲解：Wan2.1" and the
FFN-side modulation and gate that close the block):

  h1 = LN(x) (1 + e1) + e0                        adaln
  q|k|v = h1 [Wq; Wk; Wv]^T + b                   linear (fused [B, L, 3C] buffer)
  q, k <- RMSNorm + 3D RoPE, in place             qk_norm_rope3d
  o = self_attention(q, k, v)                     self_attn
  x' = x + e2 (o Wo^T + bo); h3 = LN(x')          linear, adaln (norm3: gamma 1, beta 0)
  cq = RMSNorm(h3 Wcq^T + bcq)                    linear, qk_norm_rope3d (no RoPE)
  ck|cv = ctx [Wck; Wcv]^T + b; ck <- RMSNorm     linear, qk_norm_rope3d (no RoPE)
  ik|iv = img [Wik; Wiv]^T + b; ik <- RMSNorm     linear, qk_norm_rope3d (no RoPE)
  oc = cross(cq, ck, cv) + cross(cq, ik, iv)      cross_attn x 2, adaln (sum, no norm)
  x'' = x' + (oc Wco^T + bco); h2 = LN(x'') (1 + e4) + e3    linear, adaln
  x''' = x'' + e5 f       (f stands in for ffn(h2))          adaln

Every library output is bf16, so the oracle rounds to bf16 at the same
points (x' feeds norm3 unrounded, as in the library) and the two chains are
compared at h1, o, x', x'', h2 and x''' (after the first call with the
chain rule of tests/_parity.py, which carries upstream rounding flips
along). Tiny workload: every token row;
1.3B-480P: the seeded sampled rows (keys and values of every token are still
computed by the oracle).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from attention_wan_qk_amd import ops, synth
from attention_wan_qk_amd.workloads import BY_NAME
from tests._parity import compare, compare_chain

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _gpu_chain(w, t):
    H, C, eps = w.heads, w.dim, w.eps
    e = t["mod"]
    _, h1 = ops.adaln_modulate_gate(t["x"], None, None, e[:, 0], e[:, 1], eps, want_x=False)
    qkv = ops.linear_fwd(h1, t["w_qkv"], t["b_qkv"])
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    ops.qk_norm_rope3d(q, k, H, w.grid, t["gain_q"], t["gain_k"], eps=eps, theta=w.rope_theta,
                       inplace=True)
    o = ops.self_attn_fwd(q, k, v, H)
    y = ops.linear_fwd(o, t["w_o"], t["b_o"])
    x2, h3 = ops.adaln_modulate_gate(t["x"], y, e[:, 2], None, None, eps)
    cq = ops.linear_fwd(h3, t["w_cq"], t["b_cq"])
    ops.qk_norm_rope3d(cq, None, H, None, t["gain_cq"], eps=eps, rope=False, inplace=True)
    ckv = ops.linear_fwd(t["context"], t["w_ckv"], t["b_ckv"])
    ops.qk_norm_rope3d(None, ckv[..., :C], H, None, None, t["gain_ck"], eps=eps, rope=False,
                       inplace=True)
    ikv = ops.linear_fwd(t["img_context"], t["w_ikv"], t["b_ikv"])
    ops.qk_norm_rope3d(None, ikv[..., :C], H, None, None, t["gain_ik"], eps=eps, rope=False,
                       inplace=True)
    oc = ops.cross_attn_fwd(cq, ckv[..., :C], ckv[..., C:], H)
    oi = ops.cross_attn_fwd(cq, ikv[..., :C], ikv[..., C:], H)
    osum, _ = ops.adaln_modulate_gate(oc, oi, None, None, None, eps, want_h=False)
    yc = ops.linear_fwd(osum, t["w_co"], t["b_co"])
    x3, h2 = ops.adaln_modulate_gate(x2, yc, None, e[:, 3], e[:, 4], eps)
    x4, _ = ops.adaln_modulate_gate(x3, t["ffn_out"], e[:, 5], None, None, eps, want_h=False)
    torch.cuda.synchronize()
    return {"h1": h1, "o": o, "x'": x2, "x''": x3, "h2": h2, "x'''": x4}


def _oracle_chain(w, t, rows):
    """The same chain in float64 with bf16 rounding at each library output.
    Only ``rows`` of the token-local tensors are computed; keys and values of
    self-attention cover every token."""
    H, C, eps, rb = w.heads, w.dim, w.eps, O.bf16_round
    b = synth.bf16_bits
    f = lambda n: t[n].cpu().numpy().astype(np.float64)
    e = f("mod")
    x_all = b(t["x"])
    h1_all = rb(O.adaln_modulate_gate(x_all, None, None, e[:, 0], e[:, 1], eps)[1])
    wqkv, bqkv = b(t["w_qkv"]), f("b_qkv")
    k = rb(O.linear(h1_all, wqkv[C:2 * C], bqkv[C:2 * C]))
    v = rb(O.linear(h1_all, wqkv[2 * C:], bqkv[2 * C:]))
    q = rb(O.linear(h1_all[:, rows], wqkv[:C], bqkv[:C]))
    kr = rb(O.qk_norm_rope3d(k, f("gain_k"), w.grid, H, eps=eps, theta=w.rope_theta))
    qr = rb(O.qk_norm_rope3d(q, f("gain_q"), w.grid, H, eps=eps, theta=w.rope_theta, rows=rows))
    o = rb(O.self_attention(qr, kr, v, H)[0])
    y = rb(O.linear(o, b(t["w_o"]), f("b_o")))
    xr = x_all[:, rows]
    x2u, h3 = O.adaln_modulate_gate(xr, y, e[:, 2], None, None, eps)
    x2, h3 = rb(x2u), rb(h3)
    cq = rb(O.linear(h3, b(t["w_cq"]), f("b_cq")))
    cq = rb(O.qk_norm_rope3d(cq, f("gain_cq"), None, H, eps=eps, rope=False))

    def kv(ctx, wn, bn, gn):
        wkv, bkv = b(t[wn]), f(bn)
        kk = rb(O.linear(b(t[ctx]), wkv[:C], bkv[:C]))
        vv = rb(O.linear(b(t[ctx]), wkv[C:], bkv[C:]))
        return rb(O.qk_norm_rope3d(kk, f(gn), None, H, eps=eps, rope=False)), vv

    ck, cv = kv("context", "w_ckv", "b_ckv", "gain_ck")
    ik, iv = kv("img_context", "w_ikv", "b_ikv", "gain_ik")
    oc = rb(O.cross_attention(cq, ck, cv, H)[0])
    oi = rb(O.cross_attention(cq, ik, iv, H)[0])
    osum = rb(O.adaln_modulate_gate(oc, oi, None, None, None, eps)[0])
    yc = rb(O.linear(osum, b(t["w_co"]), f("b_co")))
    x3u, h2 = O.adaln_modulate_gate(x2, yc, None, e[:, 3], e[:, 4], eps)
    x3 = rb(x3u)
    x4 = O.adaln_modulate_gate(x3, b(t["ffn_out"])[:, rows], e[:, 5], None, None, eps)[0]
    return {"h1": h1_all[:, rows], "o": o, "x'": x2, "x''": x3, "h2": h2, "x'''": x4}


TAGS = ("x", "mod", "w_qkv", "b_qkv", "gain_q", "gain_k", "w_o", "b_o", "w_cq", "b_cq",
        "gain_cq", "context", "w_ckv", "b_ckv", "gain_ck", "img_context", "w_ikv", "b_ikv",
        "gain_ik", "w_co", "b_co", "ffn_out")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny-5x8x8", "wan1.3b-480p"])
def test_block_chain(name):
    w = BY_NAME[name]
    print(f"[case] block chain {name}", flush=True)
    t = {n: synth.tensor(w, n, DEV) for n in TAGS}
    got = _gpu_chain(w, t)
    rows = np.arange(w.tokens) if w.tokens <= 4096 else synth.sample_rows(w)
    ref = _oracle_chain(w, t, rows)
    sel = torch.as_tensor(rows)
    # h1 is the first call: the single-call rule applies
    compare(f"{name} chain h1", synth.bf16_bits(got["h1"][:, sel]), ref["h1"])
    for key in ("o", "x'", "x''", "h2", "x'''"):
        compare_chain(f"{name} chain {key}", synth.bf16_bits(got[key][:, sel]), ref[key])
