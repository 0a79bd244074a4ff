"""The library's calls inside a captured HIP graph.

Every call only enqueues kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a whole sublayer step can be captured once
and replayed, which is how a serving loop removes launch overhead at small
shapes. The graph is replayed several times with eager work of the program in
between, and every replay must reproduce the eager result bit for bit."""

from __future__ import annotations

import pytest
import torch

from attention_wan_qk_amd import ops, synth
from attention_wan_qk_amd.workloads import BY_NAME

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


TAGS = ("x", "mod", "w_qkv", "b_qkv", "gain_q", "gain_k", "w_o", "b_o", "w_cq", "b_cq",
        "gain_cq", "context", "w_ckv", "b_ckv", "gain_ck", "w_co", "b_co")


def _step(w, t, out):
    """One sublayer step (projections, both attention paths, chunk-causal
    attention) writing into the preallocated tensors of ``out``."""
    H, C, eps = w.heads, w.dim, w.eps
    e = t["mod"]
    ops.adaln_modulate_gate(t["x"], None, None, e[:, 0], e[:, 1], eps, want_x=False,
                            h_out=out["h1"])
    ops.linear_fwd(out["h1"], t["w_qkv"], t["b_qkv"], out=out["qkv"])
    qkv = out["qkv"]
    q, k, v = qkv[..., :C], qkv[..., C:2 * C], qkv[..., 2 * C:]
    ops.qk_norm_rope3d(q, k, H, w.grid, t["gain_q"], t["gain_k"], eps=eps, theta=w.rope_theta,
                       inplace=True)
    ops.self_attn_fwd(q, k, v, H, out=out["o"])
    ops.linear_fwd(out["o"], t["w_o"], t["b_o"], out=out["y"])
    ops.adaln_modulate_gate(t["x"], out["y"], e[:, 2], None, None, eps, x_out=out["x2"],
                            h_out=out["h3"])
    ops.linear_fwd(out["h3"], t["w_cq"], t["b_cq"], out=out["cq"])
    ops.qk_norm_rope3d(out["cq"], None, H, None, t["gain_cq"], eps=eps, rope=False, inplace=True)
    ops.linear_fwd(t["context"], t["w_ckv"], t["b_ckv"], out=out["ckv"])
    ckv = out["ckv"]
    ops.qk_norm_rope3d(None, ckv[..., :C], H, None, None, t["gain_ck"], eps=eps, rope=False,
                       inplace=True)
    ops.cross_attn_fwd(out["cq"], ckv[..., :C], ckv[..., C:], H, out=out["oc"])
    ops.linear_fwd(out["oc"], t["w_co"], t["b_co"], out=out["yc"])
    ops.adaln_modulate_gate(out["x2"], out["yc"], None, None, None, eps, want_h=False,
                            x_out=out["x3"])
    ops.quantize_qkv_8bit(q, k, v, H, out=out["qz"])
    ops.self_attn_fwd_8bit(out["qz"], out=out["o8"])
    ops.chunk_causal_attn_fwd(q, k, v, H, 0, w.grid[1] * w.grid[2], out=out["occ"])


def test_graph_replay_matches_eager():
    w = BY_NAME["tiny-5x8x8"]
    print("[case] graph capture of the tiny sublayer step", flush=True)
    t = {n: synth.tensor(w, n, DEV) for n in TAGS}
    B, L, C, Lt = w.batch, w.tokens, w.dim, w.text_len
    emp = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=DEV)
    out = {"h1": emp(B, L, C), "qkv": emp(B, L, 3 * C), "o": emp(B, L, C), "y": emp(B, L, C),
           "x2": emp(B, L, C), "h3": emp(B, L, C), "cq": emp(B, L, C), "ckv": emp(B, Lt, 2 * C),
           "oc": emp(B, L, C), "yc": emp(B, L, C), "x3": emp(B, L, C), "o8": emp(B, L, C),
           "occ": emp(B, L, C)}
    q0 = out["qkv"][..., :C]
    out["qz"] = ops.quantize_qkv_8bit(q0, q0, q0, w.heads)      # buffers made once
    torch.cuda.synchronize()

    _step(w, t, out)                                             # eager reference
    torch.cuda.synchronize()
    tensors = {k: v for k, v in out.items() if isinstance(v, torch.Tensor)}
    tensors.update({"qz." + k: v for k, v in out["qz"].items() if isinstance(v, torch.Tensor)})
    ref = {k: v.clone() for k, v in tensors.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(w, t, out)                                         # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(w, t, out)
    for rep in range(3):
        for v in tensors.values():                               # eager work between replays
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, r in ref.items():
            assert torch.equal(tensors[k], r), f"replay {rep}: {k} differs from the eager result"
        print(f"[graph] replay {rep}: all {len(ref)} outputs equal to eager", flush=True)
