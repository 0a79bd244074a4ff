"""Seeded random small shapes for every call (odd grids, ragged lengths,
partial masks, optional inputs), compared in full with the oracle."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from attention_wan_qk_amd import ops, synth
from tests._parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _bf16(rng, shape, std=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("seed", range(10))
def test_fuzz_qk_norm_rope3d(seed):
    rng = np.random.default_rng(7000 + seed)
    f, h, w = (int(v) for v in rng.integers(1, 10, size=3))
    B, H = int(rng.integers(1, 3)), int(rng.choice([1, 2, 3, 5]))
    L, C = f * h * w, 128 * H
    norm = bool(rng.integers(0, 2)) or seed % 3 == 0
    rope = bool(rng.integers(0, 2)) or not norm
    per_head = norm and bool(rng.integers(0, 2))
    with_k = bool(rng.integers(0, 2))
    theta = float(rng.choice([10000.0, 500.0]))
    print(f"[case] fuzz norm_rope seed={seed} grid={f,h,w} B={B} H={H} norm={norm} rope={rope} "
          f"per_head={per_head} k={with_k} theta={theta}", flush=True)
    q = _bf16(rng, (B, L, C), 2.0)
    k = _bf16(rng, (B, L, C), 0.5) if with_k else None
    gq = torch.from_numpy((1 + 0.1 * rng.standard_normal(C)).astype(np.float32))
    g_dev = gq.to(DEV) if norm else None
    qo, ko = ops.qk_norm_rope3d(q.to(DEV), k.to(DEV) if with_k else None, H, (f, h, w), g_dev,
                                g_dev if with_k else None, norm=norm, rope=rope,
                                per_head=per_head, eps=1e-6, theta=theta)
    torch.cuda.synchronize()
    g = gq.numpy() if norm else None
    ref = O.qk_norm_rope3d(synth.bf16_bits(q), g, (f, h, w), H, eps=1e-6, theta=theta, norm=norm,
                           rope=rope, per_head=per_head)
    compare(f"fuzz q {seed}", synth.bf16_bits(qo), ref)
    if with_k:
        ref_k = O.qk_norm_rope3d(synth.bf16_bits(k), g, (f, h, w), H, eps=1e-6, theta=theta,
                                 norm=norm, rope=rope, per_head=per_head)
        compare(f"fuzz k {seed}", synth.bf16_bits(ko), ref_k)


@pytest.mark.parametrize("seed", range(12))
def test_fuzz_attention(seed):
    rng = np.random.default_rng(8000 + seed)
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    Lq = int(rng.integers(1, 700))
    cross = seed % 2 == 1
    Lk = int(rng.choice([1, 7, 33, 511, 512, 513, 600])) if cross else Lq
    C = 128 * H
    lens = rng.integers(0, Lk + 1, size=B).astype(np.int32)
    lens[0] = Lk if seed % 3 else lens[0]
    scale = float(rng.choice([0.0, 0.05, 0.2]))
    print(f"[case] fuzz attn seed={seed} cross={cross} B={B} H={H} Lq={Lq} Lk={Lk} lens={lens} "
          f"scale={scale}", flush=True)
    q = _bf16(rng, (B, Lq, C))
    k = _bf16(rng, (B, Lk, C))
    v = _bf16(rng, (B, Lk, C))
    kl = torch.from_numpy(lens).to(DEV)
    if cross:
        o = ops.cross_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, context_lens=kl, scale=scale)
        lse = None
    else:
        o, lse = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, k_lens=kl, scale=scale,
                                   return_lse=True)
    torch.cuda.synchronize()
    ref, rl = O.cross_attention(synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(v), H,
                                lens, scale if scale > 0 else None)
    compare(f"fuzz attn {seed}", synth.bf16_bits(o), ref)
    if lse is not None:
        got = lse.cpu().numpy()
        fin = np.isfinite(rl)
        assert np.array_equal(np.isfinite(got), fin)
        assert np.max(np.abs(got[fin] - rl[fin]), initial=0.0) < 1e-3


@pytest.mark.parametrize("seed", range(10))
def test_fuzz_adaln(seed):
    rng = np.random.default_rng(9000 + seed)
    B, L = int(rng.integers(1, 3)), int(rng.integers(1, 40))
    C = 8 * int(rng.integers(1, 1025))
    has_y = bool(rng.integers(0, 2))
    has_gate = has_y and bool(rng.integers(0, 2))
    want_x = bool(rng.integers(0, 2))
    want_h = (not want_x) or bool(rng.integers(0, 2))
    per_token = bool(rng.integers(0, 2))
    print(f"[case] fuzz adaln seed={seed} B={B} L={L} C={C} y={has_y} gate={has_gate} x={want_x} "
          f"h={want_h} per_token={per_token}", flush=True)
    x = _bf16(rng, (B, L, C), 3.0)
    y = _bf16(rng, (B, L, C)) if has_y else None
    shape = (B, L, 3, C) if per_token else (B, 3, C)
    e = torch.from_numpy((0.3 * rng.standard_normal(shape)).astype(np.float32)).to(DEV)
    pick = (lambda i: e[:, :, i]) if per_token else (lambda i: e[:, i])
    gate = pick(0) if has_gate else None
    xo, ho = ops.adaln_modulate_gate(x.to(DEV), y.to(DEV) if has_y else None, gate, pick(1),
                                     pick(2), 1e-6, want_x=want_x, want_h=want_h)
    torch.cuda.synchronize()
    en = e.cpu().numpy().astype(np.float64)
    pk = (lambda i: en[:, :, i]) if per_token else (lambda i: en[:, i])
    r, hh = O.adaln_modulate_gate(synth.bf16_bits(x), synth.bf16_bits(y) if has_y else None,
                                  pk(0) if has_gate else None, pk(1), pk(2), 1e-6)
    if want_x:
        compare(f"fuzz adaln x' {seed}", synth.bf16_bits(xo), r)
    if want_h:
        compare(f"fuzz adaln h {seed}", synth.bf16_bits(ho), hh)
