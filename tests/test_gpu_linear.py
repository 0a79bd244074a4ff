"""Parity of wan_linear_fwd (the q/k/v/o projections) with the float64
oracle through the C ABI: ragged M, N and K over several 256 x 256 tiles and
64-deep K steps, with and without bias, strided input rows and output written
into a slice of a fused buffer, and the fused q/k/v projection of the A14B
720P CFG workload (151200 x 15360 x 5120) on sampled token rows."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from attention_wan_qk_amd import ops, synth
from attention_wan_qk_amd.workloads import BY_NAME
from tests._parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rand(shape, seed, std=1.0, dtype=torch.bfloat16):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(dtype)


@pytest.mark.parametrize("M,N,K,bias", [(1, 8, 8, False), (7, 24, 72, True), (300, 264, 200, True),
                                        (257, 512, 128, False), (513, 1536, 1536, True),
                                        (1024, 768, 4096, True), (64, 5120, 40, True),
                                        (100, 264, 136, True), (65, 392, 192, False)])
def test_linear_shapes(M, N, K, bias):
    print(f"[case] linear M={M} N={N} K={K} bias={bias}", flush=True)
    x = _rand((M, K), 71)
    w = _rand((N, K), 72, std=K ** -0.5)
    b = _rand((N,), 73, std=0.5, dtype=torch.float32) if bias else None
    y = ops.linear_fwd(x.to(DEV), w.to(DEV), None if b is None else b.to(DEV))
    torch.cuda.synchronize()
    ref = O.linear(synth.bf16_bits(x), synth.bf16_bits(w), None if b is None else b.numpy())
    compare(f"linear {M}x{N}x{K}", synth.bf16_bits(y), ref)


def test_linear_strided_rows_into_fused_buffer():
    """x rows are a column slice of a wider buffer; y is the middle third of
    a fused [B, L, 3C] buffer whose other thirds must stay untouched."""
    B, L, C, K = 2, 150, 256, 320
    print("[case] linear strided", flush=True)
    big = _rand((B, L, K + 64), 74).to(DEV)
    x = big[..., 32:32 + K]
    w = _rand((C, K), 75, std=K ** -0.5).to(DEV)
    b = _rand((C,), 76, dtype=torch.float32).to(DEV)
    fused = torch.full((B, L, 3 * C), 7.0, dtype=torch.bfloat16, device=DEV)
    ops.linear_fwd(x, w, b, out=fused[..., C:2 * C])
    torch.cuda.synchronize()
    assert torch.all(fused[..., :C] == 7.0) and torch.all(fused[..., 2 * C:] == 7.0)
    ref = O.linear(synth.bf16_bits(x), synth.bf16_bits(w), b.cpu().numpy())
    compare("linear strided", synth.bf16_bits(fused[..., C:2 * C]), ref)


@pytest.mark.timeout(600)
def test_linear_fused_qkv_a14b_720p_cfg():
    w = BY_NAME["a14b-720p-cfg"]
    print("[case] linear fused qkv a14b-720p-cfg", flush=True)
    x = synth.tensor(w, "x", DEV)
    wq = synth.tensor(w, "w_qkv", DEV)
    bq = synth.tensor(w, "b_qkv", DEV)
    y = ops.linear_fwd(x, wq, bq)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w)
    ref = O.linear(synth.bf16_bits(x[:, rows]), synth.bf16_bits(wq), bq.cpu().numpy())
    compare("fused qkv 720p", synth.bf16_bits(y[:, rows]), ref)
