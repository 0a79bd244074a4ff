"""8-bit self-attention through the C ABI against the float64 oracle of the
"8-bit FlashAttention" reading: the quantiser's codes and scales bit for bit
(q, k and v codes are integers decided in fp32 on both sides), the attention
output within max(1e-2, one bf16 quantum) plus the derived bound on the FP8
weight codes an fp32 evaluation may pick (tests/_parity.py compare_8bit), on
ragged shapes, key lengths (with inf/NaN padding), peaked logits, zero
blocks, the Wan 480p grid and the benchmark's 720P launch (sampled rows)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from attention_wan_qk_amd import ops, synth
from attention_wan_qk_amd.workloads import BY_NAME
from tests._parity import P8Bound, compare_8bit

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rand(shape, seed, std=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _heads(bits, H, hs):
    """Channels of heads ``hs`` of a [B, L, H*d] array, as [B, L, len(hs)*d]."""
    B, L, C = bits.shape
    return np.ascontiguousarray(bits.reshape(B, L, H, C // H)[:, :, hs].reshape(B, L, -1))


def _check_quantised(qz, q, k, v, H, hs=None, k_lens=None):
    """Codes and scales of heads ``hs`` (all if None) bit for bit against the
    oracle's quantisers on those heads' channels (every block is per (batch,
    head), so a head's codes do not depend on the other heads)."""
    B, L = qz["B"], qz["L"]
    nT = (L + 63) // 64
    hs = list(range(H)) if hs is None else list(hs)
    sel = torch.tensor(hs, device=qz["q8"].device)
    for name, x, lens in (("q8", q, None), ("k8", k, k_lens)):
        codes, sc = O.quantize_int8_blocks(_heads(synth.bf16_bits(x), H, hs), len(hs), lens=lens)
        got = qz[name].index_select(1, sel).cpu().numpy().reshape(B, len(hs), nT * 64, -1)
        assert np.array_equal(got[:, :, :L], codes), name
        assert not got[:, :, L:].any(), name + " padding"
        gs = qz["q_scale" if name == "q8" else "k_scale"].index_select(1, sel).cpu().numpy()
        assert np.array_equal(gs, sc), name + " scales"
    codes, ex, vdeq = O.quantize_v_mxfp8(_heads(synth.bf16_bits(v), H, hs), len(hs), lens=k_lens)
    got = qz["v8"].index_select(1, sel).cpu().numpy()
    got = got.transpose(0, 1, 2, 4, 3).reshape(B, len(hs), nT * 64, -1)
    assert np.array_equal(got[:, :, :L], codes), "v8"
    sv = qz["v_scale"].index_select(1, sel).cpu().numpy()    # [B, h, nT, 2, 32, D/32]
    D = sv.shape[-1] * 32
    byt = sv.transpose(0, 1, 2, 3, 5, 4).reshape(B, len(hs), nT * 2, D)
    nb = ex.shape[2]
    assert np.array_equal(byt[:, :, :nb].astype(np.int64), ex + 127), "v scales"


def _run(name, q, k, v, H, k_lens=None, scale=0.0, rows=None, hs=None):
    """Quantise and attend on the GPU over all heads; check heads ``hs`` (all
    if None) and query rows ``rows`` (all if None) against the oracle."""
    print(f"[case] attn8 {name}: {tuple(q.shape)} H={H} k_lens={k_lens} heads={hs}", flush=True)
    kl = None if k_lens is None else torch.tensor(k_lens, dtype=torch.int32, device=DEV)
    qz = ops.quantize_qkv_8bit(q.to(DEV), k.to(DEV), v.to(DEV), H, k_lens=kl)
    o, lse = ops.self_attn_fwd_8bit(qz, k_lens=kl, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    _check_quantised(qz, q, k, v, H, hs, k_lens)
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    hsel = list(range(H)) if hs is None else list(hs)
    nrows = q.shape[1] if rows is None else len(rows)
    bound = P8Bound(q.shape[0], nrows, len(hsel), 128)
    ref, rl = O.attention_8bit(*(_heads(synth.bf16_bits(x), H, hsel) for x in (q, k, v)),
                               len(hsel), k_lens=k_lens, scale=scale or None, rows=rows,
                               on_head=bound)
    got = o[:, sel].view(o.shape[0], -1, H, o.shape[2] // H)[:, :, hsel].flatten(2)
    compare_8bit(f"attn8 {name}", synth.bf16_bits(got), ref, bound.bound)
    gl = lse[:, hsel][:, :, sel].cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.max(np.abs(gl[fin] - rl[fin]), initial=0.0) < 1e-3
    return o


@pytest.mark.parametrize("B,L,H", [(1, 1, 1), (1, 64, 1), (2, 150, 2), (1, 257, 3), (2, 383, 2),
                                   (1, 600, 1)])
def test_attn8_shapes(B, L, H):
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (81, 82, 83))
    _run(f"{B}x{L}x{H}", q, k, v, H)


def test_attn8_key_lengths_and_peaked():
    B, L, H = 3, 300, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s, std) for s, std in ((84, 1.0), (85, 1.0), (86, 3.0)))
    o = _run("k_lens", q, k, v, H, k_lens=[0, 1, 200])
    assert torch.all(o[0] == 0)
    _run("peaked", q, k, v, H, scale=4.0 / 128 ** 0.5)


def test_attn8_keys_past_length_hold_inf_and_nan():
    """Key and value rows at or past k_len hold inf, NaN and huge values
    (inside the 64-key block that holds k_len and in whole blocks past it):
    the quantiser must leave them out of the block scales and the output must
    equal the oracle's, which never reads them."""
    B, L, H = 2, 300, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (94, 95, 96))
    k[0, 100:] = float("inf")
    v[0, 100:] = float("nan")
    k[1, 37:] = 3e38
    v[1, 37:] = float("-inf")
    o = _run("inf/NaN past k_len", q, k, v, H, k_lens=[100, 37])
    assert torch.isfinite(o).all()


def test_attn8_zero_blocks():
    """All-zero q, k and v blocks (scale 0) next to ordinary ones."""
    B, L, H = 1, 200, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (87, 88, 89))
    q[:, :64] = 0
    k[:, 64:128, :128] = 0
    v[:, 128:160] = 0
    _run("zero blocks", q, k, v, H)


@pytest.mark.timeout(600)
def test_attn8_wan_480p_and_bf16_agreement():
    w = BY_NAME["wan1.3b-480p"]
    q, k, v = (synth.tensor(w, t, "cpu") for t in ("q", "k", "v"))
    rows = synth.sample_rows(w)
    o8 = _run("480p", q, k, v, w.heads, rows=rows)
    o16 = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), w.heads)
    torch.cuda.synchronize()
    d = (o8.float() - o16.float()).pow(2).mean().sqrt().item()
    ref = o16.float().pow(2).mean().sqrt().item()
    print(f"[attn8] 480p relative RMS difference from the bf16 kernel: {d / ref:.4f}", flush=True)
    assert d < 0.06 * ref


@pytest.mark.timeout(900)
def test_attn8_a14b_720p_cfg_sampled_heads():
    """The shape the benchmark times the 8-bit call on: 2 x 75,600 tokens
    (21 x 45 x 80 grid, both CFG halves), 40 heads, one launch of each call.
    Codes and scales of heads 0, 13, 26 and 39 are checked bit for bit on
    every token; the output and lse on the sampled rows of those heads in
    both batch entries."""
    w = BY_NAME["a14b-720p-cfg"]
    q, k, v = (synth.tensor(w, t, "cpu") for t in ("q", "k", "v"))
    _run("a14b-720p-cfg", q, k, v, w.heads, rows=synth.sample_rows(w), hs=[0, 13, 26, 39])


@pytest.mark.timeout(600)
def test_attn8_longest_sequence():
    """L = 262144 (4096 key blocks), the most the 8-bit call accepts: its
    per-block key scales fill the LDS table exactly. One head; all codes and
    scales, and sampled rows including block and tile edges."""
    L, H = 1 << 18, 1
    q, k, v = (_rand((1, L, 128 * H), s) for s in (91, 92, 93))
    rows = np.array([0, 1, 63, 64, 255, 256, 131071, 131072, L - 257, L - 256, L - 65, L - 1])
    _run("L=262144", q, k, v, H, rows=rows)
