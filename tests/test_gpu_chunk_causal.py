"""Parity of wan_chunk_causal_attn_fwd (self-attention under chunk-wise
autoregression with a key cache) with the float64 oracle, through the C ABI:
token-causal and chunked masks over several query and key tiles with ragged
tails, the cache form (newest chunk after earlier keys), key lengths that cut
into a chunk, and the Wan 480p latent grid split into chunks of 3 latent
frames (sampled rows)."""

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


def _rand(shape, seed, std=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _heads(bits, H, hs):
    """Channels of heads ``hs`` of a [B, L, H*d] array, as [B, L, len(hs)*d]."""
    B, L, C = bits.shape
    return np.ascontiguousarray(bits.reshape(B, L, H, C // H)[:, :, hs].reshape(B, L, -1))


def _check(name, q, k, v, H, q_offset, chunk_len, k_lens=None, rows=None, scale=0.0, hs=None):
    """One launch over all heads; heads ``hs`` (all if None) and query rows
    ``rows`` (all if None) compared with the oracle."""
    print(f"[case] chunk-causal {name}: q {tuple(q.shape)} k {tuple(k.shape)} "
          f"offset {q_offset} chunk {chunk_len} heads {hs}", flush=True)
    kl_dev = None if k_lens is None else torch.tensor(k_lens, dtype=torch.int32, device=DEV)
    o, lse = ops.chunk_causal_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, q_offset, chunk_len,
                                       k_lens=kl_dev, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else torch.as_tensor(rows)
    hsel = list(range(H)) if hs is None else list(hs)
    ref, rl = O.chunk_causal_attention(*(_heads(synth.bf16_bits(x), H, hsel) for x in (q, k, v)),
                                       len(hsel), q_offset, chunk_len, k_lens=k_lens,
                                       scale=scale or None, rows=rows)
    got = o[:, sel].view(o.shape[0], -1, H, o.shape[2] // H)[:, :, hsel].flatten(2)
    compare(name, synth.bf16_bits(got), ref)
    got_l = lse[:, hsel][:, :, sel].cpu().numpy().astype(np.float64)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(got_l), fin), f"{name}: -inf lse pattern differs"
    assert np.max(np.abs(got_l[fin] - rl[fin]), initial=0.0) < 1e-3, name
    return o


@pytest.mark.parametrize("B,L,H,chunk", [(1, 1, 1, 1), (2, 200, 2, 1), (1, 300, 1, 48),
                                         (2, 383, 2, 100), (1, 520, 1, 256), (1, 257, 2, 64)])
def test_chunked_mask_no_cache(B, L, H, chunk):
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (21, 22, 23))
    _check(f"{B}x{L}x{H} chunk {chunk}", q, k, v, H, 0, chunk)


@pytest.mark.parametrize("Lq,Lk,chunk", [(250, 700, 250), (250, 700, 100), (97, 1000, 37),
                                         (300, 300, 1 << 20)])
def test_key_cache(Lq, Lk, chunk):
    """Newest Lq tokens (positions Lk - Lq ..) against cache + themselves."""
    B, H = 2, 2
    C = 128 * H
    q = _rand((B, Lq, C), 31)
    k, v = _rand((B, Lk, C), 32), _rand((B, Lk, C), 33)
    _check(f"cache {Lq}/{Lk} chunk {chunk}", q, k, v, H, Lk - Lq, chunk)


def test_huge_chunk_is_full_attention():
    """A chunk longer than every position leaves no mask: same values as the
    full self-attention call on the same inputs."""
    B, L, H = 2, 333, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (41, 42, 43))
    o = _check("huge chunk", q, k, v, H, 0, 1 << 30)
    full = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H)
    torch.cuda.synchronize()
    compare("huge chunk vs full", synth.bf16_bits(o), O.bf16_bits_to_f64(synth.bf16_bits(full)))


def test_key_lengths_cut_chunks():
    """k_lens of 0, inside the first chunk, inside a later chunk, and full;
    rows left with no visible key give o = 0 and lse = -inf."""
    B, Lq, Lk, H, off, chunk = 4, 130, 400, 1, 270, 90
    C = 128 * H
    q = _rand((B, Lq, C), 51)
    k, v = _rand((B, Lk, C), 52), _rand((B, Lk, C), 53)
    o = _check("k_lens cut", q, k, v, H, off, chunk, k_lens=[0, 50, 301, 400])
    assert torch.all(o[0] == 0)


def test_peaked_logits():
    B, L, H = 1, 300, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (61, 62, 63))
    _check("peaked", q, k, v, H, 0, 70, scale=4.0 / 128 ** 0.5)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("form", ["whole-clip", "newest-chunk"])
def test_wan_480p_three_frame_chunks(form):
    """21 x 30 x 52 latent grid, 12 heads, chunks of 3 latent frames (4680
    tokens): the whole clip at once, or its last chunk against the cache."""
    w = BY_NAME["wan1.3b-480p"]
    chunk = 3 * 30 * 52
    q = synth.tensor(w, "q", "cpu")
    k = synth.tensor(w, "k", "cpu")
    v = synth.tensor(w, "v", "cpu")
    rows = synth.sample_rows(w)
    if form == "whole-clip":
        _check("480p 3-frame chunks", q, k, v, w.heads, 0, chunk, rows=rows)
    else:
        off = w.tokens - chunk
        q = q[:, off:].contiguous()
        rows = np.unique(np.concatenate([rows % chunk, [0, chunk - 1]]))
        _check("480p newest chunk", q, k, v, w.heads, off, chunk, rows=rows)


@pytest.mark.timeout(900)
def test_a14b_720p_cfg_three_frame_chunks():
    """The launch the benchmark times: the whole 21 x 45 x 80 clip (2 x 75,600
    tokens, 40 heads) in chunks of 3 latent frames (10,800 tokens). Sampled
    rows of heads 0, 21 and 39 in both batch entries, plus the first and last
    row of every chunk."""
    w = BY_NAME["a14b-720p-cfg"]
    chunk = 3 * 45 * 80
    q, k, v = (synth.tensor(w, t, "cpu") for t in ("q", "k", "v"))
    starts = np.arange(0, w.tokens, chunk)
    rows = np.unique(np.concatenate([synth.sample_rows(w), starts,
                                     np.minimum(starts + chunk, w.tokens) - 1]))
    _check("a14b-720p-cfg 3-frame chunks", q, k, v, w.heads, 0, chunk, rows=rows, hs=[0, 21, 39])
