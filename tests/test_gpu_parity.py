"""Parity of the four library calls with the float64 oracle on the five
Wan-shaped workloads (all rows for the tiny one, seeded sampled rows plus
edge rows for the large ones), through the C ABI."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle as O
from attention_wan_qk_amd import ops, synth
from attention_wan_qk_amd.workloads import BY_NAME, WORKLOADS
from tests._parity import compare

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
IDS = [w.name for w in WORKLOADS]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _rows(w):
    return np.arange(w.tokens) if w.tokens <= 4096 else synth.sample_rows(w)


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
def test_qk_norm_rope3d(w):
    _announce(f"qk_norm_rope3d {w.name}")
    q = synth.tensor(w, "q", DEV)
    k = synth.tensor(w, "k", DEV)
    gq = synth.tensor(w, "gain_q", DEV)
    gk = synth.tensor(w, "gain_k", DEV)
    qo, ko = ops.qk_norm_rope3d(q, k, w.heads, w.grid, gq, gk, eps=w.eps, theta=w.rope_theta)
    torch.cuda.synchronize()
    rows = _rows(w)
    for name, x, g, out in (("q", q, gq, qo), ("k", k, gk, ko)):
        ref = O.qk_norm_rope3d(synth.bf16_bits(x[:, rows]), g.cpu().numpy(), w.grid, w.heads,
                               eps=w.eps, theta=w.rope_theta, rows=rows)
        compare(f"{w.name} {name}", synth.bf16_bits(out[:, rows]), ref)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
def test_self_attn(w):
    _announce(f"self_attn {w.name}")
    q = synth.tensor(w, "q", DEV)
    k = synth.tensor(w, "k", DEV)
    v = synth.tensor(w, "v", DEV)
    o, lse = ops.self_attn_fwd(q, k, v, w.heads, return_lse=True)
    torch.cuda.synchronize()
    rows = _rows(w)
    ref_o, ref_lse = O.self_attention(synth.bf16_bits(q[:, rows]), synth.bf16_bits(k),
                                      synth.bf16_bits(v), w.heads)
    compare(f"{w.name} o", synth.bf16_bits(o[:, rows]), ref_o)
    got_lse = lse[:, :, rows].cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got_lse - ref_lse)) < 1e-3


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
def test_cross_attn(w):
    _announce(f"cross_attn {w.name}")
    q = synth.tensor(w, "cross_q", DEV)
    k = synth.tensor(w, "text_k", DEV)
    v = synth.tensor(w, "text_v", DEV)
    o = ops.cross_attn_fwd(q, k, v, w.heads)
    torch.cuda.synchronize()
    rows = _rows(w)
    ref, _ = O.cross_attention(synth.bf16_bits(q[:, rows]), synth.bf16_bits(k),
                               synth.bf16_bits(v), w.heads)
    compare(f"{w.name} cross o", synth.bf16_bits(o[:, rows]), ref)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", WORKLOADS, ids=IDS)
def test_adaln_modulate_gate(w):
    _announce(f"adaln {w.name}")
    x = synth.tensor(w, "x", DEV)
    y = synth.tensor(w, "y", DEV)
    e = synth.tensor(w, "mod", DEV)   # [B, 6, C]: shift, scale, gate, shift2, scale2, gate2
    rows = _rows(w)
    xb, yb = synth.bf16_bits(x[:, rows]), synth.bf16_bits(y[:, rows])
    eh = e.cpu().numpy().astype(np.float64)
    # norm1 + modulate (no residual)
    _, h1 = ops.adaln_modulate_gate(x, None, None, e[:, 0], e[:, 1], w.eps, want_x=False)
    # gated residual + norm3 (gamma = 1, beta = 0 -> scale = shift = 0)
    x2, h3 = ops.adaln_modulate_gate(x, y, e[:, 2], None, None, w.eps)
    # ungated residual only
    x3, _ = ops.adaln_modulate_gate(x, y, None, None, None, w.eps, want_h=False)
    torch.cuda.synchronize()
    _, r1 = O.adaln_modulate_gate(xb, None, None, eh[:, 0], eh[:, 1], w.eps)
    compare(f"{w.name} norm1-modulate", synth.bf16_bits(h1[:, rows]), r1)
    r2, r3 = O.adaln_modulate_gate(xb, yb, eh[:, 2], None, None, w.eps)
    compare(f"{w.name} gate-residual", synth.bf16_bits(x2[:, rows]), r2)
    compare(f"{w.name} norm3", synth.bf16_bits(h3[:, rows]), r3)
    r4, _ = O.adaln_modulate_gate(xb, yb, None, None, None, w.eps)
    compare(f"{w.name} residual", synth.bf16_bits(x3[:, rows]), r4)


# ----------------------------------------------------------------- edges ----
def _rand(shape, seed, std=1.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


@pytest.mark.parametrize("B,L,H", [(1, 1, 1), (1, 7, 1), (2, 63, 3), (1, 64, 2), (2, 65, 1),
                                   (1, 129, 2), (1, 200, 1), (2, 383, 2)])
def test_self_attn_ragged(B, L, H):
    _announce(f"self_attn ragged B={B} L={L} H={H}")
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (1, 2, 3))
    kl = torch.tensor([L, max(1, L // 2 + 1)][:B], dtype=torch.int32)
    o, lse = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, k_lens=kl.to(DEV),
                               return_lse=True)
    torch.cuda.synchronize()
    qb, kb, vb = (synth.bf16_bits(t) for t in (q, k, v))
    ref, rl = O.self_attention(qb, kb, vb, H, kl.numpy())
    compare(f"ragged {B}x{L}x{H}", synth.bf16_bits(o), ref)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3


@pytest.mark.parametrize("n_tiles", [1, 2, 3, 4, 5, 6, 7, 8])
def test_attn_every_key_tile_count(n_tiles):
    """Self- and cross-attention over 1 to 8 key tiles of 64 (even and odd
    counts take different last loop iterations), with a full and a ragged
    last tile, on peaked logits (scale 4/sqrt(d)): a key tile counted twice
    or skipped moves outputs by O(1) there, where diffuse logits would hide
    it. All rows and lse against the oracle."""
    H = 2
    C = 128 * H
    sc = 4.0 / math.sqrt(128)
    for L in (64 * n_tiles, 64 * n_tiles - 5):
        _announce(f"self/cross attn over {L} keys ({n_tiles} tiles)")
        q, k, v = (_rand((1, L, C), s) for s in (21, 22, 23))
        o, lse = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, scale=sc, return_lse=True)
        qc = _rand((1, 300, C), 24)
        oc = ops.cross_attn_fwd(qc.to(DEV), k.to(DEV), v.to(DEV), H, scale=sc)
        torch.cuda.synchronize()
        qb, kb, vb = (synth.bf16_bits(t) for t in (q, k, v))
        ref, rl = O.self_attention(qb, kb, vb, H, scale=sc)
        st = compare(f"self {L} keys", synth.bf16_bits(o), ref)
        assert st["rel_l2"] < 1e-2
        assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3
        refc, _ = O.cross_attention(synth.bf16_bits(qc), kb, vb, H, scale=sc)
        st = compare(f"cross {L} keys", synth.bf16_bits(oc), refc)
        assert st["rel_l2"] < 1e-2


@pytest.mark.timeout(600)
def test_self_attn_key_split_of_the_last_round():
    """The binding's workspace call splits the work items of the last round
    into key ranges when they would leave half of the device idle (here 2
    samples x 3 heads x 16 query tiles = 96 items of 64 key tiles on a
    256-unit device, so each splits 2 ways) and merges the ranges; the second
    sample's key length of 50 (one key tile) leaves one range of each of its
    items empty.
    All rows of every head and lse against the oracle, and against the
    unsplit call (wan_self_attn_fwd) to rounding."""
    from attention_wan_qk_amd import _lib
    B, L, H = 2, 4096, 3
    C = 128 * H
    _announce("self_attn key split of the last round")
    need = _lib.lib().wan_self_attn_workspace_size(B, L, H, 128)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    items = B * H * (L // 256)
    if items % cus == 0 or 2 * (items % cus) > cus:
        pytest.skip(f"no split on a device of {cus} units")
    assert need > 0
    q, k, v = (_rand((B, L, C), s) for s in (31, 32, 33))
    kl = torch.tensor([L, 50], dtype=torch.int32)
    qd, kd, vd, kld = q.to(DEV), k.to(DEV), v.to(DEV), kl.to(DEV)   # held: pointers go to C
    o, lse = ops.self_attn_fwd(qd, kd, vd, H, k_lens=kld, return_lse=True)
    o_plain = torch.empty_like(o)
    lse_plain = torch.empty_like(lse)
    st = _lib.lib().wan_self_attn_fwd(o_plain.data_ptr(), lse_plain.data_ptr(), qd.data_ptr(),
                                      kd.data_ptr(), vd.data_ptr(), kld.data_ptr(), B, L, H, 128,
                                      0, 0, 0, 0, 0.0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    qb, kb, vb = (synth.bf16_bits(t) for t in (q, k, v))
    ref, rl = O.self_attention(qb, kb, vb, H, kl.numpy())
    compare("split tail", synth.bf16_bits(o), ref)
    assert np.max(np.abs(lse.cpu().numpy() - rl)) < 1e-3
    d = (o.float() - o_plain.float()).abs().max().item()
    assert d <= 2.0 ** -7 * max(1.0, o_plain.float().abs().max().item())
    assert torch.allclose(lse, lse_plain, rtol=0, atol=1e-5)


@pytest.mark.parametrize("Lk", [1, 7, 32, 511, 512, 513])
def test_cross_attn_key_lengths(Lk):
    _announce(f"cross_attn Lk={Lk}")
    B, Lq, H = 2, 150, 2
    C = 128 * H
    q = _rand((B, Lq, C), 4)
    k = _rand((B, Lk, C), 5)
    v = _rand((B, Lk, C), 6)
    cl = torch.tensor([Lk, max(1, Lk // 2 + 1)], dtype=torch.int32)
    o = ops.cross_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, context_lens=cl.to(DEV))
    torch.cuda.synchronize()
    ref, _ = O.cross_attention(synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(v), H,
                               cl.numpy())
    compare(f"cross Lk={Lk}", synth.bf16_bits(o), ref)


def test_attn_empty_keys_and_peaked_logits():
    _announce("self_attn k_len=0 and peaked")
    B, L, H = 2, 96, 2
    C = 128 * H
    q, k, v = (_rand((B, L, C), s) for s in (7, 8, 9))
    kl = torch.tensor([0, 40], dtype=torch.int32)
    o, lse = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, k_lens=kl.to(DEV),
                               return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ref, _ = O.self_attention(*(synth.bf16_bits(t) for t in (q, k, v)), H, kl.numpy())
    compare("k_len 0/40", synth.bf16_bits(o), ref)
    # peaked: scale 4/sqrt(d) gives logits of std ~4 (position/scale bugs change o by O(1))
    sc = 4.0 / math.sqrt(128)
    o2 = ops.self_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, scale=sc)
    torch.cuda.synchronize()
    ref2, _ = O.self_attention(*(synth.bf16_bits(t) for t in (q, k, v)), H, scale=sc)
    compare("peaked", synth.bf16_bits(o2), ref2)


@pytest.mark.parametrize("kind", ["self", "cross", "chunk-causal"])
def test_keys_past_length_take_no_part(kind):
    """Key and value rows at or past a batch entry's key length hold +inf and
    NaN: they must not reach the output (o would turn NaN if a value row past
    the length entered the P V product, even with P = 0). Lengths 70 and 131
    end inside a 64-key tile and are not tile multiples; the oracle gets the
    same tensors with those rows zeroed, which by definition changes nothing."""
    _announce(f"{kind}: keys past the length hold inf / NaN")
    B, H, Lq = 2, 2, 200
    C = 128 * H
    Lk = 300 if kind == "cross" else Lq
    q = _rand((B, Lq, C), 71)
    k, v = _rand((B, Lk, C), 72), _rand((B, Lk, C), 73)
    lens = [70, 131]
    kz, vz = k.clone(), v.clone()
    for b, n in enumerate(lens):
        k[b, n:] = float("inf")
        v[b, n:] = float("nan")
        kz[b, n:] = 0
        vz[b, n:] = 0
    kl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    qb, kb, vb = (synth.bf16_bits(t) for t in (q, kz, vz))
    if kind == "self":
        o = ops.self_attn_fwd(qd, kd, vd, H, k_lens=kl)
        ref, _ = O.self_attention(qb, kb, vb, H, lens)
    elif kind == "cross":
        o = ops.cross_attn_fwd(qd, kd, vd, H, context_lens=kl)
        ref, _ = O.cross_attention(qb, kb, vb, H, lens)
    else:
        o = ops.chunk_causal_attn_fwd(qd, kd, vd, H, 0, 64, k_lens=kl)
        ref, _ = O.chunk_causal_attention(qb, kb, vb, H, 0, 64, k_lens=lens)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any(), f"{kind}: a key row past the length reached the output"
    compare(f"{kind} keys past length", synth.bf16_bits(o), ref)


@pytest.mark.parametrize("flags", ["norm+rope", "norm", "rope", "per_head_norm+rope"])
def test_norm_rope_flags_and_fused_buffer(flags):
    _announce(f"norm_rope flags={flags}")
    B, grid, H = 2, (3, 5, 7), 3
    L, C = 105, 384
    norm = "norm" in flags
    rope = "rope" in flags
    per_head = "per_head" in flags
    qkv = _rand((B, L, 3 * C), 11, std=2.0).to(DEV)       # fused projection buffer
    gq = (1 + 0.1 * torch.randn(C, generator=torch.Generator().manual_seed(3))).float()
    gk = (1 + 0.1 * torch.randn(C, generator=torch.Generator().manual_seed(4))).float()
    ref_in = synth.bf16_bits(qkv)
    q, k = qkv[..., :C], qkv[..., C:2 * C]
    ops.qk_norm_rope3d(q, k, H, grid, gq.to(DEV), gk.to(DEV), norm=norm, rope=rope,
                       per_head=per_head, inplace=True)
    torch.cuda.synchronize()
    out = synth.bf16_bits(qkv)
    for name, sl, g in (("q", slice(0, C), gq), ("k", slice(C, 2 * C), gk)):
        ref = O.qk_norm_rope3d(ref_in[..., sl], g.numpy(), grid, H, norm=norm, rope=rope,
                               per_head=per_head)
        compare(f"fused {flags} {name}", out[..., sl], ref)
    assert np.array_equal(out[..., 2 * C:], ref_in[..., 2 * C:])   # v untouched


@pytest.mark.parametrize("H", [44, 61, 64])
def test_widest_rows(H):
    """Rows of 5632, 7808 and 8192 channels (up to the 8192-channel limit of
    the row kernels; 7808 ends inside a 512-channel chunk): q/k RMSNorm over
    the whole row and per head with RoPE, and the AdaLN call with and
    without a gated residual."""
    _announce(f"widest rows: H={H} C={128 * H}")
    B, grid = 2, (3, 4, 5)
    L, C = 60, 128 * H
    q, k = _rand((B, L, C), 91, std=2.0), _rand((B, L, C), 92)
    g = torch.Generator().manual_seed(9)
    gq, gk = (1 + 0.1 * torch.randn(C, generator=g)).float(), (1 + 0.1 * torch.randn(C, generator=g)).float()
    for per_head in (False, True):
        qo, ko = ops.qk_norm_rope3d(q.to(DEV), k.to(DEV), H, grid, gq.to(DEV), gk.to(DEV),
                                    per_head=per_head)
        torch.cuda.synchronize()
        for name, x, gn, out in (("q", q, gq, qo), ("k", k, gk, ko)):
            ref = O.qk_norm_rope3d(synth.bf16_bits(x), gn.numpy(), grid, H, per_head=per_head)
            compare(f"C={C} per_head={per_head} {name}", synth.bf16_bits(out), ref)
    x, y = _rand((B, L, C), 93), _rand((B, L, C), 94)
    e = (torch.randn(B, 6, C, generator=g) * 0.3).float()
    en = e.numpy().astype(np.float64)
    xb, yb = synth.bf16_bits(x), synth.bf16_bits(y)
    ed = e.to(DEV)
    xo, ho = ops.adaln_modulate_gate(x.to(DEV), y.to(DEV), ed[:, 2], ed[:, 0], ed[:, 1])
    _, h1 = ops.adaln_modulate_gate(x.to(DEV), None, None, ed[:, 3], ed[:, 4], want_x=False)
    torch.cuda.synchronize()
    r, h = O.adaln_modulate_gate(xb, yb, en[:, 2], en[:, 0], en[:, 1], 1e-6)
    compare(f"C={C} adaln x'", synth.bf16_bits(xo), r)
    compare(f"C={C} adaln h", synth.bf16_bits(ho), h)
    _, h1r = O.adaln_modulate_gate(xb, None, None, en[:, 3], en[:, 4], 1e-6)
    compare(f"C={C} adaln h (no residual)", synth.bf16_bits(h1), h1r)


@pytest.mark.parametrize("grid", [(1024, 1, 3), (2, 1024, 1), (1, 3, 1024)])
def test_rope_grid_at_table_limit(grid):
    """Grid axes of 1024 positions, the length of the per-axis frequency
    table the RoPE call supports."""
    _announce(f"rope grid {grid}")
    B, H = 1, 2
    L, C = grid[0] * grid[1] * grid[2], 128 * H
    q = _rand((B, L, C), 95)
    qo, _ = ops.qk_norm_rope3d(q.to(DEV), None, H, grid, norm=False)
    torch.cuda.synchronize()
    ref = O.qk_norm_rope3d(synth.bf16_bits(q), None, grid, H, norm=False)
    compare(f"rope grid {grid}", synth.bf16_bits(qo), ref)


def test_adaln_per_token_modulation_and_inplace():
    _announce("adaln per-token + in place")
    B, L, C = 2, 33, 1536
    x = _rand((B, L, C), 21).to(DEV)
    y = _rand((B, L, C), 22).to(DEV)
    e = (torch.randn(B, L, 6, C, generator=torch.Generator().manual_seed(5)) * 0.3).float()
    ed = e.to(DEV)
    xb, yb = synth.bf16_bits(x), synth.bf16_bits(y)
    x_work = x.clone()
    xo, ho = ops.adaln_modulate_gate(x_work, y, ed[:, :, 2], ed[:, :, 0], ed[:, :, 1], 1e-6,
                                     x_out=x_work)
    torch.cuda.synchronize()
    en = e.numpy().astype(np.float64)
    r, h = O.adaln_modulate_gate(xb, yb, en[:, :, 2], en[:, :, 0], en[:, :, 1], 1e-6)
    compare("per-token x'", synth.bf16_bits(xo), r)
    compare("per-token h", synth.bf16_bits(ho), h)


def test_cross_attn_many_tiles_mixed_lengths():
    """More query tiles than the 256 persistent cross-attention workgroups
    (2 x 8 heads x 20 tiles = 320), so workgroups loop over several tiles;
    sample 0 has no text keys (zero output), sample 1 a ragged 300."""
    _announce("cross_attn 320 query tiles, context lens 0/300")
    B, Lq, Lk, H = 2, 20 * 256, 512, 8
    C = 128 * H
    q, k, v = _rand((B, Lq, C), 41), _rand((B, Lk, C), 42), _rand((B, Lk, C), 43)
    cl = torch.tensor([0, 300], dtype=torch.int32)
    o = ops.cross_attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), H, context_lens=cl.to(DEV))
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0)
    ref, _ = O.cross_attention(synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(v), H,
                               cl.numpy())
    compare("cross 320 tiles", synth.bf16_bits(o), ref)


def test_cross_attn_staged_items_ragged_strided():
    """Persistent cross-attention workgroups taking several items (2 x 8
    heads x 20 query tiles = 320 > 256): after its first item a workgroup
    reads Q rows staged in LDS during the previous item and stores outputs
    as whole rows through LDS. Ragged last tile (Lq = 20 x 256 - 37),
    context lengths 0 and 300, q and o rows with a stride of C + 64: the
    padding columns and the rows after the output must stay untouched."""
    _announce("cross_attn staged items, ragged Lq, strided q/o")
    B, Lq, Lk, H = 2, 20 * 256 - 37, 512, 8
    C = 128 * H
    ld = C + 64
    qb = _rand((B, Lq, ld), 44)
    k, v = _rand((B, Lk, C), 45), _rand((B, Lk, C), 46)
    cl = torch.tensor([0, 300], dtype=torch.int32)
    sentinel = torch.tensor(3.0, dtype=torch.bfloat16)
    obuf = torch.full((B * Lq + 3, ld), 3.0, dtype=torch.bfloat16, device=DEV)
    out = obuf[:B * Lq].view(B, Lq, ld)[:, :, :C]
    o = ops.cross_attn_fwd(qb.to(DEV)[:, :, :C], k.to(DEV), v.to(DEV), H, context_lens=cl.to(DEV),
                           out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    assert torch.all(o[0] == 0)
    assert torch.all(obuf[:B * Lq, C:].cpu() == sentinel)
    assert torch.all(obuf[B * Lq:].cpu() == sentinel)
    ref, _ = O.cross_attention(synth.bf16_bits(qb[:, :, :C].contiguous()), synth.bf16_bits(k),
                               synth.bf16_bits(v), H, cl.numpy())
    compare("cross staged ragged strided", synth.bf16_bits(o.contiguous()), ref)


@pytest.mark.parametrize("pattern", ["rising", "falling", "spike", "sawtooth"])
def test_self_attn_running_max_paths(pattern):
    """Logits whose tile maxima follow a set pattern across the 12 key tiles
    of a 768-token sequence. The kernel keeps the running max m lazily: a
    tile's max is only formed on a row's first tile and when a lane's sum of
    P exceeds 2^8. 'rising' (+~10 in log2 units per tile) moves m on every
    tile, 'falling' never after the first (later tiles underflow), 'spike'
    puts one key 20 above the rest in tile 6, 'sawtooth' alternates."""
    _announce(f"self_attn running-max pattern {pattern}")
    rng = np.random.default_rng({"rising": 1, "falling": 2, "spike": 3, "sawtooth": 4}[pattern])
    L, d = 768, 128
    u = rng.choice([-1.0, 1.0], size=d)               # |u|^2 = 128: q.k ~ 128 c per unit of c
    q = u[None, :] + 0.05 * rng.standard_normal((L, d))
    tile = np.arange(L) // 64
    # c per key: log2-unit logit of a key is about 16.3 c at scale 1/sqrt(d)
    if pattern == "rising":
        c = 0.6 * tile
    elif pattern == "falling":
        c = 0.6 * (11 - tile)
    elif pattern == "spike":
        c = np.zeros(L)
        c[6 * 64 + 17] = 1.25
    else:
        c = np.where(tile % 2 == 0, 0.0, 0.9)
    k = c[:, None] * u[None, :] + 0.3 * rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    qt, kt, vt = (torch.from_numpy(x[None].astype(np.float32)).to(torch.bfloat16)
                  for x in (q, k, v))
    o = ops.self_attn_fwd(qt.to(DEV), kt.to(DEV), vt.to(DEV), 1)
    torch.cuda.synchronize()
    ref, _ = O.self_attention(*(synth.bf16_bits(t) for t in (qt, kt, vt)), 1)
    compare(f"running max {pattern}", synth.bf16_bits(o), ref)


@pytest.mark.parametrize("per_token", [False, True])
def test_adaln_row_pairs_across_samples(per_token):
    """Without a residual input a wavefront owns two consecutive token rows.
    With an odd L one pair holds the last row of sample 0 and the first of
    sample 1 (different modulation vectors), and the odd total leaves a single
    row at the end; h is written in place over x."""
    _announce(f"adaln row pairs, per_token={per_token}")
    B, L, C = 3, 37, 1536
    x = _rand((B, L, C), 31).to(DEV)
    shape = (B, L, 6, C) if per_token else (B, 6, C)
    e = (torch.randn(*shape, generator=torch.Generator().manual_seed(6)) * 0.3).float()
    ed = e.to(DEV)
    pick = (lambda t, i: t[:, :, i]) if per_token else (lambda t, i: t[:, i])
    xb = synth.bf16_bits(x)
    x_work = x.clone()
    _, ho = ops.adaln_modulate_gate(x_work, None, None, pick(ed, 0), pick(ed, 1), 1e-6,
                                    want_x=False, h_out=x_work)
    torch.cuda.synchronize()
    en = e.numpy().astype(np.float64)
    _, h = O.adaln_modulate_gate(xb, None, None, pick(en, 0), pick(en, 1), 1e-6)
    compare(f"row pairs h (per_token={per_token})", synth.bf16_bits(ho), h)


def test_determinism_and_side_stream():
    _announce("determinism + side stream")
    w = WORKLOADS[0]
    q, k, v = (synth.tensor(w, t, DEV) for t in ("q", "k", "v"))
    o1 = ops.self_attn_fwd(q, k, v, w.heads)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2 = ops.self_attn_fwd(q, k, v, w.heads)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.timeout(600)
def test_determinism_at_full_size():
    """Two launches of the benchmark's self-attention (2 x 75,600 tokens x 40
    heads), of the same shape's chunk-causal call (3-frame chunks) and of the
    cross-attention are bitwise equal, lse included: no atomics, and the lazy
    rescale, the LDS-direct loads and the fence-free barriers take the same
    path on every run."""
    w = BY_NAME["a14b-720p-cfg"]
    _announce("determinism at full size (a14b-720p-cfg)")
    q, k, v = (synth.tensor(w, t, DEV) for t in ("q", "k", "v"))
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    runs = []
    for _ in range(2):
        o, lse = ops.self_attn_fwd(q, k, v, w.heads, return_lse=True)
        chunk = 3 * w.grid[1] * w.grid[2]
        oc, lc = ops.chunk_causal_attn_fwd(q, k, v, w.heads, 0, chunk, return_lse=True)
        tq, tk, tv = (synth.tensor(w, t, DEV) for t in ("cross_q", "text_k", "text_v"))
        ox = ops.cross_attn_fwd(tq, tk, tv, w.heads)
        torch.cuda.synchronize()
        runs.append([bits(t).clone() for t in (o, lse, oc, lc, ox)])
        del o, lse, oc, lc, ox, tq, tk, tv
    for a, b, name in zip(runs[0], runs[1], ("self o", "self lse", "chunk o", "chunk lse",
                                             "cross o")):
        assert torch.equal(a, b), f"{name} differs between two launches"


@pytest.mark.timeout(600)
def test_keys_spanning_more_than_2gib():
    """One head over 2^23 + 1000 keys: each of K and V spans 2.15 GB, past the
    2^31-byte mark of the kernels' 32-bit in-buffer offsets (the calls accept
    up to 4 GiB). Cross-attention over all keys, and the chunk-causal call in
    its key-cache form with a key length that ends inside the last tile;
    sampled query rows against the oracle."""
    Lk, Lq, C = (1 << 23) + 1000, 256, 128
    _announce(f"keys spanning {Lk * C * 2 / 1e9:.3f} GB (Lk={Lk}, one head)")
    q = _rand((1, Lq, C), 81)
    k, v = _rand((1, Lk, C), 82), _rand((1, Lk, C), 83)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o_x = ops.cross_attn_fwd(qd, kd, vd, 1)
    kl = Lk - 500
    o_c = ops.chunk_causal_attn_fwd(qd, kd, vd, 1, Lk - Lq, 1 << 30,
                                    k_lens=torch.tensor([kl], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    del qd, kd, vd
    rows = np.array([0, 1, 31, 32, 127, 128, 200, 255])
    qb, kb, vb = synth.bf16_bits(q), synth.bf16_bits(k), synth.bf16_bits(v)
    ref, _ = O.cross_attention(qb, kb, vb, 1, rows=rows)
    compare("cross over 2^23 keys", synth.bf16_bits(o_x[:, torch.as_tensor(rows)]), ref)
    ref, _ = O.chunk_causal_attention(qb, kb, vb, 1, Lk - Lq, 1 << 30, k_lens=[kl], rows=rows)
    compare("key cache over 2^23 keys, k_len cut", synth.bf16_bits(o_c[:, torch.as_tensor(rows)]),
            ref)
