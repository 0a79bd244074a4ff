"""Pins of the float64 oracle against facts that do not come from the oracle:
closed forms, invariants, library routines for special cases, brute force on
tiny inputs and the shapes the pages print. CPU only."""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261203)


# ---------------------------------------------------------------- bf16 ----
def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001],
                    dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0,
            (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133]
    got = O.bf16_bits_to_f64(bits)
    assert got.tolist() == want


def test_bf16_rounding_ties_to_even_and_overflow():
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8),
                  1 + 2.0 ** -8 + 2.0 ** -30, 3.5e38, 2.0 ** -134 * 3])
    got = O.bf16_round(x)
    assert got[0] == 1.0                      # tie -> even mantissa
    assert got[1] == 1 + 2.0 ** -6            # tie -> even (0000010)
    assert got[2] == -1.0
    assert got[3] == 1 + 2.0 ** -7            # just above the tie rounds up
    assert np.isinf(got[4])
    assert got[5] == 2.0 ** -132              # subnormal: 1.5 quanta -> 2 (even)


def test_bf16_rounding_matches_torch_for_fp32_values():
    # torch's float32 -> bfloat16 conversion rounds to nearest even; for values
    # that are exactly float32 the float64 route must agree bit for bit.
    x32 = (RNG.standard_normal(200000) * np.exp(RNG.uniform(-20, 20, 200000))
           ).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy()
    got = O.f64_to_bf16_bits(x32.astype(np.float64))
    assert np.array_equal(got, want.view(np.uint16))


# ----------------------------------------------------------- LayerNorm ----
def test_layer_norm_closed_form():
    # r = [1,2,3,4]: mean 2.5, population variance 1.25.
    r = np.array([[1.0, 2.0, 3.0, 4.0]])
    want = (r - 2.5) / math.sqrt(1.25 + 1e-6)
    assert np.allclose(O.layer_norm(r, 1e-6), want, atol=1e-15)


def test_layer_norm_matches_torch():
    x = RNG.standard_normal((3, 7, 96)) * 3 + 1
    want = F.layer_norm(torch.from_numpy(x), (96,), eps=1e-6).numpy()
    assert np.allclose(O.layer_norm(x, 1e-6), want, atol=1e-12)


def test_layer_norm_moments():
    x = RNG.standard_normal((5, 256)) * 0.01
    n = O.layer_norm(x, 1e-6)
    var = x.var(axis=1)
    assert np.allclose(n.mean(axis=1), 0, atol=1e-12)
    assert np.allclose((n ** 2).mean(axis=1), var / (var + 1e-6), atol=1e-12)


# ---------------------------------------------------------------- AdaLN ----
def test_adaln_closed_form_gate_scale_shift():
    # x = 0, y = [1,2,3,4], gate = 2 -> r = [2,4,6,8]: mean 5, var 5;
    # LN(r) = [-3,-1,1,3]/sqrt(5); scale = 1 doubles it; shift adds 0.5.
    x = np.zeros((1, 1, 4))
    y = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    gate = np.full((1, 4), 2.0)
    scale = np.full((1, 4), 1.0)
    shift = np.full((1, 4), 0.5)
    r, h = O.adaln_modulate_gate(x, y, gate, shift, scale, eps=0.0)
    assert np.allclose(r, [[[2, 4, 6, 8]]])
    want = np.array([-3, -1, 1, 3]) / math.sqrt(5) * 2 + 0.5
    assert np.allclose(h[0, 0], want, atol=1e-14)


def test_adaln_special_cases():
    B, L, C = 2, 5, 64
    x = RNG.standard_normal((B, L, C))
    y = RNG.standard_normal((B, L, C))
    zero = np.zeros((B, C))
    r, h = O.adaln_modulate_gate(x, y, zero, zero, zero)
    assert np.array_equal(r, x)                       # gate 0 -> x' = x
    assert np.allclose(h, O.layer_norm(x, 1e-6))      # scale=shift=0 -> LN
    r2, _ = O.adaln_modulate_gate(x, None)
    assert np.array_equal(r2, x)                      # no y -> x' = x
    r3, _ = O.adaln_modulate_gate(x, y)               # no gate -> x + y
    assert np.allclose(r3, x + y)


def test_adaln_per_sample_equals_repeated_per_token():
    B, L, C = 2, 6, 32
    x, y = RNG.standard_normal((2, B, L, C))
    g, sh, sc = RNG.standard_normal((3, B, C))
    r1, h1 = O.adaln_modulate_gate(x, y, g, sh, sc)
    rep = lambda v: np.repeat(v[:, None, :], L, axis=1)
    r2, h2 = O.adaln_modulate_gate(x, y, rep(g), rep(sh), rep(sc))
    assert np.allclose(r1, r2) and np.allclose(h1, h2)
    # batches are independent: sample 1 uses sample 1's vectors
    _, h3 = O.adaln_modulate_gate(x[1:], y[1:], g[1:], sh[1:], sc[1:])
    assert np.allclose(h1[1:], h3)


# -------------------------------------------------------------- RMSNorm ----
def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    y = O.rms_norm(x, np.array([2.0, 0.5]), 0.0, 2)
    rms = math.sqrt(12.5)
    assert np.allclose(y, [[2 * 3 / rms, 0.5 * 4 / rms]], atol=1e-15)


def test_rms_norm_matches_torch_and_invariants():
    x = RNG.standard_normal((4, 9, 256)) * 2.5
    g = 1 + 0.1 * RNG.standard_normal(256)
    want = F.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(g),
                      eps=1e-6).numpy()
    assert np.allclose(O.rms_norm(x, g, 1e-6, 256), want, atol=1e-12)
    y = O.rms_norm(x, None, 1e-6, 256)
    m = (x ** 2).mean(axis=-1)
    assert np.allclose((y ** 2).mean(axis=-1), m / (m + 1e-6), atol=1e-12)
    assert np.allclose(O.rms_norm(7.0 * x, None, 0.0, 256),
                       O.rms_norm(x, None, 0.0, 256), atol=1e-12)


def test_rms_norm_per_head_groups():
    x = RNG.standard_normal((2, 3, 4 * 32))
    y = O.rms_norm(x, None, 1e-6, 32)
    for h in range(4):
        sl = slice(32 * h, 32 * h + 32)
        want = F.rms_norm(torch.from_numpy(x[..., sl]), (32,), eps=1e-6).numpy()
        assert np.allclose(y[..., sl], want, atol=1e-12)


# ----------------------------------------------------------------- RoPE ----
def test_rope_split_d128():
    # c = 64: [64 - 2*21, 21, 21]
    assert O.rope3d_pair_split(128) == (22, 21, 21)
    assert sum(O.rope3d_pair_split(128)) == 64


def test_token_order_brute_force():
    f, h, w = 3, 4, 5
    pos = O.rope3d_token_positions(f, h, w)
    n = 0
    for t in range(f):
        for y in range(h):
            for x in range(w):
                assert tuple(pos[n]) == (t, y, x)
                n += 1
    assert n == len(pos)


def test_token_grids_printed_on_pages():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "wan_token_grids.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for frames, lf, lh, lw, ph, pw, tokens, _src in rows:
        f, h, w = int(lf), int(lh) // int(ph), int(lw) // int(pw)
        assert 1 + (int(frames) - 1) // 4 == f     # 4x causal time stride
        pos = O.rope3d_token_positions(f, h, w)
        assert len(pos) == int(tokens)
        assert tuple(pos[-1]) == (f - 1, h - 1, w - 1)


def test_rope_closed_form_angles():
    f, h, w, d, th = 4, 6, 7, 128, 10000.0
    phi = O.rope3d_angles(f, h, w, d, th)
    n = 3 * h * w + 5 * w + 6        # token (t, y, x) = (3, 5, 6)
    assert phi[n, 0] == 3.0 and phi[n, 22] == 5.0 and phi[n, 43] == 6.0
    assert math.isclose(phi[n, 21], 3 * th ** (-42 / 44), rel_tol=1e-14)
    assert math.isclose(phi[n, 42], 5 * th ** (-40 / 42), rel_tol=1e-14)
    assert math.isclose(phi[n, 63], 6 * th ** (-40 / 42), rel_tol=1e-14)
    assert math.isclose(phi[n, 1], 3 * th ** (-2 / 44), rel_tol=1e-14)
    assert math.isclose(phi[n, 44], 6 * th ** (-2 / 42), rel_tol=1e-14)
    assert np.all(phi[0] == 0)


def _rope(x, grid, d=128, theta=10000.0):
    f, h, w = grid
    return O.rope3d_rotate(x, O.rope3d_angles(f, h, w, d, theta))


def test_rope_identity_at_origin_and_pair_norms():
    grid = (2, 3, 4)
    x = RNG.standard_normal((24, 2, 128))
    y = _rope(x, grid)
    assert np.array_equal(y[0], x[0])
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(nx, ny, rtol=1e-13)


def test_rope_is_complex_multiply():
    grid = (3, 2, 5)
    x = RNG.standard_normal((30, 3, 128))
    phi = O.rope3d_angles(*grid, 128)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * phi)[:, None, :]
    y = O.rope3d_rotate(x, phi)
    assert np.allclose(y[..., 0::2], z.real, atol=1e-13)
    assert np.allclose(y[..., 1::2], z.imag, atol=1e-13)


def _roformer_1d(vec, m, theta=10000.0):
    """Textbook 1D RoPE (RoFormer): block-diagonal 2x2 rotations with
    angles m * theta**(-2(i-1)/D), i = 1..D/2, as an explicit matrix."""
    D = vec.shape[-1]
    R = np.zeros((D, D))
    for i in range(D // 2):
        a = m * theta ** (-2.0 * i / D)
        R[2 * i:2 * i + 2, 2 * i:2 * i + 2] = [[math.cos(a), -math.sin(a)],
                                               [math.sin(a), math.cos(a)]]
    return R @ vec


def test_rope_each_axis_is_textbook_1d_rope():
    f, h, w = 5, 6, 7
    x = RNG.standard_normal((f * h * w, 1, 128))
    y = _rope(x, (f, h, w))
    for (t, yy, xx) in [(4, 0, 0), (0, 5, 0), (0, 0, 6), (3, 2, 1)]:
        n = t * h * w + yy * w + xx
        assert np.allclose(y[n, 0, 0:44], _roformer_1d(x[n, 0, 0:44], t))
        assert np.allclose(y[n, 0, 44:86], _roformer_1d(x[n, 0, 44:86], yy))
        assert np.allclose(y[n, 0, 86:128], _roformer_1d(x[n, 0, 86:128], xx))


def test_rope_scores_depend_only_on_offset():
    f, h, w = 6, 7, 8
    grid = (f, h, w)
    q = RNG.standard_normal(128)
    k = RNG.standard_normal(128)
    X = np.zeros((f * h * w, 1, 128))
    X[:] = q
    Rq = _rope(X, grid)[:, 0]
    X[:] = k
    Rk = _rope(X, grid)[:, 0]
    idx = lambda t, y, x: t * h * w + y * w + x
    p, pp = (1, 2, 3), (3, 1, 0)
    base = Rq[idx(*p)] @ Rk[idx(*pp)]
    for delta in [(1, 0, 0), (0, 2, 0), (0, 0, 4), (2, 3, 1)]:
        a = tuple(u + dd for u, dd in zip(p, delta))
        b = tuple(u + dd for u, dd in zip(pp, delta))
        assert math.isclose(Rq[idx(*a)] @ Rk[idx(*b)], base, rel_tol=1e-10,
                            abs_tol=1e-10)
    # and it does change with the offset
    assert not math.isclose(Rq[idx(1, 2, 4)] @ Rk[idx(*pp)], base,
                            rel_tol=1e-6)


def test_rope_axis_separation():
    # tokens that differ only in x leave the t and h pairs unchanged
    f, h, w = 2, 3, 9
    x = RNG.standard_normal((1, 128))
    X = np.repeat(x[None], f * h * w, axis=0)
    Y = _rope(X, (f, h, w))
    a, b = 1 * h * w + 2 * w + 0, 1 * h * w + 2 * w + 8
    assert np.allclose(Y[a, 0, :86], Y[b, 0, :86])
    assert not np.allclose(Y[a, 0, 86:], Y[b, 0, 86:])


def test_norm_and_rope_commute_with_unit_gain():
    B, f, h, w, H = 1, 2, 3, 4, 3
    L, C = f * h * w, H * 128
    x = RNG.standard_normal((B, L, C))
    a = O.qk_norm_rope3d(x, None, (f, h, w), H)
    rot = _rope(x.reshape(B, L, H, 128)[0], (f, h, w)).reshape(B, L, C)
    b = O.rms_norm(rot, None, 1e-6, C)
    assert np.allclose(a, b, atol=1e-12)
    m = (x ** 2).mean(-1)
    assert np.allclose((a ** 2).mean(-1), m / (m + 1e-6), atol=1e-12)


# ------------------------------------------------------------ attention ----
def _sdpa64(q, k, v, scale):
    return F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], scale=scale).numpy()[0, 0]


def test_attention_matches_torch_sdpa_fp64():
    q, k, v = RNG.standard_normal((3, 37, 64)) * 2
    o, lse = O.attention(q, k, v, 37, 0.125)
    assert np.allclose(o, _sdpa64(q, k, v, 0.125), atol=1e-12)
    assert np.allclose(lse, logsumexp(q @ k.T * 0.125, axis=1), atol=1e-12)


def test_attention_brute_force_scalar_loops():
    M, N, d = 3, 5, 4
    q = RNG.standard_normal((M, d))
    k = RNG.standard_normal((N, d))
    v = RNG.standard_normal((N, d))
    scale = 0.7
    o, _ = O.attention(q, k, v, N, scale)
    for i in range(M):
        w = []
        for j in range(N):
            s = 0.0
            for c in range(d):
                s += q[i, c] * k[j, c]
            w.append(math.exp(s * scale))
        tot = sum(w)
        for c in range(d):
            acc = 0.0
            for j in range(N):
                acc += w[j] * v[j, c]
            assert math.isclose(o[i, c], acc / tot, rel_tol=1e-12, abs_tol=1e-12)


def test_attention_invariants():
    M, N, d = 16, 40, 32
    q = RNG.standard_normal((M, d)) * 3
    k = RNG.standard_normal((N, d))
    v = RNG.standard_normal((N, d))
    s = 1 / math.sqrt(d)
    o1, _ = O.attention(q, k, np.ones((N, d)), N, s)
    assert np.allclose(o1, 1.0, atol=1e-13)                   # rows sum to 1
    c = RNG.standard_normal(d)
    oc, _ = O.attention(q, k, np.tile(c, (N, 1)), N, s)
    assert np.allclose(oc, c, atol=1e-13)                     # constant V
    oz, _ = O.attention(np.zeros((M, d)), k, v, 25, s)
    assert np.allclose(oz, v[:25].mean(axis=0), atol=1e-13)   # q=0 -> mean
    perm = RNG.permutation(N)
    o, _ = O.attention(q, k, v, N, s)
    op, _ = O.attention(q, k[perm], v[perm], N, s)
    assert np.allclose(o, op, atol=1e-12)                     # no hidden order
    k2, v2 = k.copy(), v.copy()
    k2[30:] = 100 * RNG.standard_normal((10, d))
    v2[30:] = 1e3
    oa, la = O.attention(q, k, v, 30, s)
    ob, lb = O.attention(q, k2, v2, 30, s)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)  # mask
    o0, l0 = O.attention(q, k, v, 0, s)
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))       # empty
    kp = k.copy()
    kp[7] = q[3] * 50                                          # peaked key
    opk, _ = O.attention(q[3:4], kp, v, N, 1.0)
    assert np.allclose(opk[0], v[7], atol=1e-10)


def test_multihead_rows_batches_and_heads():
    B, L, H, d = 2, 23, 3, 16
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    kl = np.array([23, 11])
    o, lse = O.self_attention(q, k, v, H, kl, None)
    for b in range(B):
        for h in range(H):
            sl = slice(h * d, (h + 1) * d)
            want = _sdpa64(q[b, :, sl], k[b, :kl[b], sl], v[b, :kl[b], sl],
                           1 / math.sqrt(d))
            assert np.allclose(o[b, :, sl], want, atol=1e-12)
    rows = np.array([0, 5, 22])
    o2, l2 = O.self_attention(q, k, v, H, kl, None, rows=rows)
    assert np.array_equal(o2, o[:, rows]) and np.array_equal(l2, lse[:, :, rows])
    # cross-attention: separate key length, mask per batch
    kt, vt = RNG.standard_normal((2, B, 9, H * d))
    oc, _ = O.cross_attention(q, kt, vt, H, np.array([9, 4]))
    want = _sdpa64(q[1, :, :d], kt[1, :4, :d], vt[1, :4, :d], 1 / math.sqrt(d))
    assert np.allclose(oc[1, :, :d], want, atol=1e-12)


def test_oracle_bf16_bits_inputs():
    x = RNG.standard_normal((1, 4, 256)).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wid = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(O.bf16_bits_to_f64(bits), wid)
    assert np.allclose(O.rms_norm(bits, None, 1e-6, 256),
                       O.rms_norm(wid, None, 1e-6, 256))


def test_oracle_is_independent_of_the_library():
    import ast
    src_dir = os.path.join(os.path.dirname(GOLDEN), "..", "oracle")
    for name in os.listdir(src_dir):
        if name.endswith(".py"):
            tree = ast.parse(open(os.path.join(src_dir, name)).read())
            for node in ast.walk(tree):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in node.names] if isinstance(node, ast.Import) \
                        else [node.module or ""]
                    for m in mods:
                        assert not m.startswith("attention_wan_qk_amd"), name
                        assert m.split(".")[0] in ("numpy", "__future__", "") or \
                            m.startswith("wan_oracle"), (name, m)


def test_qk_norm_rope3d_row_subset_equals_full():
    B, grid, H = 2, (3, 4, 5), 2
    L, C = 60, 256
    x = RNG.standard_normal((B, L, C))
    g = 1 + 0.1 * RNG.standard_normal(C)
    full = O.qk_norm_rope3d(x, g, grid, H)
    rows = np.array([0, 7, 33, 59])
    sub = O.qk_norm_rope3d(x[:, rows], g, grid, H, rows=rows)
    assert np.array_equal(sub, full[:, rows])


# ------------------------------------------------------- chunk-causal ----
def test_chunk_causal_with_one_chunk_is_full_attention():
    B, L, H, d = 2, 37, 2, 16
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    kl = np.array([37, 20])
    full, fl = O.self_attention(q, k, v, H, kl)
    cc, cl = O.chunk_causal_attention(q, k, v, H, 0, 1000, kl)
    assert np.allclose(cc, full, atol=1e-12) and np.allclose(cl, fl, atol=1e-12)


def test_chunk_causal_with_unit_chunks_is_torch_causal():
    L, d = 29, 16
    q, k, v = RNG.standard_normal((3, 1, L, d))
    cc, _ = O.chunk_causal_attention(q, k, v, 1, 0, 1)
    want = F.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None], torch.from_numpy(k)[:, None],
        torch.from_numpy(v)[:, None], is_causal=True).numpy()[:, 0]
    assert np.allclose(cc, want, atol=1e-12)


def test_chunk_causal_visibility_brute_force_and_cache_offset():
    Lq, Lk, off, cl = 6, 14, 8, 4
    vis = O.chunk_causal_visible(Lq, Lk, off, cl, 13)
    for i in range(Lq):
        for j in range(Lk):
            assert vis[i, j] == (j < 13 and (j // cl) <= ((off + i) // cl))
    # newest tokens attending to a cache: equal to the matching rows of the
    # whole sequence computed at once
    B, H, d = 1, 2, 16
    q, k, v = RNG.standard_normal((3, B, Lk, H * d))
    whole, _ = O.chunk_causal_attention(q, k, v, H, 0, cl)
    tail, _ = O.chunk_causal_attention(q[:, off:], k, v, H, off, cl)
    assert np.allclose(tail, whole[:, off:], atol=1e-12)


def test_chunk_causal_future_chunks_have_no_effect():
    B, L, H, d, cl = 1, 40, 1, 16, 8
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    o1, _ = O.chunk_causal_attention(q, k, v, H, 0, cl)
    k2, v2 = k.copy(), v.copy()
    k2[:, 24:] = 50 * RNG.standard_normal((B, 16, d))
    v2[:, 24:] = 1e3
    o2, _ = O.chunk_causal_attention(q, k2, v2, H, 0, cl)
    assert np.array_equal(o1[:, :24], o2[:, :24])      # chunks 0..2 never see 3, 4
    assert not np.allclose(o1[:, 24:], o2[:, 24:])


def test_chunk_causal_row_subset_equals_full():
    B, Lq, Lk, H, d, off, cl = 2, 23, 50, 2, 16, 27, 10
    q = RNG.standard_normal((B, Lq, H * d))
    k, v = RNG.standard_normal((2, B, Lk, H * d))
    kl = np.array([50, 31])
    full, fl = O.chunk_causal_attention(q, k, v, H, off, cl, kl)
    rows = np.array([0, 2, 3, 12, 22])
    sub, sl = O.chunk_causal_attention(q, k, v, H, off, cl, kl, rows=rows)
    assert np.array_equal(sub, full[:, rows]) and np.array_equal(sl, fl[:, :, rows])
    assert np.array_equal(O.chunk_causal_visible(Lq, Lk, off, cl, 31, rows),
                          O.chunk_causal_visible(Lq, Lk, off, cl, 31)[rows])


# ---------------------------------------------------------------- linear ----
def test_linear_brute_force_loops():
    M, N, K = 3, 5, 7
    x = RNG.standard_normal((M, K))
    w = RNG.standard_normal((N, K))
    b = RNG.standard_normal(N)
    y = O.linear(x, w, b)
    for m in range(M):
        for n in range(N):
            acc = b[n]
            for k in range(K):
                acc += x[m, k] * w[n, k]
            assert abs(y[m, n] - acc) < 1e-12


def test_linear_special_cases_and_torch():
    x = RNG.standard_normal((2, 9, 16))
    eye = np.eye(16)
    assert np.array_equal(O.linear(x, eye), x)                     # identity weight
    b = RNG.standard_normal(4)
    assert np.array_equal(O.linear(x, np.zeros((4, 16)), b), np.broadcast_to(b, (2, 9, 4)))
    w = RNG.standard_normal((12, 16))
    want = F.linear(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b.repeat(3))).numpy()
    assert np.allclose(O.linear(x, w, b.repeat(3)), want, atol=1e-12)
    # a fused [Wq; Wk; Wv] weight gives the three projections side by side
    ws = np.split(w, 3)
    parts = np.concatenate([O.linear(x, wi) for wi in ws], axis=-1)
    assert np.allclose(O.linear(x, w), parts, atol=1e-12)
    # bf16 bit patterns are widened exactly: 1.0 = 0x3f80, 2.0 = 0x4000
    xb = np.array([[0x3F80, 0x4000]], dtype=np.uint16)
    wb = np.array([[0x4000, 0x3F80]], dtype=np.uint16)
    assert O.linear(xb, wb)[0, 0] == 4.0


# ---------------------------------------------------------------- 8-bit ----
def test_e4m3_codec_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_bits_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    assert np.array_equal(mine[~np.isnan(mine)], ref[~np.isnan(ref)])
    finite = mine[~np.isnan(mine)]
    assert finite.max() == 448.0 and np.min(finite[finite > 0]) == 2.0 ** -9
    # random magnitudes over every binade, exact ties between neighbours, out of range
    rng = np.random.default_rng(5)
    x = rng.standard_normal(100000) * np.exp2(rng.uniform(-12, 9.5, 100000))
    pos = np.sort(finite[finite > 0])
    ties = (pos[:-1] + pos[1:]) / 2
    x = np.concatenate([x, ties, -ties, [464.0, 470.0, -1e4, 0.0, 2.0 ** -11]]).astype(np.float32)
    got = O.f64_to_e4m3_bits(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def test_int8_block_quantization():
    B, L, H, d = 2, 150, 2, 16          # blocks of 64, 64, 22 tokens
    x = RNG.standard_normal((B, L, H * d)) * 3
    x[1, 64:128, :d] = 0.0              # one all-zero block
    codes, sc = O.quantize_int8_blocks(x, H)
    assert codes.shape == (B, H, L, d) and sc.shape == (B, H, 3)
    xh = x.reshape(B, L, H, d).transpose(0, 2, 1, 3)
    for b in range(B):
        for h in range(H):
            for j in range(3):
                blk = xh[b, h, j * 64:(j + 1) * 64]
                c = codes[b, h, j * 64:(j + 1) * 64].astype(np.float64)
                amax = np.abs(blk).max()
                if amax == 0:
                    assert sc[b, h, j] == 0 and not c.any()
                    continue
                assert sc[b, h, j] == np.float32(np.float32(amax) / np.float32(127))
                assert np.abs(c).max() == 127                       # the block max maps to +-127
                assert np.all(np.abs(c * sc[b, h, j] - blk) <= sc[b, h, j] * 0.5001)
    # one element by hand: code = round_half_even(fp32(x * fp32(127 / amax)))
    b, h, i, e = 0, 1, 70, 5
    amax = np.float32(np.abs(xh[b, h, 64:128]).max())
    inv = np.float32(np.float32(127) / amax)
    assert codes[b, h, i, e] == np.rint(np.float32(np.float32(xh[b, h, i, e]) * inv))


def test_mxfp8_value_quantization():
    B, L, H, d = 1, 80, 1, 8            # key blocks of 32, 32, 16
    v = RNG.standard_normal((B, L, H * d)) * np.exp2(RNG.integers(-6, 6, size=(1, 1, H * d)))
    v[0, 32:64, 3] = 0.0                 # a zero block
    codes, ex, deq = O.quantize_v_mxfp8(v, H)
    for j in range(3):
        for c in range(d):
            blk = v[0, j * 32:(j + 1) * 32, c]
            amax = np.abs(blk).max()
            if amax == 0:
                assert ex[0, 0, j, c] == -127 and not codes[0, 0, j * 32:(j + 1) * 32, c].any()
                continue
            e = math.frexp(amax)[1] - 1 - 8                      # floor(log2 amax) - 8
            assert ex[0, 0, j, c] == e
            scaled = blk / 2.0 ** e
            assert 256 <= np.abs(scaled).max() < 512
            r = deq[0, 0, j * 32:(j + 1) * 32, c]
            small = np.abs(scaled) < 2.0 ** -6
            big = np.abs(scaled) >= E4M3_CLAMP
            rel = np.abs(r - blk) / np.abs(np.where(blk == 0, 1, blk))
            assert np.all(rel[~small & ~big] <= 2.0 ** -4 + 1e-12)   # half a quantum of 2^-3
            assert np.all(np.abs(r[big]) == 448 * 2.0 ** e)          # clamped to the largest code


E4M3_CLAMP = 448.0


def test_quantizers_leave_out_keys_past_length():
    """Keys at or past k_len are padding: the k and v quantisers form their
    block scales from the valid rows only and give the padding code 0."""
    B, L, H, d = 2, 150, 1, 16
    x = RNG.standard_normal((B, L, H * d))
    x[0, 100:] *= 1000.0                 # huge padding past k_len = 100 (block 1 is mixed)
    x[1, 40:] = np.inf                   # non-finite padding past k_len = 40
    lens = [100, 40]
    codes, sc = O.quantize_int8_blocks(x, H, lens=lens)
    vc, ex, vd = O.quantize_v_mxfp8(x, H, lens=lens)
    for b, n in enumerate(lens):
        assert not codes[b, 0, n:].any() and not vc[b, 0, n:].any() and not vd[b, 0, n:].any()
        for j in range(3):
            valid = x[b, j * 64:min((j + 1) * 64, n), :]
            amax = np.abs(valid).max() if valid.size else 0.0
            assert sc[b, 0, j] == (np.float32(np.float32(amax) / np.float32(127)) if amax else 0)
        for j in range(5):
            valid = x[b, j * 32:min((j + 1) * 32, n), :]
            for c in range(d):
                amax = np.abs(valid[:, c]).max() if valid.size else 0.0
                want = math.frexp(amax)[1] - 1 - 8 if amax > 0 else -127
                assert ex[b, 0, j, c] == want
    # the valid rows' codes are those of the same rows with zero padding
    z = np.where(np.arange(L)[None, :, None] < np.array(lens)[:, None, None], x, 0.0)
    cz, sz = O.quantize_int8_blocks(z, H)
    assert np.array_equal(codes, cz) and np.array_equal(sc, sz)
    assert np.array_equal(vd, O.quantize_v_mxfp8(z, H)[2])


def _dequantised(q, k, v, H, k_lens):
    """Dequantised operands [B, H, L, d]: code * block scale."""
    qc, sq = O.quantize_int8_blocks(q, H)
    kc, sk = O.quantize_int8_blocks(k, H, lens=k_lens)
    _, _, vd = O.quantize_v_mxfp8(v, H, lens=k_lens)
    blk = np.arange(qc.shape[2]) // 64
    qd = qc.astype(np.float64) * sq[:, :, blk][..., None].astype(np.float64)
    kd = kc.astype(np.float64) * sk[:, :, blk][..., None].astype(np.float64)
    return qd, kd, vd


def test_attention_8bit_against_exact_attention_on_dequantised_operands():
    """Against exact attention (torch SDPA, float64) on the dequantised
    operands, only the rounding of the weights in the P V product differs:
    each P_ij is within half an E4M3 spacing of p_ij, i.e. 2^-4 p_ij where p
    is normal (>= 2^-6) and 2^-10 below, and the denominator is exact. With
    w = p / l the softmax weights and l >= 2^6 (the row maximum of p lies in
    (2^6, 2^7]):  |o - o_exact|_d <= 2^-4 sum_j w_j |v_jd| + 2^-16 sum_j |v_jd|.
    lse is exactly the log-sum-exp of the scores (scipy)."""
    B, L, H, d = 2, 150, 2, 32
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    k_lens = [150, 97]
    for scale in (None, 0.6):
        o, lse = O.attention_8bit(q, k, v, H, k_lens=k_lens, scale=scale)
        qd, kd, vd = _dequantised(q, k, v, H, k_lens)
        sc = scale or 1 / math.sqrt(d)
        for b, n in enumerate(k_lens):
            for h in range(H):
                Q, K, V = (torch.from_numpy(np.ascontiguousarray(a)) for a in
                           (qd[b, h], kd[b, h, :n], vd[b, h, :n]))
                ex = F.scaled_dot_product_attention(Q[None], K[None], V[None], scale=sc)[0].numpy()
                s = qd[b, h] @ kd[b, h, :n].T * sc
                w = np.exp(s - s.max(axis=1, keepdims=True))
                w /= w.sum(axis=1, keepdims=True)
                av = np.abs(vd[b, h, :n])
                bound = 2.0 ** -4 * (w @ av) + 2.0 ** -16 * av.sum(axis=0)[None, :] + 1e-12
                got = o[b, :, h * d:(h + 1) * d]
                assert np.all(np.abs(got - ex) <= bound)
                assert np.abs(got - ex).max() > 1e-6       # the weights really are rounded
                assert np.allclose(lse[b, h], logsumexp(s, axis=1), rtol=0, atol=1e-12)


def test_attention_8bit_p_codes_against_torch():
    """The FP8 weights: P_ij = E4M3(2^(t_ij - m_i)) with t the score in log2
    units from the dequantised operands and m_i = ceil(max_j t_ij) - 7, an
    integer; E4M3 rounding by torch's float8_e4m3fn. torch converts through
    fp32, so pairs whose p lies within 1e-9 of a rounding boundary (or whose
    fp32 value is one) are left out of the code comparison."""
    B, L, H, d = 2, 200, 2, 64
    q = RNG.standard_normal((B, L, H * d)) * np.array([1.0, 3.0])[:, None, None]
    k, v = RNG.standard_normal((2, B, L, H * d))
    k_lens = [200, 131]
    seen = {}
    O.attention_8bit(q, k, v, H, k_lens=k_lens,
                     on_head=lambda b, h, z: seen.__setitem__((b, h), (z["t"], z["m"], z["p"],
                                                                       z["P"])))
    qd, kd, _ = _dequantised(q, k, v, H, k_lens)
    e4 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float8_e4m3fn).double().numpy()
    skipped = 0
    for (b, h), (t_o, m_o, p_o, P_o) in seen.items():
        n = k_lens[b]
        t = qd[b, h] @ kd[b, h, :n].T / math.sqrt(d) / math.log(2.0)
        m = np.ceil(t.max(axis=1)) - 7
        p = np.exp2(t - m[:, None])
        assert np.array_equal(m_o, m)
        assert np.allclose(p_o, p, rtol=1e-12, atol=0)
        assert np.all(p.max(axis=1) > 64) and np.all(p.max(axis=1) <= 128)
        sure = e4(p * (1 - 1e-9)) == e4(p * (1 + 1e-9))
        skipped += int((~sure).sum())
        assert np.array_equal(P_o[sure], e4(p)[sure])
    assert skipped < 50


def test_attention_8bit_closed_forms():
    B, L, H, d = 2, 150, 2, 32
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    # all scores equal (q = 0): every p is 2^7 exactly, so o is the mean of the
    # dequantised values and lse = ln n
    _, _, vd = O.quantize_v_mxfp8(v, H, lens=[150, 77])
    oz, lz = O.attention_8bit(np.zeros_like(q), k, v, H, k_lens=[150, 77])
    for b, n in enumerate((150, 77)):
        for h in range(H):
            assert np.allclose(oz[b, :, h * d:(h + 1) * d], vd[b, h, :n].mean(axis=0)[None, :],
                               rtol=1e-14, atol=1e-15)
        assert np.allclose(lz[b], np.log(n), rtol=0, atol=1e-13)
    # one visible key: o = (E4M3(p) / p) v with p = 2^(t - ceil(t) + 7), lse = the score
    o1, l1 = O.attention_8bit(q, k, v, H, k_lens=[1, 1])
    qd, kd, vd1 = _dequantised(q, k, v, H, [1, 1])
    for b in range(B):
        for h in range(H):
            s = qd[b, h] @ kd[b, h, 0] / math.sqrt(d)
            t = s / math.log(2.0)
            p = np.exp2(t - np.ceil(t) + 7)
            ratio = O.e4m3_bits_to_f64(O.f64_to_e4m3_bits(p)) / p
            assert np.allclose(o1[b, :, h * d:(h + 1) * d], ratio[:, None] * vd1[b, h, 0],
                               rtol=1e-12, atol=1e-15)
            assert np.allclose(l1[b, h], s, rtol=0, atol=1e-12)
    # k_len 0: zeros and -inf
    o0, l0 = O.attention_8bit(q, k, v, H, k_lens=[0, 150])
    assert not o0[0].any() and np.all(np.isneginf(l0[0]))


def test_attention_8bit_keys_past_length_take_no_part():
    """Non-finite or huge keys and values at or past k_len change nothing."""
    B, L, H, d = 2, 150, 2, 32
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    o, lse = O.attention_8bit(q, k, v, H, k_lens=[100, 61])
    k2, v2 = k.copy(), v.copy()
    k2[0, 100:] = np.inf
    v2[0, 100:] = np.nan
    k2[1, 61:] = 1e4
    v2[1, 61:] = -3e4
    o2, lse2 = O.attention_8bit(q, k2, v2, H, k_lens=[100, 61])
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_attention_8bit_scalar_loops():
    """Vectorised indexing (row and key blocks, heads, rows subset) against a
    scalar loop over the same steps (tiny inputs; a consistency check, the
    pins above tie the steps to exact attention and torch's E4M3)."""
    B, L, H, d = 1, 70, 2, 16
    q, k, v = RNG.standard_normal((3, B, L, H * d))
    rows = np.array([0, 5, 63, 64, 69])
    o, lse = O.attention_8bit(q, k, v, H, k_lens=[61], scale=0.3, rows=rows)
    qc, sq = O.quantize_int8_blocks(q, H)
    kc, sk = O.quantize_int8_blocks(k, H, lens=[61])
    _, _, vd = O.quantize_v_mxfp8(v, H, lens=[61])
    for h in range(H):
        for r, i in enumerate(rows):
            ts = []
            for j in range(61):
                S = sum(int(qc[0, h, i, e]) * int(kc[0, h, j, e]) for e in range(d))
                ts.append(S * float(sq[0, h, i // 64]) * float(sk[0, h, j // 64]) * 0.3
                          / math.log(2.0))
            m = math.ceil(max(ts)) - 7
            num, den = np.zeros(d), 0.0
            for j, t in enumerate(ts):
                p = 2.0 ** (t - m)
                num += float(O.e4m3_bits_to_f64(O.f64_to_e4m3_bits(p))) * vd[0, h, j]
                den += p
            assert np.allclose(o[0, r, h * d:(h + 1) * d], num / den, rtol=1e-12, atol=1e-14)
            assert abs(lse[0, h, r] - math.log(2.0) * (m + math.log2(den))) < 1e-12
