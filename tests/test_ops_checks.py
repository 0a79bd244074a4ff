"""The torch binding checks every shape, stride and length before anything
reaches the library (CPU only). The C ABI receives pointers and sizes, so a
mismatch the binding let through would become out-of-bounds device reads or
writes; here a stub stands in for the library and fails the test if called."""

import pytest
import torch

from attention_wan_qk_amd import ops

bf = torch.bfloat16


@pytest.fixture(autouse=True)
def _no_library(monkeypatch):
    def forbidden():
        raise AssertionError("the library was reached")
    monkeypatch.setattr(ops, "lib", forbidden)


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def test_self_attention_shapes():
    q, k, v = t(2, 64, 256), t(2, 64, 256), t(2, 64, 256)
    with pytest.raises(ValueError):
        ops.self_attn_fwd(q, t(2, 65, 256), v, 2)          # k has more tokens
    with pytest.raises(ValueError):
        ops.self_attn_fwd(q, k, t(1, 64, 256), 2)          # v has another batch
    with pytest.raises(ValueError):
        ops.self_attn_fwd(q, k, v, 2, out=t(2, 63, 256))   # output too short
    with pytest.raises(ValueError):
        ops.self_attn_fwd(q, k, v, 2, k_lens=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(TypeError):
        ops.self_attn_fwd(q, k, v, 2, k_lens=torch.zeros(2, dtype=torch.int64))
    with pytest.raises(TypeError):                          # consistent, but not on a GPU
        ops.self_attn_fwd(q, k, v, 2, k_lens=torch.zeros(2, dtype=torch.int32))


def test_cross_and_chunk_causal_shapes():
    q, k, v = t(2, 64, 256), t(2, 32, 256), t(2, 32, 256)
    for fn in (lambda *a, **kw: ops.cross_attn_fwd(*a, **kw),
               lambda *a, **kw: ops.chunk_causal_attn_fwd(*a, q_offset=0, chunk_len=8, **kw)):
        with pytest.raises(ValueError):
            fn(q, k, t(2, 33, 256), 2)                     # v and k differ in length
        with pytest.raises(ValueError):
            fn(q, t(1, 32, 256), t(1, 32, 256), 2)         # k, v of another batch
        with pytest.raises(ValueError):
            fn(q, k, v, 2, out=t(2, 32, 256))              # output sized like k
        with pytest.raises(TypeError):
            fn(q, k, v, 2)


def test_norm_rope_outputs():
    q, k = t(1, 40, 256), t(1, 40, 256)
    wide = t(1, 40, 512)
    with pytest.raises(ValueError):                          # k_out's row stride differs from q_out's
        ops.qk_norm_rope3d(q, k, 2, (2, 4, 5), q_out=t(1, 40, 256), k_out=wide[:, :, :256])
    with pytest.raises(ValueError):
        ops.qk_norm_rope3d(q, k, 2, (2, 4, 5), q_out=t(1, 39, 256), k_out=t(1, 39, 256))
    with pytest.raises(ValueError):
        ops.qk_norm_rope3d(q, None, 2, (2, 4, 5), k_out=t(1, 40, 256))
    with pytest.raises(ValueError):
        ops.qk_norm_rope3d(q, t(1, 41, 256), 2, (2, 4, 5))
    with pytest.raises(TypeError):
        ops.qk_norm_rope3d(q, k, 2, (2, 4, 5))


def test_adaln_outputs():
    x = t(2, 10, 64)
    e = torch.zeros(2, 64)
    with pytest.raises(ValueError):
        ops.adaln_modulate_gate(x, t(2, 10, 64), e, x_out=t(2, 9, 64))
    with pytest.raises(ValueError):
        ops.adaln_modulate_gate(x, None, None, e, e, h_out=t(2, 64, 10).transpose(1, 2))
    with pytest.raises(ValueError):
        ops.adaln_modulate_gate(x, None, None, torch.zeros(3, 64), e)
    with pytest.raises(TypeError):
        ops.adaln_modulate_gate(x, None, None, e, e)


def test_linear_and_8bit():
    with pytest.raises(ValueError):
        ops.linear_fwd(t(4, 64), t(32, 64), out=t(4, 31))
    with pytest.raises(ValueError):
        ops.linear_fwd(t(4, 64), t(32, 63))
    q = t(2, 100, 256)
    with pytest.raises(ValueError):
        ops.quantize_qkv_8bit(q, q, t(2, 99, 256), 2)
    with pytest.raises(ValueError):
        ops.quantize_qkv_8bit(q, q, q, 2, k_lens=torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError):
        ops.quantize_qkv_8bit(q, q, q, 2)
    qz = {"q8": torch.zeros(1, dtype=torch.int8), "B": 2, "L": 100, "H": 2, "D": 128}
    with pytest.raises(ValueError):
        ops.self_attn_fwd_8bit(qz, out=t(2, 101, 256))
    with pytest.raises(ValueError):
        ops.self_attn_fwd_8bit(qz, k_lens=torch.zeros(5, dtype=torch.int32))
