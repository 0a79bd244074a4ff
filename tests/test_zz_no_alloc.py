"""The allocation-free self-attention entry point (wan_self_attn_fwd_noalloc)
through the C ABI against the workspace entry point it stands in for
(wan_self_attn_fwd_ws): two calls in a row on one device, the second with a
smaller input, both splitting the last round of work items into key ranges
(so the static scratch array carries partial results), must give bitwise the
same output and lse as the workspace call on the same inputs (same kernels,
same split; the workspace call gets a fresh torch buffer)."""

from __future__ import annotations

import pytest
import torch

from attention_wan_qk_amd import _lib, synth
from attention_wan_qk_amd.workloads import BY_NAME

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _rand(shape, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16).to(DEV)


def _both(q, k, v, H, k_lens=None):
    """(o, lse) of the allocation-free call and of the workspace call."""
    L = _lib.lib()
    B, T, C = q.shape
    st = torch.cuda.current_stream().cuda_stream
    kl = k_lens.data_ptr() if k_lens is not None else None
    outs = []
    for form in ("noalloc", "ws"):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, T), float("nan"), dtype=torch.float32, device=DEV)
        if form == "noalloc":
            r = L.wan_self_attn_fwd_noalloc(o.data_ptr(), lse.data_ptr(), q.data_ptr(),
                                            k.data_ptr(), v.data_ptr(), kl, B, T, H, 128, 0, 0,
                                            0, 0, 0.0, st)
        else:
            need = L.wan_self_attn_workspace_size(B, T, H, 128)
            assert need > 0, "the case must split the last round"
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            r = L.wan_self_attn_fwd_ws(o.data_ptr(), lse.data_ptr(), q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), kl, B, T, H, 128, 0, 0, 0, 0, 0.0,
                                       ws.data_ptr(), need, st)
        torch.cuda.synchronize()
        assert r == 0, f"{form}: status {r}"
        outs.append((o, lse))
    return outs


def test_no_alloc_matches_the_workspace_call_twice():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if cus != 256:
        pytest.skip(f"cases are sized for a 256-unit device, this one has {cus}")
    # first call: TI2V-5B 720P shape, 2568 items, 8 in the last round split 32 ways
    w = BY_NAME["ti2v5b-720p"]
    print("[case] no-alloc call 1: ti2v5b-720p self-attention", flush=True)
    q, k, v = (synth.tensor(w, t, DEV) for t in ("q", "k", "v"))
    (o1, l1), (o2, l2) = _both(q, k, v, w.heads)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    del q, k, v, o1, o2, l1, l2
    # second, smaller call: 2 x 4096 tokens x 3 heads (96 items, split 2 ways),
    # one sample with 50 keys, so the array keeps stale partials from call 1
    print("[case] no-alloc call 2: 2 x 4096 x 3 heads, k_lens 4096/50", flush=True)
    q, k, v = (_rand((2, 4096, 384), s) for s in (41, 42, 43))
    kl = torch.tensor([4096, 50], dtype=torch.int32, device=DEV)
    (o1, l1), (o2, l2) = _both(q, k, v, 3, kl)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.isfinite(o1.float()).all()
