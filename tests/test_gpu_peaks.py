"""The measurement aids of libwanpeak.so on the GPU: the MFMA loop's FLOP
accounting (all-ones operands make every accumulator element 16 per MFMA,
so a thread's sum is 4 chains x 16 elements x 16 x iters), the copy (bytes
identical, including a ragged last workgroup), the read (each 16 KiB block's
XOR of 4-byte words, computed again on the CPU) and the fill."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from attention_wan_qk_amd import peaks

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 5), (512, 7)])
def test_mfma_loop_counts(blocks, iters):
    print(f"[case] mfma loop blocks={blocks} iters={iters}", flush=True)
    ops_ = torch.ones(2 * peaks.THREADS * 8, dtype=torch.bfloat16, device=DEV)
    out = torch.full((blocks * peaks.THREADS,), -1.0, dtype=torch.float32, device=DEV)
    peaks.mfma_bf16_loop(ops_, out, blocks, iters)
    torch.cuda.synchronize()
    assert torch.all(out == 4 * 16 * 16 * iters)


@pytest.mark.parametrize("nbytes", [16, 16 * 1024 + 48, (1 << 20) + 48])
def test_copy(nbytes):
    print(f"[case] copy {nbytes} bytes", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8).to(DEV)
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    peaks.copy(dst[:nbytes], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src)
    assert not dst[nbytes:].any()


@pytest.mark.parametrize("nbytes", [16, 16 * 1024, 16 * 1024 + 48, (3 << 20) + 80])
def test_read_xor(nbytes):
    print(f"[case] read {nbytes} bytes", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(nbytes + 1)
    src = torch.randint(0, 256, (nbytes,), generator=g, dtype=torch.uint8)
    nb = peaks.read_blocks(nbytes)
    out = torch.full((nb,), -1, dtype=torch.int32, device=DEV)
    peaks.read(out, src.to(DEV))
    torch.cuda.synchronize()
    words = src.view(torch.int32).numpy()
    per = peaks.STREAM_BLOCK_BYTES // 4
    want = [int(np.bitwise_xor.reduce(words[i * per:(i + 1) * per])) for i in range(nb)]
    assert out.cpu().tolist() == want


@pytest.mark.parametrize("nbytes", [16, 16 * 1024 + 48, (1 << 20) + 48])
def test_fill(nbytes):
    print(f"[case] fill {nbytes} bytes", flush=True)
    buf = torch.zeros(nbytes + 64, dtype=torch.uint8, device=DEV)
    peaks.fill(buf[:nbytes], 0x3F803F80)
    torch.cuda.synchronize()
    assert torch.all(buf[:nbytes].view(torch.int32) == 0x3F803F80)
    assert not buf[nbytes:].any()
