"""The C ABI library: it loads, exports every call declared in
include/wanattn.h, and rejects bad arguments on the host before launching
anything. No kernel runs here: every call below either fails a host check or
has no work (B * L == 0), and the fake device addresses are never
dereferenced.

Not collected on its own: tests/test_abi.py runs this file in a child process
that sees no GPU (so a host check that regressed would end in a launch error,
not a device access), and again against a host-only build of the ABI layer
under the address and undefined-behaviour sanitizers (WANATTN_TEST_LIB names
that build)."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wanattn.h")

INV, NS, OK = 1, 2, 0
A = 0x10000          # fake, 16-byte aligned "device" addresses: never dereferenced
MB = 1 << 26


def lib_path():
    from attention_wan_qk_amd import _lib
    return os.environ.get("WANATTN_TEST_LIB") or _lib.LIB_PATH


@pytest.fixture(scope="module")
def L():
    from attention_wan_qk_amd import _lib
    path = lib_path()
    if not os.path.exists(path):
        pytest.fail(f"{path} is missing: build it first")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _lib.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def declared_calls():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(wan_\w+)\s*\(", src, re.M)))


def test_header_declares_every_call():
    calls = declared_calls()
    for name in ("wan_qk_norm_rope3d", "wan_self_attn_fwd", "wan_cross_attn_fwd",
                 "wan_adaln_modulate_gate", "wan_chunk_causal_attn_fwd", "wan_linear_fwd",
                 "wan_status_string", "wan_version"):
        assert name in calls


def test_library_exports_every_declared_symbol(L):
    from attention_wan_qk_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (wan_\w+)", out))
    for name in declared_calls():
        assert name in exported, name
        assert hasattr(L, name)
    assert set(_lib.SIGNATURES) == set(declared_calls())


def test_status_strings_and_version(L):
    assert L.wan_status_string(0) == b"WAN_SUCCESS"
    assert L.wan_status_string(1) == b"WAN_ERROR_INVALID_VALUE"
    assert L.wan_status_string(2) == b"WAN_ERROR_NOT_SUPPORTED"
    assert L.wan_status_string(3) == b"WAN_ERROR_LAUNCH"
    assert L.wan_version() >= 100


def norm_rope(L, **kw):
    a = dict(q_out=A, k_out=A + MB, q=A + 2 * MB, k=A + 3 * MB, gq=None, gk=None, B=1, Lt=12,
             H=2, D=128, f=1, h=3, w=4, ld_in=0, ld_out=0, eps=1e-6, theta=1e4, flags=3)
    a.update(kw)
    return L.wan_qk_norm_rope3d(a["q_out"], a["k_out"], a["q"], a["k"], a["gq"], a["gk"],
                                a["B"], a["Lt"], a["H"], a["D"], a["f"], a["h"], a["w"],
                                a["ld_in"], a["ld_out"], a["eps"], a["theta"], a["flags"], None)


def test_norm_rope_rejections(L):
    assert norm_rope(L, D=64) == NS
    assert norm_rope(L, H=65) == NS                       # C > 8192
    assert norm_rope(L, q=None, k=None, q_out=None, k_out=None) == INV
    assert norm_rope(L, q=None) == INV                    # output without input
    assert norm_rope(L, q=A + 2 * MB + 2) == INV          # misaligned
    assert norm_rope(L, f=2) == INV                       # grid != L
    assert norm_rope(L, h=1025, w=1, f=1, Lt=1025) == INV  # > table length
    assert norm_rope(L, flags=8) == INV
    assert norm_rope(L, flags=4) == INV                   # per-head without norm
    assert norm_rope(L, ld_in=200) == INV                 # < C
    assert norm_rope(L, ld_in=260) == INV                 # not a multiple of 8
    assert norm_rope(L, eps=-1.0) == INV
    assert norm_rope(L, theta=1.0) == INV
    assert norm_rope(L, q_out=A + 2 * MB + 16) == INV     # partial overlap with q
    assert norm_rope(L, q_out=A + 2 * MB, ld_out=512) == INV  # in place, stride differs
    assert norm_rope(L, q_out=A + 3 * MB) == INV          # q_out == k (other input)
    assert norm_rope(L, B=0) == OK                        # nothing to do
    assert norm_rope(L, Lt=0) == OK


def attn(L, **kw):
    a = dict(o=A, lse=None, q=A + MB, k=A + 2 * MB, v=A + 3 * MB, kl=None, B=1, Lt=64, H=2,
             D=128, lq=0, lk=0, lv=0, lo=0, scale=0.0)
    a.update(kw)
    return L.wan_self_attn_fwd(a["o"], a["lse"], a["q"], a["k"], a["v"], a["kl"], a["B"],
                               a["Lt"], a["H"], a["D"], a["lq"], a["lk"], a["lv"], a["lo"],
                               a["scale"], None)


def test_self_attn_rejections(L):
    assert attn(L, D=64) == NS
    assert attn(L, o=None) == INV
    assert attn(L, v=None) == INV
    assert attn(L, q=A + MB + 8) == INV
    assert attn(L, o=A + MB) == INV                       # o aliases q
    assert attn(L, o=A + 2 * MB + 256) == INV             # o overlaps k
    assert attn(L, lse=A + 3 * MB) == INV                 # lse overlaps v
    assert attn(L, lq=100) == INV
    assert attn(L, lk=248) == INV                         # multiple of 8 but < C=256
    assert attn(L, lo=260) == INV
    assert attn(L, H=0) == INV
    assert attn(L, B=-1) == INV
    assert attn(L, scale=float("nan")) == INV
    assert attn(L, scale=float("inf")) == INV
    assert attn(L, B=0) == OK
    assert attn(L, Lt=0) == OK
    # keys of one (batch, head) spanning more than 4 GiB (32-bit byte offsets)
    far = dict(o=A, q=A + (1 << 36), k=A + (2 << 36), v=A + (3 << 36), lq=4096, lk=4096,
               lv=4096, lo=4096)
    assert attn(L, Lt=1 << 20, **far) == NS


def test_self_attn_workspace_rejections(L):
    G = 1 << 28                          # fake tensors of 167 MB each stay apart
    B, Lq, H = 1, 27280, 24              # 2568 work items: 8 in the last round of a 256-unit device
    need = L.wan_self_attn_workspace_size(B, Lq, H, 128)
    assert L.wan_self_attn_workspace_size(0, Lq, H, 128) == 0
    assert L.wan_self_attn_workspace_size(B, Lq, H, 64) == 0
    assert L.wan_self_attn_workspace_size(1, 1024, 1, 128) == 0     # too few key tiles to split

    def ws(**kw):
        a = dict(o=A, lse=None, q=A + G, k=A + 2 * G, v=A + 3 * G, kl=None, B=B, L=Lq, H=H,
                 D=128, ws=A + 4 * G, wsb=need, scale=0.0)
        a.update(kw)
        return L.wan_self_attn_fwd_ws(a["o"], a["lse"], a["q"], a["k"], a["v"], a["kl"], a["B"],
                                      a["L"], a["H"], a["D"], 0, 0, 0, 0, a["scale"], a["ws"],
                                      a["wsb"], None)
    assert ws(B=0, ws=None, wsb=0) == OK
    assert ws(D=64) == NS
    assert ws(q=None) == INV
    assert ws(o=A + G) == INV                # o overlaps q
    if need == 0:                            # no device to plan for: the workspace is unused
        return
    assert need == 8 * 32 * (256 * 128 + 2 * 256) * 4
    assert ws(ws=None) == INV
    assert ws(wsb=need - 16) == INV
    assert ws(ws=A + 4 * G + 8) == INV       # misaligned
    assert ws(ws=A + 2 * G) == INV           # overlaps k
    assert ws(lse=A + 4 * G + 64, ws=A + 4 * G) == INV   # overlaps lse


def test_self_attn_noalloc_rejections(L):
    def na(**kw):
        a = dict(o=A, lse=None, q=A + MB, k=A + 2 * MB, v=A + 3 * MB, kl=None, B=1, L=100, H=2,
                 D=128, lq=0, lk=0, lv=0, lo=0, scale=0.0)
        a.update(kw)
        return L.wan_self_attn_fwd_noalloc(a["o"], a["lse"], a["q"], a["k"], a["v"], a["kl"],
                                           a["B"], a["L"], a["H"], a["D"], a["lq"], a["lk"],
                                           a["lv"], a["lo"], a["scale"], None)
    assert na(B=0) == OK
    assert na(D=64) == NS
    assert na(q=None) == INV
    assert na(o=A + 8) == INV                # misaligned
    assert na(o=A + MB) == INV               # o overlaps q
    assert na(lo=100) == INV
    assert na(scale=float("nan")) == INV
    if os.environ.get("WANATTN_TEST_LIB"):
        # host-only build: a call that needs the scratch array cannot look it up
        # there (its stand-in reports no device) and must say so, not launch
        G = 1 << 28
        assert na(q=A + G, k=A + 2 * G, v=A + 3 * G, L=27280, H=24) == 3


def test_cross_attn_rejections(L):
    def cross(**kw):
        a = dict(o=A, q=A + MB, k=A + 2 * MB, v=A + 3 * MB, cl=None, B=1, Lq=64, Lk=32, H=2,
                 D=128, lq=0, lkv=0, lo=0, scale=0.0)
        a.update(kw)
        return L.wan_cross_attn_fwd(a["o"], a["q"], a["k"], a["v"], a["cl"], a["B"], a["Lq"],
                                    a["Lk"], a["H"], a["D"], a["lq"], a["lkv"], a["lo"],
                                    a["scale"], None)
    assert cross(Lk=0) == INV
    assert cross(D=96) == NS
    assert cross(o=A + 3 * MB) == INV
    assert cross(k=A + 2 * MB + 4) == INV
    assert cross(Lq=0) == OK


def test_adaln_rejections(L):
    def adaln(**kw):
        a = dict(xo=A, ho=A + MB, x=A + 2 * MB, y=A + 3 * MB, g=A + 4 * MB, sh=A + 5 * MB,
                 sc=A + 6 * MB, B=1, Lt=8, C=256, sb=0, sl=0, eps=1e-6)
        a.update(kw)
        return L.wan_adaln_modulate_gate(a["xo"], a["ho"], a["x"], a["y"], a["g"], a["sh"],
                                         a["sc"], a["B"], a["Lt"], a["C"], a["sb"], a["sl"],
                                         a["eps"], None)
    assert adaln(C=100) == INV                  # not a multiple of 8
    assert adaln(C=8200) == NS
    assert adaln(xo=None, ho=None) == INV
    assert adaln(x=None) == INV
    assert adaln(ho=A) == INV                   # x_out and h_out overlap
    assert adaln(xo=A + 2 * MB + 16) == INV     # partial overlap with x
    assert adaln(g=A + 4 * MB + 4) == INV       # misaligned modulation
    assert adaln(sb=-8) == INV
    assert adaln(eps=float("nan")) == INV
    assert adaln(B=0) == OK


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from attention_wan_qk_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_chunk_causal_rejections(L):
    def cc(**kw):
        a = dict(o=A, lse=None, q=A + MB, k=A + 2 * MB, v=A + 3 * MB, kl=None, B=1, Lq=64, Lk=96,
                 H=2, D=128, off=32, cl=16, lq=0, lk=0, lv=0, lo=0, scale=0.0)
        a.update(kw)
        return L.wan_chunk_causal_attn_fwd(a["o"], a["lse"], a["q"], a["k"], a["v"], a["kl"],
                                           a["B"], a["Lq"], a["Lk"], a["H"], a["D"], a["off"],
                                           a["cl"], a["lq"], a["lk"], a["lv"], a["lo"],
                                           a["scale"], None)
    assert cc(cl=0) == INV
    assert cc(off=-1) == INV
    assert cc(Lk=0) == INV
    assert cc(D=64) == NS
    assert cc(o=A + MB) == INV
    assert cc(Lq=0) == OK


def test_linear_rejections(L):
    def lin(**kw):
        a = dict(y=A, x=A + MB, w=A + 2 * MB, b=None, M=300, N=264, K=200, lx=0, lw=0, ly=0)
        a.update(kw)
        return L.wan_linear_fwd(a["y"], a["x"], a["w"], a["b"], a["M"], a["N"], a["K"],
                                a["lx"], a["lw"], a["ly"], None)
    assert lin(M=0) == OK
    assert lin(M=-1) == INV
    assert lin(N=0) == INV
    assert lin(K=0) == INV
    assert lin(N=260) == INV           # N not a multiple of 8
    assert lin(K=204) == INV           # K not a multiple of 8
    assert lin(lx=192) == INV          # ld_x < K
    assert lin(lw=208, ly=260) == INV  # ld_y not a multiple of 8
    assert lin(x=None) == INV
    assert lin(y=A + 8) == INV         # misaligned
    assert lin(b=A + 2 * MB + 4) == INV
    assert lin(y=A + MB + 16) == INV   # y overlaps x
    assert lin(b=A + 16) == INV        # bias inside y
    assert lin(lx=1 << 23) == NS       # 256 rows exceed a 32-bit buffer range


def test_8bit_rejections(L):
    def qz(**kw):
        a = dict(q8=A, k8=A + MB, v8=A + 2 * MB, sq=A + 3 * MB, sk=A + 4 * MB, sv=A + 5 * MB,
                 q=A + 6 * MB, k=A + 7 * MB, v=A + 8 * MB, kl=None, B=1, L=100, H=2, D=128,
                 lq=0, lk=0, lv=0)
        a.update(kw)
        return L.wan_quantize_qkv_8bit(a["q8"], a["k8"], a["v8"], a["sq"], a["sk"], a["sv"],
                                       a["q"], a["k"], a["v"], a["kl"], a["B"], a["L"], a["H"],
                                       a["D"], a["lq"], a["lk"], a["lv"], None)
    assert qz(L=0) == OK
    assert qz(D=64) == NS
    assert qz(H=0) == INV
    assert qz(q8=None) == INV
    assert qz(sk=A + 4 * MB + 4) == INV       # misaligned
    assert qz(lq=200) == INV                  # row stride < H*D
    assert qz(k8=A + 16) == INV               # outputs overlap
    assert qz(q=A + 2 * MB) == INV            # output overlaps an input
    assert qz(B=1 << 20, L=1 << 18) == NS     # 2^33 blocks: beyond one launch
    assert qz(kl=A + 9 * MB + 2) == INV       # misaligned key lengths

    def at(**kw):
        a = dict(o=A, lse=None, q8=A + MB, k8=A + 2 * MB, v8=A + 3 * MB, sq=A + 4 * MB,
                 sk=A + 5 * MB, sv=A + 6 * MB, kl=None, B=1, L=100, H=2, D=128, lo=0, scale=0.0)
        a.update(kw)
        return L.wan_self_attn_fwd_8bit(a["o"], a["lse"], a["q8"], a["k8"], a["v8"], a["sq"],
                                        a["sk"], a["sv"], a["kl"], a["B"], a["L"], a["H"], a["D"],
                                        a["lo"], a["scale"], None)
    assert at(B=0) == OK
    assert at(D=256) == NS
    assert at(o=A + MB) == INV                # o overlaps q8
    assert at(lse=A + 6 * MB + 8) == INV      # lse inside v_scale
    assert at(lo=100) == INV
    assert at(scale=float("nan")) == INV
    assert at(v8=None) == INV
    assert at(L=(1 << 18) + 1) == NS          # key-block scales beyond the LDS table
    assert at(B=1 << 20, L=1 << 18, H=16) == NS   # 2^34 workgroups: beyond one launch


PEAK_HEADER = os.path.join(ROOT, "include", "wanpeak.h")


@pytest.fixture(scope="module")
def P():
    from attention_wan_qk_amd import peaks
    if not os.path.exists(peaks.LIB_PATH):
        from attention_wan_qk_amd.build import build
        build(verbose=False)
    return peaks.lib()


def test_peak_library_exports_and_host_checks(P):
    """libwanpeak.so (the benchmark's measurement aids) exports what
    include/wanpeak.h declares and rejects bad arguments before launching."""
    from attention_wan_qk_amd import peaks
    declared = sorted(set(re.findall(r"^\s*int\s+(wanpeak_\w+)\s*\(", open(PEAK_HEADER).read(),
                                     re.M)))
    assert declared == ["wanpeak_copy", "wanpeak_fill", "wanpeak_mfma_bf16_loop",
                        "wanpeak_read"]
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert set(re.findall(r"\bT (wanpeak_\w+)", out)) == set(declared)
    loop = P.wanpeak_mfma_bf16_loop
    assert loop(None, A, 1, 1, None) == 1
    assert loop(A, None, 1, 1, None) == 1
    assert loop(A, A, 0, 1, None) == 1
    assert loop(A, A, 65537, 1, None) == 1
    assert loop(A, A, 1, 0, None) == 1
    assert loop(A + 8, A, 1, 1, None) == 1          # operands not 16-byte aligned
    assert loop(A, A + 2, 1, 1, None) == 1          # out not 4-byte aligned
    cp = P.wanpeak_copy
    assert cp(None, A, 16, None) == 1
    assert cp(A, A + MB, 24, None) == 1              # not a multiple of 16
    assert cp(A + 8, A + MB, 16, None) == 1          # misaligned
    assert cp(A, A + 16, 32, None) == 1              # overlapping ranges
    assert cp(A, A + MB, 0, None) == 0               # nothing to do: no launch
    rd = P.wanpeak_read
    assert rd(None, A, 16, None) == 1
    assert rd(A, None, 16, None) == 1
    assert rd(A + MB, A, 24, None) == 1              # not a multiple of 16
    assert rd(A + MB, A + 8, 16, None) == 1          # source misaligned
    assert rd(A + MB + 2, A, 16, None) == 1          # out not 4-byte aligned
    assert rd(A + 16, A, 1 << 20, None) == 1         # out inside the source
    assert rd(A + MB, A, 0, None) == 0               # nothing to do: no launch
    fl = P.wanpeak_fill
    assert fl(None, 16, 0, None) == 1
    assert fl(A, 24, 0, None) == 1                   # not a multiple of 16
    assert fl(A + 8, 16, 0, None) == 1               # misaligned
    assert fl(A, 0, 0, None) == 0                    # nothing to do: no launch
    assert peaks.read_blocks(1) == 1 and peaks.read_blocks(16384) == 1
    assert peaks.read_blocks(16385) == 2
    assert peaks.mfma_loop_flop(512, 10) == 512 * 4 * 10 * 4 * 32768
