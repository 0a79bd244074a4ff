"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of ``oracle/wan_oracle.py``
(a flipped sign, a wrong split or index, a dropped term, a transposed
operand, a missing mask) and runs ``tests/test_oracle_pins.py`` against that
copy in a scratch directory; every planted mistake must make a pin fail.
The oracle in the repository is never modified.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("rope sign", "out[..., 1::2] = a * s + b * c", "out[..., 1::2] = -a * s + b * c"),
    ("rope split", "return (c - 2 * (c // 3), c // 3, c // 3)",
     "return (c // 3, c // 3, c - 2 * (c // 3))"),
    ("rope ladder", "(2.0 * np.arange(n_a)) / (2.0 * n_a)", "(2.0 * np.arange(n_a)) / 128.0"),
    ("token order", "return np.stack([n // (h * w), (n // w) % h, n % w], axis=1)",
     "return np.stack([n // (h * w), n % h, (n // h) % w], axis=1)"),
    ("sample variance", "var = ((r - mu) ** 2).mean(axis=-1, keepdims=True)",
     "var = ((r - mu) ** 2).sum(axis=-1, keepdims=True) / (r.shape[-1] - 1)"),
    ("missing scale", "s = (q @ kk.T) * scale", "s = (q @ kk.T)"),
    ("modulation without 1+", "h = h * (1.0 + _per_row(scale, x.ndim))",
     "h = h * _per_row(scale, x.ndim)"),
    ("truncating bf16", "r = np.rint(xf / q) * q", "r = np.trunc(xf / q) * q"),
    ("half-split pairs", "a = x[..., 0::2]\n    b = x[..., 1::2]",
     "a = x[..., :x.shape[-1]//2]\n    b = x[..., x.shape[-1]//2:]"),
    ("gate on x", "r = r + (y if gate is None else _per_row(gate, x.ndim) * y)",
     "r = r + (y if gate is None else _per_row(gate, x.ndim) * x)"),
    ("rms sum", "ms = (g * g).mean(axis=-1, keepdims=True)",
     "ms = (g * g).sum(axis=-1, keepdims=True)"),
    ("ignored k_len", "n = max(0, min(int(k_len), np.shape(k)[0]))", "n = np.shape(k)[0]"),
    ("broadcast axis", "return v[:, None, :] if v.ndim == 2 and ndim == 3 else v",
     "return v[None, :, :] if v.ndim == 2 and ndim == 3 else v"),
    ("chunk of key vs query swapped", "(kj // chunk_len <= qi // chunk_len)",
     "(kj // chunk_len >= qi // chunk_len)"),
    ("cache offset ignored", "qi = q_offset + rows[:, None]", "qi = rows[:, None]"),
    ("chunk mask strict", "(kj // chunk_len <= qi // chunk_len)",
     "(kj // chunk_len < qi // chunk_len)"),
    ("linear transposed weight", "y = _f64(x) @ _f64(w).T", "y = _f64(x) @ _f64(w)"),
    ("linear bias dropped", "        y = y + _f64(bias)", "        y = y"),
    ("int8 codes truncated", "        c = np.rint((blk * inv[:, :, None, None]).astype(np.float32))",
     "        c = np.trunc((blk * inv[:, :, None, None]).astype(np.float32))"),
    ("mx scale one binade low", "        ex = np.where(amax > 0, np.maximum((fe - 1) - 8, -127), -127)",
     "        ex = np.where(amax > 0, np.maximum((fe - 1) - 7, -127), -127)"),
    ("fp8 ties away from zero", "    n = np.rint(a / q)                          # ties to even",
     "    n = np.floor(a / q + 0.5)"),
    ("P left unrounded", "            P = e4m3_bits_to_f64(f64_to_e4m3_bits(p))", "            P = p"),
    ("denominator of rounded P", "            l = p.sum(axis=1)", "            l = P.sum(axis=1)"),
    ("P offset not an integer", "m = np.ceil(t.max(axis=1)) - P_OFFSET",
     "m = t.max(axis=1) - P_OFFSET"),
    ("P offset one binade low", "P_OFFSET = 7 ", "P_OFFSET = 8 "),
    ("8-bit score without softmax scale",
     "* sk[b, h, kblk[:n]].astype(np.float64)[None, :] * sc",
     "* sk[b, h, kblk[:n]].astype(np.float64)[None, :]"),
    ("q scale of the wrong block", "    qblk = rows // INT8_BLOCK", "    qblk = 0 * rows"),
    ("key padding in k scales", "    kc, sk = quantize_int8_blocks(k, H, lens=k_lens)",
     "    kc, sk = quantize_int8_blocks(k, H)"),
    ("padding rows kept by the quantisers", "    x = np.where(valid[:, :, None], x, 0.0)",
     "    x = x"),
]


def _pins_on_copy(tmp_path, old=None, new=None):
    src = open(os.path.join(ROOT, "oracle", "wan_oracle.py")).read()
    if old is not None:
        assert src.count(old) >= 1, f"mutation site {old!r} not found"
        src = src.replace(old, new)
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle")
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / "wan_oracle.py").write_text(src)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "tests/test_oracle_pins.py"], cwd=tmp_path, env=env,
                          capture_output=True, text=True, timeout=300)


def test_unmodified_copy_passes(tmp_path):
    """Control: the scratch copy itself passes, so a failure below is the mutation's."""
    r = _pins_on_copy(tmp_path)
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(name, old, new, tmp_path):
    r = _pins_on_copy(tmp_path, old, new)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
