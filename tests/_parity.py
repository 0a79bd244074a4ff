"""Comparison rule for bf16 outputs of the HIP path against the float64 oracle.

Tolerance (bf16 inputs, fp32 accumulation): max-abs 1e-2 and mean-abs 1e-3,
measured against the oracle's float64 result rounded to bf16 (nearest even),
because the output itself is bf16. Where one bf16 quantum of the value
exceeds 1e-2 (|v| >= 2), a single rounding-boundary flip between the
kernel's fp32 value and the exact value costs one quantum, so the element
bound there is that quantum; such flips must stay rare (<= 1e-3 of the
elements), which rules out a systematic one-quantum error.
"""

from __future__ import annotations

import numpy as np

import oracle as O

MAX_ABS = 1e-2
MEAN_ABS = 1e-3
MAX_FLIP_FRACTION = 1e-3


def bf16_quantum(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |r| (2**(e-8) for |r| in [2**(e-1), 2**e))."""
    _, e = np.frexp(np.abs(r))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def compare(name: str, got_bits: np.ndarray, ref64: np.ndarray, max_abs: float = MAX_ABS,
            mean_abs: float = MEAN_ABS) -> dict:
    got = O.bf16_bits_to_f64(got_bits)
    ref = O.bf16_round(ref64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    d = np.abs(got - ref)
    allowed = np.maximum(max_abs, bf16_quantum(ref))
    over = d > max_abs
    stats = {
        "n": int(d.size),
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "flips_over_1e-2": int(over.sum()),
        "rel_l2": float(np.linalg.norm(got - ref64) / max(np.linalg.norm(ref64), 1e-300)),
    }
    print(f"[parity] {name}: {stats}", flush=True)
    bad = d > allowed
    assert not bad.any(), (
        f"{name}: {int(bad.sum())} elements beyond tolerance; worst at "
        f"{np.unravel_index(np.argmax(d - allowed), d.shape)}: {stats}")
    assert stats["mean_abs"] <= mean_abs, f"{name}: mean-abs {stats['mean_abs']}"
    assert over.sum() <= max(1, MAX_FLIP_FRACTION * d.size), f"{name}: too many flips {stats}"
    return stats



def compare_chain(name: str, got_bits: np.ndarray, ref64: np.ndarray) -> dict:
    """Comparison after several dependent library calls.

    Both chains round to bf16 at every library output, so each upstream
    call's error (a rounding-boundary flip of one quantum, or the up to 1e-3
    mean error one call is allowed) is carried into every later value and
    moves later values across their own rounding boundaries; the difference
    grows along the chain (measured: mean-abs 1e-4 after the first residual,
    9e-4 six calls later). The bound for a chain takes the per-call budget
    twice (quadrature growth over about four dependent calls): mean-abs
    2e-3, elements beyond 1e-2 at most 2%, each element within four quanta
    of the reference or 2e-2, and the relative L2 error within 4e-3 (two
    bf16 unit roundoffs). A systematic error in any call (a dropped term,
    wrong gate or bias, wrong row) moves the relative L2 error by far more.
    """
    got = O.bf16_bits_to_f64(got_bits)
    ref = O.bf16_round(ref64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    d = np.abs(got - ref)
    allowed = np.maximum(2 * MAX_ABS, 4 * bf16_quantum(ref))
    over = d > MAX_ABS
    stats = {
        "n": int(d.size),
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "over_1e-2": int(over.sum()),
        "rel_l2": float(np.linalg.norm(got - ref64) / max(np.linalg.norm(ref64), 1e-300)),
    }
    print(f"[parity chain] {name}: {stats}", flush=True)
    bad = d > allowed
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond four quanta: {stats}"
    assert stats["mean_abs"] <= 2 * MEAN_ABS, f"{name}: mean-abs {stats['mean_abs']}"
    assert over.sum() <= max(1, 2e-2 * d.size), f"{name}: too many elements over 1e-2 {stats}"
    assert stats["rel_l2"] <= 4e-3, f"{name}: relative L2 error {stats['rel_l2']}"
    return stats


def _e4m3(x):
    return O.e4m3_bits_to_f64(O.f64_to_e4m3_bits(x))


def p_code_spread(z: dict) -> np.ndarray:
    """How far an fp32 evaluation of the 8-bit attention may move each FP8
    weight P_ij from the oracle's (per (row, key), in the oracle's units).

    The oracle forms t - m exactly. An fp32 evaluation from the integer
    score S has |error in t - m| <= eps_ij, the sum of:
      * 2^-20 |t_ij|: its multiplier sq sk scale log2(e) after five fp32
        roundings (2^-24 each) and truncation to 22 significant bits
        (3 * 2^-23);
      * unit_ij + 2^-24 (|m_i| + 1): a folded constant of magnitude up to
        1.5 * 2^23 * unit + |m| rounded once (half an ulp: 0.75 unit), which
        is how an fp32 value of the INT8 accumulator offset by 2^23 + 2^22
        is cancelled;
      * 2^-24 |t_ij - m_i| (the fused multiply-add) and 2^-22 (exp2 to one ulp).
    Its integer offset may also sit at m - 3 .. m + 1: a streaming evaluation
    need only raise its running offset before a weight would pass 448,
    E4M3's largest value (448 < 2^9, and the offset it then takes is the
    ceiling of an fp32 maximum, minus 7). That multiplies every weight by
    2^s, s in {-1, 0, 1, 2, 3}, which leaves normal E4M3 roundings unchanged
    and moves only weights below 2^-4 (subnormal under some s). The spread is
    the largest minus the smallest E4M3 value among those choices.
    """
    t, m, p, unit = z["t"], z["m"], z["p"], z["unit"]
    eps = (2.0 ** -20 * np.abs(t) + unit + 2.0 ** -24 * (np.abs(m)[:, None] + 1)
           + 2.0 ** -24 * np.abs(t - m[:, None]) + 2.0 ** -22)
    f = np.exp2(eps)
    lo, hi = _e4m3(p / f), _e4m3(p * f)
    spread = hi - lo
    small = p < 2.0 ** -4
    if small.any():
        ps, fs = p[small], f[small]
        c = [lo[small], hi[small]]
        for s in (-1, 1, 2, 3):
            k = 2.0 ** s
            c += [_e4m3(ps * k / fs) / k, _e4m3(ps * k * fs) / k]
        c = np.stack(c)
        spread[small] = c.max(axis=0) - c.min(axis=0)
    return spread


class P8Bound:
    """Collects, through the oracle's ``on_head`` hook, the per-element bound
    sum_j spread_ij |v_jd| / l_i on how far the P codes an fp32 evaluation
    may pick move o (output layout [B, rows, H*d])."""

    def __init__(self, B: int, rows: int, H: int, d: int):
        self.d = d
        self.bound = np.zeros((B, rows, H * d))

    def __call__(self, b, h, z):
        s = p_code_spread(z)
        self.bound[b, :, h * self.d:(h + 1) * self.d] = (s @ np.abs(z["v"])) / z["l"][:, None]


def compare_8bit(name: str, got_bits: np.ndarray, ref64: np.ndarray, p_bound: np.ndarray) -> dict:
    """Comparison for the 8-bit attention output against the oracle that
    follows the "8-bit FlashAttention" reading (exact scores and
    denominators, E4M3 weights in the P V product).

    q, k and v codes are identical on both sides (checked bit for bit
    elsewhere). Per element: |got - bf16(ref)| <= max(1e-2, one bf16
    quantum of ref) + p_bound, where p_bound (P8Bound) is what the FP8
    weights an fp32 evaluation may legitimately pick can move that element;
    the 1e-2 term covers fp32 accumulation of sum P v and sum p over the
    keys (relative error <= (keys / 8) 2^-24, well under 1e-2 at the
    values' sizes). Mean-abs <= 1e-3 as for every call.
    """
    got = O.bf16_bits_to_f64(got_bits)
    ref = O.bf16_round(ref64)
    assert got.shape == ref.shape == p_bound.shape, (name, got.shape, ref.shape, p_bound.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    d = np.abs(got - ref)
    base = np.maximum(MAX_ABS, bf16_quantum(ref))
    allowed = base + p_bound
    stats = {
        "n": int(d.size),
        "max_abs": float(d.max()) if d.size else 0.0,
        "mean_abs": float(d.mean()) if d.size else 0.0,
        "beyond_per_call_rule": int((d > base).sum()),
        "max_p_bound": float(p_bound.max()) if d.size else 0.0,
        "mean_p_bound": float(p_bound.mean()) if d.size else 0.0,
        "rel_l2": float(np.linalg.norm(got - ref64) / max(np.linalg.norm(ref64), 1e-300)),
    }
    print(f"[parity 8bit] {name}: {stats}", flush=True)
    bad = d > allowed
    assert not bad.any(), (
        f"{name}: {int(bad.sum())} elements beyond the bound; worst at "
        f"{np.unravel_index(np.argmax(d - allowed), d.shape)}: {stats}")
    assert stats["mean_abs"] <= MEAN_ABS, f"{name}: mean-abs {stats['mean_abs']}"
    return stats
