"""Benchmark of the Wan attention sublayer (one block's library calls).

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM:
  adaln (norm1 + modulate) -> qk RMSNorm + 3D RoPE -> self-attention ->
  gated residual + norm3 -> cross q/k RMSNorm -> cross-attention ->
  cross residual.
The projection GEMMs between the calls are not part of the library; their
outputs are synthetic tensors of the same shape.

Prints one JSON line (rank 0). `value` is the self-attention FLOP of a step
(4 L^2 d H B) divided by the whole step's time; the roofline object reports
the self-attention kernel alone, timed with events on its stream, against
the spec peak and against the rate of a plain MFMA loop measured in the same
run after the timed steps (libwanpeak.so; --no-measured-peaks skips it).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 / int8 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="a14b-720p-cfg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="budget of the oracle sample on the host")
    p.add_argument("--with-projections", action="store_true",
                   help="also time the block with its q/k/v/o and cross projections "
                        "(wan_linear_fwd) included (stderr only)")
    p.add_argument("--graph", action="store_true",
                   help="also time the tiny workload's step eagerly and as a replayed HIP "
                        "graph (launch overhead; stderr only)")
    p.add_argument("--attn8", action="store_true",
                   help="also time the 8-bit self-attention (quantisation + attention, "
                        "stderr only)")
    p.add_argument("--chunk-frames", type=int, default=0,
                   help="also time chunk-causal self-attention with chunks of this many "
                        "latent frames (stderr only)")
    p.add_argument("--no-back-to-back", action="store_true",
                   help="skip the back-to-back timing of the memory-bound calls (profiler runs "
                        "that count one launch per call and step)")
    p.add_argument("--no-measured-peaks", action="store_true",
                   help="skip the sustained-MFMA loop and device copy (libwanpeak) run after "
                        "the timed steps")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="first run one device copy of this many MiB (a kernel of known "
                        "traffic, to scale HBM byte counters)")
    return p.parse_args()


def kernel_source_sha(name: str) -> str:
    path = os.path.join(ROOT, "attention_wan_qk_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the summary is absent or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel, {}).get(workload)
    if not rec or rec.get("source_sha") != kernel_source_sha(rec["source"]):
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(w, tensors, budget_s: float):
    """The float64 oracle on the host, on a bounded sample of the same
    self-attention problem: 640 seeded query rows of as many (batch, head)
    pairs as fit the time budget (about 10-15 s of host work). Reported in the
    metric's unit (TFLOP/s)."""
    import numpy as np

    import oracle as O
    from attention_wan_qk_amd import synth

    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    q, k, v = tensors
    d = w.head_dim
    rows = synth.sample_rows(w, n=640)[:640]
    flop = 0.0
    pairs = 0
    t0 = time.perf_counter()
    for b in range(w.batch):
        for h in range(w.heads):
            sl = slice(h * d, (h + 1) * d)
            qb = synth.bf16_bits(q[b, rows, sl])
            kb = synth.bf16_bits(k[b, :, sl])
            vb = synth.bf16_bits(v[b, :, sl])
            O.attention(qb, kb, vb, w.tokens, 1.0 / np.sqrt(d))
            flop += 4.0 * len(rows) * w.tokens * d
            pairs += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    rate = flop / dt
    # one (batch, head) pair on a single thread
    single = None
    try:
        from threadpoolctl import threadpool_limits
        sl = slice(0, d)
        qb = synth.bf16_bits(q[0, rows[:128], sl])
        kb, vb = synth.bf16_bits(k[0, :, sl]), synth.bf16_bits(v[0, :, sl])
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            O.attention(qb, kb, vb, w.tokens, 1.0 / np.sqrt(d))
            single = 4.0 * 128 * w.tokens * d / (time.perf_counter() - t1) / 1e12
    except Exception:  # pragma: no cover
        pass
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"self-attention of {len(rows)} query rows x {pairs} (batch, head) pairs of "
                  f"{w.name} (L={w.tokens}), float64 NumPy, {dt:.1f} s incl. host copies",
        "full_problem_s_extrapolated": round(w.self_attn_flop() / rate, 1),
        "single_thread_tflops": None if single is None else round(single, 5),
    }


def breakdown_projections(args, w, ops, synth, t, per):
    """Time the projections of one block (fused q/k/v, o, cross q, fused
    cross k/v over the text context, cross o) with wan_linear_fwd and report
    the block time with them included."""
    import torch
    dev = t["x"].device
    B, L, C, Lt = w.batch, w.tokens, w.dim, w.text_len
    wt = {n: synth.tensor(w, n, dev) for n in
          ("w_qkv", "b_qkv", "w_o", "b_o", "w_cq", "b_cq", "w_ckv", "b_ckv", "w_co", "b_co",
           "context")}
    emp = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    qkv, y, cq, ckv, yc = emp(B, L, 3 * C), emp(B, L, C), emp(B, L, C), emp(B, Lt, 2 * C), \
        emp(B, L, C)
    calls = [("qkv", t["x"], "w_qkv", "b_qkv", qkv, B * L, 3 * C),
             ("o", t["y"], "w_o", "b_o", y, B * L, C),
             ("cross_q", t["x"], "w_cq", "b_cq", cq, B * L, C),
             ("cross_kv", wt["context"], "w_ckv", "b_ckv", ckv, B * Lt, 2 * C),
             ("cross_o", t["y"], "w_co", "b_co", yc, B * L, C)]
    for _ in range(args.warmup):
        for _, xin, wn, bn, out, _, _ in calls:
            ops.linear_fwd(xin, wt[wn], wt[bn], out=out)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(args.steps)]
    for s in range(args.steps):
        for i, (_, xin, wn, bn, out, _, _) in enumerate(calls):
            ev[s][i].record()
            ops.linear_fwd(xin, wt[wn], wt[bn], out=out)
        ev[s][-1].record()
    torch.cuda.synchronize()
    rec, total_ms, total_flop = {}, 0.0, 0.0
    for i, (name, _, _, _, _, M, N) in enumerate(calls):
        ms = sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
        flop = 2.0 * M * N * C
        total_ms += ms
        total_flop += flop
        tf = flop / (ms * 1e-3) / 1e12
        rec[name] = {"ms": round(ms, 3), "tflops": round(tf, 1),
                     "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
    block_ms = sum(per.values()) + total_ms
    print(json.dumps({"projections": rec, "projections_ms": round(total_ms, 3),
                      "projections_tflop": round(total_flop / 1e12, 2),
                      "block_ms_with_projections": round(block_ms, 3)}), file=sys.stderr,
          flush=True)


def graph_launch_overhead(ops, synth, n: int = 200):
    """The tiny workload's sublayer step (8 launches) is launch-bound: time it
    eagerly and as a captured, replayed HIP graph."""
    import torch
    from attention_wan_qk_amd.workloads import BY_NAME
    w = BY_NAME["tiny-5x8x8"]
    dev = "cuda:0"
    B, L, C, H, Lt = w.batch, w.tokens, w.dim, w.heads, w.text_len
    t = {k: synth.tensor(w, k, dev) for k in
         ("x", "y", "q", "k", "v", "text_k", "text_v", "cross_q", "cross_y", "gain_q",
          "gain_k", "gain_cq", "gain_ck", "mod")}
    e = t["mod"]
    emp = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    h1, qr, kr, o, x2, h3, cq, ck, oc, x3 = (emp(B, L, C) for _ in range(10))
    ck = emp(B, Lt, C)

    def step():
        ops.adaln_modulate_gate(t["x"], None, None, e[:, 0], e[:, 1], w.eps, want_x=False,
                                h_out=h1)
        ops.qk_norm_rope3d(t["q"], t["k"], H, w.grid, t["gain_q"], t["gain_k"], eps=w.eps,
                           q_out=qr, k_out=kr)
        ops.self_attn_fwd(qr, kr, t["v"], H, out=o)
        ops.adaln_modulate_gate(t["x"], t["y"], e[:, 2], None, None, w.eps, x_out=x2, h_out=h3)
        ops.qk_norm_rope3d(t["cross_q"], None, H, None, t["gain_cq"], eps=w.eps, rope=False,
                           q_out=cq)
        ops.qk_norm_rope3d(None, t["text_k"], H, None, None, t["gain_ck"], eps=w.eps,
                           rope=False, k_out=ck)
        ops.cross_attn_fwd(cq, ck, t["text_v"], H, out=oc)
        ops.adaln_modulate_gate(x2, t["cross_y"], None, None, None, w.eps, want_h=False,
                                x_out=x3)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / n

    eager_us = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    graph_us = timed(g.replay)
    print(json.dumps({"graph": {"workload": w.name, "launches_per_step": 8,
                                "eager_us_per_step": round(eager_us, 1),
                                "graph_us_per_step": round(graph_us, 1)}}),
          file=sys.stderr, flush=True)


def breakdown_attn8(args, w, ops, q, k, v, o, full_ms):
    """Time wan_quantize_qkv_8bit and wan_self_attn_fwd_8bit on the step's
    q, k, v; FLOP counted as for the bf16 call (4 L^2 d H B)."""
    import torch
    qz = ops.quantize_qkv_8bit(q, k, v, w.heads)
    for _ in range(args.warmup):
        ops.quantize_qkv_8bit(q, k, v, w.heads)
        ops.self_attn_fwd_8bit(qz, out=o)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(args.steps):
        ops.quantize_qkv_8bit(q, k, v, w.heads)
    ev[1].record()
    for _ in range(args.steps):
        ops.self_attn_fwd_8bit(qz, out=o)
    ev[2].record()
    torch.cuda.synchronize()
    qms = ev[0].elapsed_time(ev[1]) / args.steps
    ams = ev[1].elapsed_time(ev[2]) / args.steps
    flop = w.self_attn_flop()
    qbytes = 9 * w.batch * w.tokens * w.dim        # read 3 x 2 B, write 3 x 1 B per element
    tf = flop / (ams * 1e-3) / 1e12
    print(json.dumps({"attn8": {
        "quantize_ms": round(qms, 3), "quantize_gbs": round(qbytes / (qms * 1e-3) / 1e9, 1),
        "attn_ms": round(ams, 3), "tflops_effective": round(tf, 1),
        "frac_of_8bit_peak": round(tf / MFMA_FP8_PEAK_TFLOPS, 4),
        "speedup_vs_bf16_incl_quantize": round(full_ms / (qms + ams), 3)}}), file=sys.stderr,
        flush=True)


def breakdown_causal(args, w, ops, q, k, v, o, full_ms):
    """Time wan_chunk_causal_attn_fwd over the whole clip with chunks of
    ``--chunk-frames`` latent frames; FLOPs count only visible (query, key)
    pairs: 4 d H B sum_i keys_visible(i)."""
    import torch
    L, H = w.tokens, w.heads
    chunk = args.chunk_frames * w.grid[1] * w.grid[2]
    pairs = sum(min(chunk, L - c0) * min(L, c0 + chunk) for c0 in range(0, L, chunk))
    flop = 4.0 * w.head_dim * H * w.batch * pairs
    for _ in range(args.warmup):
        ops.chunk_causal_attn_fwd(q, k, v, H, 0, chunk, out=o)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(args.steps):
        ops.chunk_causal_attn_fwd(q, k, v, H, 0, chunk, out=o)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    tf = flop / (ms * 1e-3) / 1e12
    print(json.dumps({"chunk_causal": {
        "chunk_frames": args.chunk_frames, "chunk_tokens": chunk,
        "visible_fraction": round(pairs / (L * L), 4), "ms": round(ms, 4),
        "tflops_visible": round(tf, 1), "frac_mfma": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "time_vs_full": round(ms / full_ms, 4)}}), file=sys.stderr, flush=True)


def measured_peaks(memory_gbs):
    """Sustained rates of two plain loops (libwanpeak.so), run after the timed
    steps: a bf16 MFMA loop (512 workgroups of 4 waves, 4 independent
    accumulator chains per wave, random operands, ~0.3 s per launch, so that
    the chip reaches the clock it holds under full MFMA load; fastest of 3
    launches) and a 2 GiB nontemporal device copy, then the same bytes read
    alone and written alone (fastest of 10 launches each).
    Returns (MFMA TFLOP/s, copy GB/s); the memory calls' rates are printed
    against the copy on stderr."""
    import torch
    from attention_wan_qk_amd import peaks
    dev = "cuda:0"
    g = torch.Generator(device="cpu")
    g.manual_seed(20250)
    operands = torch.randn(2 * peaks.THREADS * 8, generator=g).to(torch.bfloat16).to(dev)
    blocks, iters = 512, 2_000_000
    out = torch.empty(blocks * peaks.THREADS, dtype=torch.float32, device=dev)
    peaks.mfma_bf16_loop(operands, out, blocks, 20_000)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for i in range(3):
        peaks.mfma_bf16_loop(operands, out, blocks, iters)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(3)]
    mfma_tf = peaks.mfma_loop_flop(blocks, iters) / (min(ms) * 1e-3) / 1e12
    n = 2 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    peaks.copy(dst, src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
    ev[0].record()
    for i in range(10):
        peaks.copy(dst, src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * n / (min(ev[i].elapsed_time(ev[i + 1]) for i in range(10)) * 1e-3) / 1e9
    # the same 2 GiB read alone and written alone
    words = torch.empty(peaks.read_blocks(n), dtype=torch.int32, device=dev)
    rates = []
    for run in (lambda: peaks.read(words, src), lambda: peaks.fill(dst, 0x3F803F80)):
        run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(11)]
        ev[0].record()
        for i in range(10):
            run()
            ev[i + 1].record()
        torch.cuda.synchronize()
        rates.append(n / (min(ev[i].elapsed_time(ev[i + 1]) for i in range(10)) * 1e-3) / 1e9)
    read_gbs, write_gbs = rates
    del src, dst, words
    print(json.dumps({"measured_peaks": {
        "mfma_bf16_loop_tflops": round(mfma_tf, 1), "mfma_loop_ms": [round(m, 2) for m in ms],
        "mfma_loop_frac_of_spec": round(mfma_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "copy_gbs": round(copy_gbs, 1), "copy_frac_of_spec": round(copy_gbs / HBM_PEAK_GBS, 4),
        "read_gbs": round(read_gbs, 1), "write_gbs": round(write_gbs, 1),
        "memory_calls_frac_of_copy": {k: round(v / copy_gbs, 4) for k, v in memory_gbs.items()},
    }}), file=sys.stderr, flush=True)
    return mfma_tf, copy_gbs


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch

    from attention_wan_qk_amd import _lib, ops, synth
    from attention_wan_qk_amd.workloads import BY_NAME

    if not os.path.exists(_lib.LIB_PATH):
        from attention_wan_qk_amd.build import build
        build()
    w = BY_NAME[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    B, L, C, H, Lt = w.batch, w.tokens, w.dim, w.heads, w.text_len

    t = {n: synth.tensor(w, n, dev) for n in
         ("x", "y", "q", "k", "v", "text_k", "text_v", "cross_q", "cross_y",
          "gain_q", "gain_k", "gain_cq", "gain_ck", "mod")}
    e = t["mod"]
    emp = lambda *s: torch.empty(*s, dtype=torch.bfloat16, device=dev)
    h1, qr, kr, o = emp(B, L, C), emp(B, L, C), emp(B, L, C), emp(B, L, C)
    x2, h3, cq, ck = emp(B, L, C), emp(B, L, C), emp(B, L, C), emp(B, Lt, C)
    oc, x3 = emp(B, L, C), emp(B, L, C)
    torch.cuda.synchronize()

    names = ["adaln_norm1", "qk_norm_rope3d", "self_attn", "gate_norm3", "cross_qk_norm",
             "cross_attn", "cross_residual"]
    # algorithmic HBM bytes per call (bf16 = 2 B): reads + writes of token rows
    E = B * L * C
    bytes_per = {"adaln_norm1": 4 * E, "qk_norm_rope3d": 8 * E, "gate_norm3": 8 * E,
                 "cross_qk_norm": 4 * E + 4 * B * Lt * C, "cross_residual": 6 * E}

    def c_adaln_norm1():
        ops.adaln_modulate_gate(t["x"], None, None, e[:, 0], e[:, 1], w.eps, want_x=False,
                                h_out=h1)

    def c_qk_norm_rope3d():
        ops.qk_norm_rope3d(t["q"], t["k"], H, w.grid, t["gain_q"], t["gain_k"], eps=w.eps,
                           theta=w.rope_theta, q_out=qr, k_out=kr)

    def c_self_attn():
        ops.self_attn_fwd(qr, kr, t["v"], H, out=o)

    def c_gate_norm3():
        ops.adaln_modulate_gate(t["x"], t["y"], e[:, 2], None, None, w.eps, x_out=x2, h_out=h3)

    def c_cross_qk_norm():
        ops.qk_norm_rope3d(t["cross_q"], None, H, None, t["gain_cq"], None, eps=w.eps,
                           rope=False, q_out=cq)
        ops.qk_norm_rope3d(None, t["text_k"], H, None, None, t["gain_ck"], eps=w.eps,
                           rope=False, k_out=ck)

    def c_cross_attn():
        ops.cross_attn_fwd(cq, ck, t["text_v"], H, out=oc)

    def c_cross_residual():
        ops.adaln_modulate_gate(x2, t["cross_y"], None, None, None, w.eps, want_h=False,
                                x_out=x3)

    calls = [c_adaln_norm1, c_qk_norm_rope3d, c_self_attn, c_gate_norm3, c_cross_qk_norm,
             c_cross_attn, c_cross_residual]

    def step(ev=None):
        for i, fn in enumerate(calls):
            if ev is not None:
                ev[i].record()
            fn()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(8)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    times = {n: sorted(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps))
             for i, n in enumerate(names)}
    per = {n: sum(ts) / len(ts) for n, ts in times.items()}

    attn_flop = w.self_attn_flop()
    attn_tflops = attn_flop / (per["self_attn"] * 1e-3) / 1e12
    breakdown = {}
    for n in names:
        ts = times[n]
        rec = {"ms": round(per[n], 4), "median_ms": round(ts[len(ts) // 2], 4),
               "min_ms": round(ts[0], 4)}
        if n == "self_attn":
            rec.update(tflops=round(attn_tflops, 1), frac_mfma=round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4))
        elif n == "cross_attn":
            tf = w.cross_attn_flop() / (per[n] * 1e-3) / 1e12
            rec.update(tflops=round(tf, 1), frac_mfma=round(tf / MFMA_BF16_PEAK_TFLOPS, 4))
        else:
            gbs = bytes_per[n] / (per[n] * 1e-3) / 1e9
            rec.update(gbs=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
        breakdown[n] = rec
    # The per-call events above include each launch's ramp and the gap to the
    # previous kernel; the memory-bound calls are also timed in steady state,
    # 20 back-to-back launches between two events.
    for n, fn in zip(names, calls):
        if n not in bytes_per or args.no_back_to_back:
            continue
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        e0.record()
        for _ in range(20):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        gbs = bytes_per[n] / (ms * 1e-3) / 1e9
        breakdown[n].update(back_to_back_ms=round(ms, 4), back_to_back_gbs=round(gbs, 1),
                            back_to_back_frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
    print(json.dumps({"breakdown": breakdown}), file=sys.stderr, flush=True)

    if args.with_projections:
        breakdown_projections(args, w, ops, synth, t, per)

    if args.graph:
        graph_launch_overhead(ops, synth)

    if args.attn8:
        breakdown_attn8(args, w, ops, qr, kr, t["v"], o, per["self_attn"])

    if args.chunk_frames > 0:
        breakdown_causal(args, w, ops, qr, kr, t["v"], o, per["self_attn"])

    traffic = measured_traffic("attn_fwd_kernel", w.name)
    result = {
        "metric": ("self-attn TFLOP/s (4*L^2*d*H*B) at A14B 720P CFG (75600 tok), whole block step"
                   if w.name == "a14b-720p-cfg" else
                   f"self-attn TFLOP/s (4*L^2*d*H*B) at {w.name} ({w.tokens} tok), whole block step"),
        "value": round(attn_flop / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.1) modulation, 1+0.1N gains)",
        "config": {"workload": w.name, "batch": B, "tokens": L, "grid": list(w.grid),
                   "heads": H, "head_dim": w.head_dim, "text_len": Lt,
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel (self-attention)",
            "achieved": round(attn_tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if not args.no_measured_peaks:
        gbs = {n: r.get("back_to_back_gbs", r["gbs"]) for n, r in breakdown.items() if "gbs" in r}
        mfma_tf, _ = measured_peaks(gbs)
        result["roofline"]["measured_peak"] = round(mfma_tf, 1)
        result["roofline"]["frac_of_measured_peak"] = round(attn_tflops / mfma_tf, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, (t["q"], t["k"], t["v"]), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
