#!/usr/bin/env python3
"""Benchmark of the bifocal-attention hot path on one MI355X.

A step is one pass of the whole path over one synthetic batch: the bifocal
prefill of the prompt (g(s), the correction rotation, the three-pass merge) in
its single-kernel form -- every key tile corrected in LDS inside the attention
kernel, no corrected copy stored -- then one bifocal decode step of the next
token against the resulting cache (split-K kernel + combine).  The default
workload is the Qwen3-8B-shaped attention layer at 128K: batch 1, 32 query / 8
KV heads, head_dim 128, seq 131072, pretrained window 32768, local window 4096,
RoPE base 1e6 (g = 4), bf16 N(0,1) inputs from a fixed seed.

Printed (one JSON line): prefill TFLOP/s on the algorithmic count
4*D*Hq*B*s(s+1)/2 as ``value``; the roofline of the prefill kernel (bf16 MFMA
peak 2.5 PFLOP/s); the two-launch prefill (corrected keys written to a
workspace first: a deviation from the method, for comparison); the plain causal
prefill built the same way; the 64K Qwen3-1.7B-shaped prefill and the length
sweep 4K..128K in all three forms; decode HBM GB/s over the K+V bytes at caches
of 32K, 64K and 128K positions (cache slices rotated so the 256 MB last-level
cache cannot hold them) and its overhead vs the plain decode; the
sliding-window layers of hybrid models; a batch of 8 sequences of different
lengths; the prefill and decode under each long-range schedule; one
Qwen3-8B-shaped attention layer with the bifocal and with plain attention; and
the fp64 CPU oracle timed on a bounded sample of rows.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bifocal prefill TFLOP/s @128K (% MFMA peak) + decode GB/s and overhead vs plain"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
DECODE_LENGTHS = (32768, 65536, 131072)
SWEEP_LENGTHS = (4096, 16384, 32768, 49152, 98304, 131072)

WORKLOADS = {
    # name: (workload id, batch, seq, Hq, Hkv, L, W, base)
    "qwen3_8b_128k": (2, 1, 131072, 32, 8, 32768, 4096, 1e6),
    "qwen3_1p7b_64k": (1, 1, 65536, 16, 8, 32768, 4096, 1e6),
    "sweep_96k": (4, 1, 98304, 32, 8, 32768, 4096, 1e6),
    "sweep_48k": (4, 1, 49152, 32, 8, 32768, 4096, 1e6),
}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_bifocal_fused_qwen3_8b_128k_hbm_traffic.md")
ROOFLINE_KERNEL = "prefill_fused_kernel<false, false>"


def measured_traffic():
    """HBM bytes per launch of the dominant prefill kernel, from the committed
    rocprofv3 counter summary -- only while the kernel sources are the ones the
    counters were taken on (their sha256 is recorded there); else None."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    value, hashes = None, {}
    for ln in lines:
        ln = ln.strip()
        if ln.startswith("traffic_bytes_per_launch:"):
            value = int(ln.split(":", 1)[1])
        elif ln.startswith("source_sha256 "):
            name, digest = ln[len("source_sha256 "):].split(":", 1)
            hashes[name.strip()] = digest.strip()
    if value is None or not hashes:
        return None
    for name, digest in hashes.items():
        path = os.path.join(ROOT, "zero_shot_rope_attention_amd", "csrc", name)
        try:
            if hashlib.sha256(open(path, "rb").read()).hexdigest() != digest:
                return None
        except OSError:
            return None
    return value


def time_prefill(torch, stream, call, warmup=3, runs=10):
    """Average and minimum ms of `call` (one prefill) over `runs` timed calls after
    `warmup` untimed ones, HIP events on the library's stream."""
    for _ in range(warmup):
        call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(runs)]
    for e in ev:
        e[0].record(stream)
        call()
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    return float(np.mean(ms)), float(min(ms))


def prefill_forms(jl, torch, stream, q, k, v, big_l, w, base, ws, flops):
    """The three prefill forms on one problem: ms, TFLOP/s and fraction of the bf16 peak."""
    out = torch.empty_like(q)
    res = {}
    calls = {
        "fused": lambda: jl.jl_bifocal_prefill(q, k, v, out, None, big_l, w, base),
        "two_launch": lambda: jl.jl_bifocal_prefill_ws(q, k, v, out, None, big_l, w, base, ws),
        "plain": lambda: jl.jl_plain_prefill(q, k, v, out, None),
    }
    for name, call in calls.items():
        avg, mn = time_prefill(torch, stream, call)
        tf = flops / (avg * 1e-3) / 1e12
        res[name] = {"ms": round(avg, 4), "ms_min": round(mn, 4), "tflops": round(tf, 2),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    res["fused_over_plain_time"] = round(res["fused"]["ms"] / res["plain"]["ms"], 4)
    del out
    return res


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flops(b, s, hq, d=128):
    return 4.0 * d * hq * b * s * (s + 1) / 2.0


def cpu_baseline(qb, kb, vb, big_l, w, base, hq, hkv, n_rows, seed=0):
    """Time the fp64 oracle on a bounded sample: n_rows random query rows of the
    query heads of KV head 0; the rate is algorithmic FLOP/s of those rows."""
    import oracle
    from zero_shot_rope_attention_amd.inputs import bf16_bits_to_f64
    s = qb.shape[1]
    grp = hq // hkv
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(s, size=n_rows, replace=False))
    q = bf16_bits_to_f64(qb[:, :, :grp])
    k = bf16_bits_to_f64(kb[:, :, :1])
    v = bf16_bits_to_f64(vb[:, :, :1])
    t0 = time.perf_counter()
    oracle.bifocal_three_pass(q, k, v, big_l, w, base, rows=rows, row_block=16)
    dt = time.perf_counter() - t0
    flops = 4.0 * 128 * grp * float(np.sum(rows + 1))
    threads = os.environ.get("OMP_NUM_THREADS") or os.environ.get("OPENBLAS_NUM_THREADS")
    b = qb.shape[0]
    # the whole prefill at the sample's rate (the oracle's cost grows with the causal pairs)
    full_s = prefill_flops(b, s, hq) / (flops / dt)
    # decode: the oracle's one-query call on the decode lengths, the query being the workload's
    # row at position n - 1 and the cache its first n keys (every head)
    dec = []
    for n in [x for x in DECODE_LENGTHS if x <= s]:
        qd = bf16_bits_to_f64(qb[:, n - 1:n])
        kd = bf16_bits_to_f64(kb[:, :n])
        vd = bf16_bits_to_f64(vb[:, :n])
        t1 = time.perf_counter()
        oracle.bifocal_decode(qd, kd, vd, big_l, w, base)
        dd = time.perf_counter() - t1
        kv_bytes = 2 * b * n * hkv * 128 * 2
        dec.append({"n_kv": n, "seconds": round(dd, 4), "us_per_call": round(dd * 1e6, 1),
                    "kv_GB_s": round(kv_bytes / dd / 1e9, 4)})
        del qd, kd, vd
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads) if threads else os.cpu_count(),
            "kind": "oracle",
            "sample": f"{n_rows} random query rows x {grp} query heads (KV head 0) of the workload, "
                      f"fp64 numpy three-pass oracle, {dt:.1f} s; rate = algorithmic flops of those rows / time",
            "seconds": dt, "host_cpus": os.cpu_count(),
            "pairs_per_s": grp * float(np.sum(rows + 1)) / dt,
            "extrapolated_full_prefill_s": round(full_s, 1),
            "extrapolated_note": "the whole prefill (every row and head) at the sample's rate; not run",
            "decode": dec}


def bench_prefill_varlen(jl, torch, s, hq, hkv, big_l, w, base, args):
    """A variable-length prefill batch: 4 whole prompts of s/8, s/4, 3s/8 and s/2 tokens
    (16K..64K at 128K), packed, each with its own factor (g = 1, 1, 2, 2 at L = 32K);
    TFLOP/s on the algorithmic count of every sequence's causal pairs."""
    dev = torch.device("cuda:0")
    lens = [s // 8, s // 4, 3 * s // 8, s // 2]
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    total = sum(lens)
    n_max = max(lens)
    q = torch.randn(total, hq, 128, generator=gen, device=dev).to(torch.bfloat16)
    kc = torch.randn(len(lens), n_max, hkv, 128, generator=gen, device=dev).to(torch.bfloat16)
    vc = torch.randn(len(lens), n_max, hkv, 128, generator=gen, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev)
    ws = torch.empty(jl.jl_bifocal_prefill_workspace_size(len(lens), n_max, hkv), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    flops = sum(prefill_flops(1, x, hq) for x in lens)
    res = {"seq_lens": lens, "g": [jl.jl_group_factor(x, big_l) for x in lens], "flops": flops,
           "data": "seeded device normals"}
    for name in ("bifocal", "plain"):
        def call():
            if name == "bifocal":
                jl.jl_bifocal_prefill_varlen(q, kc, vc, out, None, cu, sl, n_max, big_l, w, base, ws)
            else:
                jl.jl_plain_prefill_varlen(q, kc, vc, out, None, cu, sl, n_max)
        call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record(stream)
            call()
            e[1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        res[name] = {"ms": round(ms, 3), "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}
    res["overhead_vs_plain"] = round(res["bifocal"]["ms"] / res["plain"]["ms"] - 1.0, 4)
    log(f"prefill varlen {lens}: bifocal {res['bifocal']['ms']:.2f} ms ({res['bifocal']['tflops']} TFLOP/s), "
        f"plain {res['plain']['ms']:.2f} ms")
    del q, kc, vc, out, ws
    return res


def bench_layer(jl, torch, s, hq, hkv, big_l, w, base, args, result):
    """One Qwen3-8B-shaped attention layer (hidden 4096) at this length: prefill of the
    whole prompt and one decode step, with the bifocal attention and with plain attention.
    Hidden states and weights are seeded device normals (N(0, 1), N(0, 1/fan_in))."""
    dev = torch.device("cuda:0")
    hidden = 4096
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)

    def randn(*shape, scale=1.0):
        return (torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32) * scale).to(torch.bfloat16)

    x = randn(1, s, hidden)
    w_qkv = randn((hq + 2 * hkv) * 128, hidden, scale=hidden ** -0.5)
    w_o = randn(hidden, hq * 128, scale=(hq * 128) ** -0.5)
    gq, gk = 1.0 + randn(128, scale=0.25).float(), 1.0 + randn(128, scale=0.25).float()
    gq, gk = gq.to(torch.bfloat16), gk.to(torch.bfloat16)
    kc = torch.empty((1, s, hkv, 128), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    out = torch.empty_like(x)
    ws = torch.empty(jl.jl_qwen3_layer_workspace_size(1, s, s, hq, hkv), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    res = {"shape": {"hidden": hidden, "q_heads": hq, "kv_heads": hkv, "head_dim": 128, "seq_len": s},
           "data": "seeded device normals; prefill projections by rocBLAS, a decode step's by the library's "
                   "weight-streaming kernel"}

    def prefill(bif):
        jl.jl_qwen3_attention_layer(x, w_qkv, gq, gk, w_o, out, kc, vc, ws, bifocal=bif, pretrained_window=big_l,
                                    local_window=w, rope_base=base)

    pre = {}
    for name, bif in (("bifocal", True), ("plain", False)):
        prefill(bif)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record(stream)
            prefill(bif)
            e[1].record(stream)
        torch.cuda.synchronize()
        pre[name] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    res["prefill"] = {"bifocal_ms": round(pre["bifocal"], 3), "plain_ms": round(pre["plain"], 3),
                      "overhead_vs_plain": round(pre["bifocal"] / pre["plain"] - 1.0, 4)}
    if "prefill_ms" in result and "plain_prefill" in result:
        att_b, att_p = result["prefill_ms"]["avg"], result["plain_prefill"]["ms"]
        res["prefill"]["attention_share"] = round(att_b / pre["bifocal"], 4)
        res["prefill"]["outside_attention_ms"] = round(pre["plain"] - att_p, 3)
    log(f"layer prefill (hidden {hidden}, {s} tokens): bifocal {pre['bifocal']:.2f} ms, plain {pre['plain']:.2f} ms")

    # one decode step: the token at position s-1 against the cache the prefill wrote
    x1 = x[:, -1:].contiguous()
    out1 = torch.empty_like(x1)
    ws1 = torch.empty(jl.jl_qwen3_layer_workspace_size(1, 1, s, hq, hkv), dtype=torch.uint8, device=dev)
    e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e_a.record(stream)
    torch.cuda._sleep(1_000_000)
    e_b.record(stream)
    torch.cuda.synchronize()
    spin_cycles = int(1_000_000 * 3.0 / max(e_a.elapsed_time(e_b), 1e-3))
    per = {"bifocal": [], "plain": []}
    for it in range(args.decode_warmup + args.decode_iters // 2):
        if it % 10 == 0:
            torch.cuda._sleep(spin_cycles)
        for name in ("bifocal", "plain"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            jl.jl_qwen3_attention_layer(x1, w_qkv, gq, gk, w_o, out1, kc, vc, ws1, bifocal=name == "bifocal",
                                        pretrained_window=big_l, local_window=w, rope_base=base)
            e1.record(stream)
            if it >= args.decode_warmup:
                per[name].append((e0, e1))
    torch.cuda.synchronize()
    dec = {n: float(np.median([a.elapsed_time(b_) * 1e3 for a, b_ in lst])) for n, lst in per.items()}
    res["decode"] = {"bifocal_us": round(dec["bifocal"], 2), "plain_us": round(dec["plain"], 2),
                     "overhead_vs_plain": round(dec["bifocal"] / dec["plain"] - 1.0, 4),
                     "timing": "HIP events per call, calls queued back to back behind a spin kernel; the "
                               "layer's 80 MiB of weights may stay in the last-level cache between calls"}
    log(f"layer decode step at {s}: bifocal {dec['bifocal']:.2f} us, plain {dec['plain']:.2f} us")
    del x, out, kc, vc, ws, ws1
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b_128k", choices=sorted(WORKLOADS))
    ap.add_argument("--decode-iters", type=int, default=200, help="timed decode calls per mode and length")
    ap.add_argument("--decode-warmup", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=3072, help="query rows in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the plain-prefill and decode comparisons")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run one 1 GiB device-to-device copy (reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this library runs on one GPU (no multi-GPU path); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.int16, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB (1073741824 bytes read, 1073741824 bytes written)")
        return

    import zero_shot_rope_attention_amd as jl
    from zero_shot_rope_attention_amd.inputs import make_qkv

    wid, b, s, hq, hkv, big_l, w, base = WORKLOADS[args.workload]
    g = jl.jl_group_factor(s, big_l)
    dev = torch.device("cuda:0")
    log(f"workload {args.workload}: B={b} s={s} Hq={hq} Hkv={hkv} L={big_l} W={w} base={base} g={g}")

    t0 = time.perf_counter()
    qb, kb, vb = make_qkv(wid, b, s, s, hq, hkv, 128)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(qb), up(kb), up(vb)
    log(f"inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
    out = torch.empty_like(q)
    lse = torch.empty((b, hq, s), dtype=torch.float32, device=dev)
    q_dec = q[:, -1:].contiguous()
    out_dec = torch.empty_like(q_dec)
    ws = torch.empty(jl.jl_bifocal_decode_workspace_size(b, s, hq, hkv), dtype=torch.uint8, device=dev)
    ws_pre = torch.empty(jl.jl_bifocal_prefill_workspace_size(b, s, hkv), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev):
        ev[0].record(stream)
        jl.jl_bifocal_prefill(q, k, v, out, lse, big_l, w, base)
        ev[1].record(stream)
        jl.jl_bifocal_decode(q_dec, k, v, out_dec, None, big_l, w, base, ws)
        ev[2].record(stream)

    for i in range(args.warmup):
        step([torch.cuda.Event(enable_timing=True) for _ in range(3)])
    torch.cuda.synchronize()
    log(f"{args.warmup} warmup steps done")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pre_ms = [e[0].elapsed_time(e[1]) for e in evs]
    dec_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    flops = prefill_flops(b, s, hq)
    pre_avg = float(np.mean(pre_ms))
    tflops = flops / (pre_avg * 1e-3) / 1e12
    log(f"prefill {pre_avg:.2f} ms avg ({min(pre_ms):.2f} min) -> {tflops:.1f} TFLOP/s; step {ms_step:.2f} ms")

    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": b, "seq_len": s, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": 128, "pretrained_window": big_l, "local_window": w, "rope_base": base,
                   "group_factor": g},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(),
                     "kernel": ROOFLINE_KERNEL + " (bifocal prefill, keys corrected tile by tile in LDS)",
                     "flops_per_launch": flops, "avg_launch_ms": round(pre_avg, 4),
                     "timing": "HIP events around the single-launch prefill call on its stream",
                     "traffic_note": "HBM bytes per launch of " + ROOFLINE_KERNEL + ": rocprofv3 FETCH_SIZE x 2.0 + "
                                     "WRITE_SIZE x 1.0 (scales from a 1 GiB copy), null if the kernel changed since"},
        "prefill_ms": {"avg": round(pre_avg, 4), "min": round(min(pre_ms), 4)},
        "prefill_pairs_per_s": b * hq * s * (s + 1) / 2 / (pre_avg * 1e-3),
        "decode_in_step_us": round(float(np.mean(dec_ms)) * 1e3, 2),
    }

    if not args.no_extras:
        # two-launch bifocal prefill: corrected keys written to a workspace by a pass of their own,
        # then staged like plain keys (a deviation from the method's single kernel, for comparison)
        ws_avg, ws_min = time_prefill(torch, stream, lambda: jl.jl_bifocal_prefill_ws(q, k, v, out, lse, big_l, w,
                                                                                        base, ws_pre), runs=args.steps)
        result["two_launch_prefill"] = {
            "ms": round(ws_avg, 4), "ms_min": round(ws_min, 4), "tflops": round(flops / (ws_avg * 1e-3) / 1e12, 2),
            "frac": round(flops / (ws_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kernels": "correct_keys_kernel<false> + prefill_pp_kernel<3, false, false>",
            "note": "stores a corrected copy of the keys in a caller workspace for the call; not the method's form"}
        log(f"two-launch bifocal prefill {ws_avg:.2f} ms")

        # plain causal prefill built the same way (same numerator)
        out_p = torch.empty_like(q)
        plain_ms, plain_min = time_prefill(torch, stream, lambda: jl.jl_plain_prefill(q, k, v, out_p, None),
                                           runs=args.steps)
        result["plain_prefill"] = {"ms": round(plain_ms, 4), "ms_min": round(plain_min, 4),
                                   "tflops": round(flops / (plain_ms * 1e-3) / 1e12, 2),
                                   "frac": round(flops / (plain_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                                   "bifocal_over_plain_time": round(pre_avg / plain_ms, 4)}
        log(f"plain prefill {plain_ms:.2f} ms")
        del out_p

        # length sweep (32 query / 8 KV heads, L = 32768): prefixes of the workload's tensors
        if b == 1 and hq == 32 and hkv == 8:
            sweep_p = []
            for n in SWEEP_LENGTHS:
                if n > s:
                    continue
                qs, ks, vs = q[:, :n], k[:, :n], v[:, :n]
                fl = prefill_flops(1, n, hq)
                r = {"seq_len": n, "g": jl.jl_group_factor(n, big_l), "flops": fl}
                r.update(prefill_forms(jl, torch, stream, qs, ks, vs, big_l, w, base, ws_pre, fl))
                sweep_p.append(r)
                log(f"prefill sweep {n} (g={r['g']}): fused {r['fused']['ms']} ms ({r['fused']['frac']}), "
                    f"two-launch {r['two_launch']['ms']} ms, plain {r['plain']['ms']} ms")
            result["prefill_sweep"] = sweep_p

        # the Qwen3-1.7B-shaped prefill: 16 query / 8 KV heads at 64K (g = 2), seeded device normals
        if s >= 65536:
            gen = torch.Generator(device=dev)
            gen.manual_seed(1717)
            n17, hq17 = 65536, 16
            q17 = torch.randn(1, n17, hq17, 128, generator=gen, device=dev).to(torch.bfloat16)
            k17 = torch.randn(1, n17, hkv, 128, generator=gen, device=dev).to(torch.bfloat16)
            v17 = torch.randn(1, n17, hkv, 128, generator=gen, device=dev).to(torch.bfloat16)
            fl = prefill_flops(1, n17, hq17)
            r = {"workload": "qwen3_1p7b_64k", "seq_len": n17, "q_heads": hq17, "kv_heads": hkv,
                 "g": jl.jl_group_factor(n17, big_l), "flops": fl, "data": "seeded device normals"}
            r.update(prefill_forms(jl, torch, stream, q17, k17, v17, big_l, w, base, ws_pre, fl))
            result["prefill_qwen3_1p7b_64k"] = r
            log(f"prefill qwen3-1.7B 64K: fused {r['fused']['ms']} ms ({r['fused']['frac']}), "
                f"two-launch {r['two_launch']['ms']} ms, plain {r['plain']['ms']} ms")
            del q17, k17, v17

        # sliding-window layers of a hybrid model (window W, base RoPE): prefill and decode at this length;
        # algorithmic work 4*D*Hq*B*sum_i min(p_i + 1, W)
        out_s = torch.empty_like(q)
        for _ in range(2):
            jl.jl_sliding_prefill(q, k, v, out_s, None, w)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for e in ev:
            e[0].record(stream)
            jl.jl_sliding_prefill(q, k, v, out_s, None, w)
            e[1].record(stream)
        torch.cuda.synchronize()
        sl_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        pairs = w * (w + 1) // 2 + (s - w) * w if s >= w else s * (s + 1) // 2
        sl_flops = 4.0 * 128 * hq * b * pairs
        out_sd = torch.empty_like(q_dec)
        sd = []
        for it in range(args.decode_warmup + args.decode_iters):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            jl.jl_sliding_decode(q_dec, k, v, out_sd, None, w, ws)
            e1.record(stream)
            if it >= args.decode_warmup:
                sd.append((e0, e1))
        torch.cuda.synchronize()
        sd_us = float(np.median([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in sd]))
        result["sliding_window"] = {
            "window": w,
            "prefill": {"ms": round(sl_ms, 4), "tflops": round(sl_flops / (sl_ms * 1e-3) / 1e12, 2),
                        "flops": sl_flops, "kernel": "prefill_pp_kernel<4, false, false>"},
            "decode": {"us_median": round(sd_us, 2), "kv_bytes": 2 * b * min(w, s) * hkv * 128 * 2},
        }
        log(f"sliding window W={w}: prefill {sl_ms:.2f} ms ({sl_flops / (sl_ms * 1e-3) / 1e12:.1f} TFLOP/s), "
            f"decode {sd_us:.2f} us")
        del out_s

        # decode: one query against caches of 32K, 64K and 128K positions (those up to the workload's
        # length).  Each length rotates among distinct cache slices, 1.5 GiB in total, so that the
        # 256 MB last-level cache cannot serve them; bifocal and plain interleaved in one process.
        caches = [(k, v)] + [(k.clone(), v.clone()) for _ in range(2)]
        # A decode call is shorter than the Python launch path at 32K, so calls are queued in batches
        # behind a short spin kernel: the GPU then runs them back to back and each event pair times
        # the call on the GPU, not the host's launch overhead.
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_a.record(stream)
        torch.cuda._sleep(1_000_000)
        e_b.record(stream)
        torch.cuda.synchronize()
        spin_cycles = int(1_000_000 * 3.0 / max(e_a.elapsed_time(e_b), 1e-3))  # about 3 ms per batch
        batch_iters = 10
        sweep = []
        for n in [x for x in DECODE_LENGTHS if x <= s]:
            offsets = range(0, s - n + 1, n) if b == 1 else [0]  # a slice along the length is contiguous at B=1
            slices = [(kc[:, o:o + n], vc[:, o:o + n]) for kc, vc in caches for o in offsets]
            g_n = jl.jl_group_factor(n, big_l)
            kv_bytes = 2 * b * n * hkv * 128 * 2
            per = {"bifocal": [], "plain": []}
            for it in range(args.decode_warmup + args.decode_iters):
                if it % batch_iters == 0:
                    torch.cuda._sleep(spin_cycles)
                for mi, mode in enumerate(("bifocal", "plain")):
                    # consecutive calls never share a slice, so neither finds the other's data cached
                    kc, vc = slices[(2 * it + mi) % len(slices)]
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if mode == "bifocal":
                        jl.jl_bifocal_decode(q_dec, kc, vc, out_dec, None, big_l, w, base, ws)
                    else:
                        jl.jl_plain_decode(q_dec, kc, vc, out_dec, None, ws)
                    e1.record(stream)
                    if it >= args.decode_warmup:
                        per[mode].append((e0, e1))
            torch.cuda.synchronize()
            dec = {"n_kv": n, "g": g_n, "kv_bytes": kv_bytes, "timed_runs": args.decode_iters,
                   "cache_slices": len(slices),
                   "timing": "HIP events per call on the GPU, calls queued back to back behind a spin kernel"}
            for mode, lst in per.items():
                us = np.array([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in lst])
                dec[mode] = {"us_median": round(float(np.median(us)), 2), "us_min": round(float(us.min()), 2),
                             "GB_s": round(kv_bytes / (np.median(us) * 1e-6) / 1e9, 1)}
            dec["hbm_frac"] = round(dec["bifocal"]["GB_s"] / PEAK_HBM_GBS, 4)
            dec["overhead_vs_plain"] = round(dec["bifocal"]["us_median"] / dec["plain"]["us_median"] - 1.0, 4)
            sweep.append(dec)
            log(f"decode n_kv={n} g={g_n}: bifocal {dec['bifocal']['us_median']} us ({dec['bifocal']['GB_s']} GB/s), "
                f"plain {dec['plain']['us_median']} us, overhead {dec['overhead_vs_plain'] * 100:.2f}%")
        if sweep and sweep[-1]["n_kv"] == s:
            result["decode"] = dict(sweep[-1])  # the workload's own length
        result["decode_sweep"] = sweep

        # long-range schedules (integer grouping, seam-shifted grouping, fractional scaling): the
        # single-kernel prefill and the decode at the workload's length, timed like the lines above
        scheds = {}
        for name in ("grouped", "seam", "fractional"):
            jl.jl_bifocal_prefill_sched(q, k, v, out, lse, big_l, w, base, name)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            for e in ev:
                e[0].record(stream)
                jl.jl_bifocal_prefill_sched(q, k, v, out, lse, big_l, w, base, name)
                e[1].record(stream)
            torch.cuda.synchronize()
            sp_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
            per = []
            n_it = args.decode_warmup + args.decode_iters // 2
            for it in range(n_it):
                if it % batch_iters == 0:
                    torch.cuda._sleep(spin_cycles)
                kc, vc = caches[it % len(caches)]
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                jl.jl_bifocal_decode_sched(q_dec, kc, vc, out_dec, None, None, big_l, w, base, name, ws)
                e1.record(stream)
                if it >= args.decode_warmup:
                    per.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in per]))
            kv_bytes = 2 * b * s * hkv * 128 * 2
            scheds[name] = {"factor": jl.jl_schedule_factor(s, big_l, w, name), "prefill_ms": round(sp_ms, 4),
                            "prefill_tflops": round(flops / (sp_ms * 1e-3) / 1e12, 2),
                            "decode_us_median": round(us, 2), "decode_GB_s": round(kv_bytes / (us * 1e-6) / 1e9, 1)}
            log(f"schedule {name} (factor {scheds[name]['factor']:.4g}): prefill {sp_ms:.2f} ms "
                f"({scheds[name]['prefill_tflops']} TFLOP/s), decode {us:.2f} us")
        result["schedules"] = scheds

        # the same 128K decode over a paged cache: pages of 256 positions in a shuffled order
        # (each cache copy reshaped to a page pool), bifocal and plain
        if b == 1:
            ps = 256
            n_pages = s // ps
            perm = np.random.default_rng(7).permutation(n_pages).astype(np.int32)
            table = torch.from_numpy(perm).view(1, n_pages).to(dev)
            sl = torch.tensor([s], dtype=torch.int32, device=dev)
            pools = [(kc.view(n_pages, ps, hkv, 128), vc.view(n_pages, ps, hkv, 128)) for kc, vc in caches]
            per = {"bifocal": [], "plain": []}
            for it in range(args.decode_warmup + args.decode_iters // 2):
                if it % batch_iters == 0:
                    torch.cuda._sleep(spin_cycles)
                for mi, mode in enumerate(("bifocal", "plain")):
                    kp, vp = pools[(2 * it + mi) % len(pools)]
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if mode == "bifocal":
                        jl.jl_bifocal_decode_paged(q_dec, kp, vp, out_dec, None, table, sl, big_l, w, base, ws)
                    else:
                        jl.jl_plain_decode_paged(q_dec, kp, vp, out_dec, None, table, sl, ws)
                    e1.record(stream)
                    if it >= args.decode_warmup:
                        per[mode].append((e0, e1))
            torch.cuda.synchronize()
            kv_bytes = 2 * s * hkv * 128 * 2
            pg = {"page_size": ps, "n_pages": n_pages, "order": "shuffled"}
            for mode, lst in per.items():
                us = float(np.median([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in lst]))
                pg[mode] = {"us_median": round(us, 2), "GB_s": round(kv_bytes / (us * 1e-6) / 1e9, 1)}
            pg["overhead_vs_plain"] = round(pg["bifocal"]["us_median"] / pg["plain"]["us_median"] - 1.0, 4)
            result["decode_paged"] = pg
            log(f"decode paged (pages of {ps}, shuffled): bifocal {pg['bifocal']['us_median']} us "
                f"({pg['bifocal']['GB_s']} GB/s), plain {pg['plain']['us_median']} us")
        del caches, slices

        # variable-length batched decode: 8 sequences of 16K..128K keys (g = 1..4 within one
        # launch) in a padded cache; rate = K+V bytes the sequences hold / time
        if b == 1 and s >= 131072:
            lens = [s - i * (s // 8) for i in range(8)]
            kv_b = torch.empty((8, s, hkv, 128), dtype=torch.bfloat16, device=dev)
            vv_b = torch.empty_like(kv_b)
            for i in range(8):
                kv_b[i].copy_(k[0])
                vv_b[i].copy_(v[0])
            q_b = q[:, -8:].reshape(8, 1, hq, 128).contiguous()
            out_b = torch.empty_like(q_b)
            sl = torch.tensor(lens, dtype=torch.int32, device=dev)
            ws_b = torch.empty(jl.jl_bifocal_decode_workspace_size(8, s, hq, hkv), dtype=torch.uint8, device=dev)
            held = 2 * sum(lens) * hkv * 128 * 2
            per = {"bifocal": [], "plain": []}
            for it in range(args.decode_warmup + args.decode_iters // 4):
                if it % batch_iters == 0:
                    torch.cuda._sleep(spin_cycles)
                for mode in ("bifocal", "plain"):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    if mode == "bifocal":
                        jl.jl_bifocal_decode_varlen(q_b, kv_b, vv_b, out_b, None, sl, big_l, w, base, ws_b)
                    else:
                        jl.jl_plain_decode_varlen(q_b, kv_b, vv_b, out_b, None, sl, ws_b)
                    e1.record(stream)
                    if it >= args.decode_warmup:
                        per[mode].append((e0, e1))
            torch.cuda.synchronize()
            vl = {"seq_lens": lens, "g": [jl.jl_group_factor(x, big_l) for x in lens], "kv_bytes_held": held,
                  "timed_runs": args.decode_iters // 4,
                  "timing": "HIP events per call on the GPU, calls queued back to back behind a spin kernel"}
            for mode, lst in per.items():
                us = np.array([e_a.elapsed_time(e_b) * 1e3 for e_a, e_b in lst])
                vl[mode] = {"us_median": round(float(np.median(us)), 2), "us_min": round(float(us.min()), 2),
                            "GB_s": round(held / (np.median(us) * 1e-6) / 1e9, 1)}
            vl["hbm_frac"] = round(vl["bifocal"]["GB_s"] / PEAK_HBM_GBS, 4)
            vl["overhead_vs_plain"] = round(vl["bifocal"]["us_median"] / vl["plain"]["us_median"] - 1.0, 4)
            result["decode_varlen"] = vl
            log(f"decode varlen 8 x (16K..128K): bifocal {vl['bifocal']['us_median']} us ({vl['bifocal']['GB_s']} GB/s), "
                f"plain {vl['plain']['us_median']} us, overhead {vl['overhead_vs_plain'] * 100:.2f}%")
            del kv_b, vv_b

    if not args.no_extras and b == 1:
        result["prefill_varlen"] = bench_prefill_varlen(jl, torch, s, hq, hkv, big_l, w, base, args)
        result["layer"] = bench_layer(jl, torch, s, hq, hkv, big_l, w, base, args, result)

    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(qb, kb, vb, big_l, w, base, hq, hkv, args.cpu_rows)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
