#!/usr/bin/env python3
"""Benchmark of the QSVD latent-attention hot path on one MI355X.

Decode leg (the headline): one decode step of a LLaVA-v1.5-7B-shaped joint-QKV
latent-attention layer, E = 4096 (32 heads x 128), r = 1536, b = 16 sequences,
L = 8192 cached bf16 latents each; the step is qsvd_decode_attn (absorb,
split-L stream, merge, finalize).  value = decode tokens/s = b / step time.

Explicit leg: the same step with K and V rebuilt explicitly on chip and
rotary positions (qsvd_decode_attn_explicit), against the bf16 MFMA peak.

Per-head latent leg: the same attention shape with per-head latents (each
head caches rk = 64 key and rv = 64 value latents per token; keys rebuilt on
chip with RoPE, B_Vh applied after the softmax; qsvd_decode_attn_headwise),
against the HBM peak.

Other decode configurations: the W8A4 shape (int4 group-128 latent cache,
r = 768, int8 W^u) and the LLaVA-v1.5-13B shape (r = 2304, 40 heads, b = 8,
L = 16384, bf16 cache; two-pass stream), each with its stream kernels priced
against the HBM peak.

Prefill leg: the shared down-projection at W8A8, X [16384][4096] int8 (H1
rotated, per-token scales) times W^d [4096][1536] int8 (per-column scales),
reported as TOPS; plus the rotate+quantise steps around it.

All inputs are seeded synthetic data (synth/); the cache copies are rotated
between steps so that the 256 MiB last-level cache cannot serve a step from
the previous one.  Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
COPY_BYTES = 1 << 30  # calibration copy (bytes read = bytes written)
MALL_BYTES = 256 << 20  # MI355X last-level (Infinity) cache
COUNTERS = os.path.join(ROOT, "profiles", "decode_stream_e4096_r1536_b16_l8192_counters.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clock climbs for ~20 ms of work after the idle input generation;
    # 200 decode steps (~22 ms) reach the steady state
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--copies", type=int, default=2,
                    help="minimum rotated cache copies (raised per leg to span 2 x 256 MiB)")
    ap.add_argument("--splits", type=int, default=0, help="L-splits (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-chain", action="store_true", help="skip the 24-layer prefill chain")
    ap.add_argument("--no-tiny", action="store_true", help="skip the tiny float32 latency leg")
    ap.add_argument("--no-explicit", action="store_true",
                    help="skip the explicit K/V reconstruction (RoPE) decode leg")
    ap.add_argument("--no-headwise", action="store_true",
                    help="skip the per-head latent (RoPE) decode leg")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the W8A4 (int4 cache) and 13B (two-pass) decode legs")
    return ap.parse_args()


def source_hash(name: str) -> str:
    h = hashlib.sha256()
    with open(os.path.join(ROOT, "rank_latent_attention_amd", "csrc", name), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    return source_hash("decode.hip")


def timed(fn, steps, warmup, stats=None):
    """Mean milliseconds per call of fn over exactly `steps` calls after `warmup`
    untimed ones, bracketed by synchronisations and a pair of HIP events on the
    current stream.  With a dict `stats`, events at block boundaries (every
    ~steps/10 calls, one marker per block) also give the median, p10 and p90 of
    the per-call time over the blocks."""
    import numpy as np
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    nblk = min(10, steps) if stats is not None else 1
    bounds = [round(k * steps / nblk) for k in range(nblk + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nblk + 1)]
    evs[0].record()
    for k in range(nblk):
        for i in range(bounds[k], bounds[k + 1]):
            fn(i)
        evs[k + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    if stats is not None:
        per = np.array([evs[k].elapsed_time(evs[k + 1]) / (bounds[k + 1] - bounds[k]) for k in range(nblk)])
        stats.update({"median_ms": round(float(np.median(per)), 5),
                      "p10_ms": round(float(np.percentile(per, 10)), 5),
                      "p90_ms": round(float(np.percentile(per, 90)), 5), "blocks": nblk})
    return ms


def kernel_times(q, torch, step, steps):
    """Per-kernel launch times over `steps` calls of step, from the library's timing
    session (one launch-boundary event before every kernel; a launch's time runs to
    the next boundary, so the kernels of a step add up to the step).  Returns
    ({kernel: mean ms per launch}, mean ms per step of this pass)."""
    with q.timing(max_launches=8 * steps + 16) as tm:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    kern = {k: v[1] / v[0] for k, v in tm.result.items()}
    per_step = sum(v[1] for v in tm.result.values()) / steps
    return kern, per_step


def copies_for(working_set_bytes, requested):
    """Cache copies rotated between steps: at least `requested`, and enough that the
    copies together span twice the 256 MiB last-level cache, so that no step is served
    from the previous step's lines."""
    return max(requested, -(-2 * MALL_BYTES // max(int(working_set_bytes), 1)))


def environment():
    import torch
    info = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip,
            "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    return info


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the latent-attention "
              "decode shards by sequence with no communication, so N GPUs run N independent "
              "copies of this single-GPU step.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import rank_latent_attention_amd as q
    import synth

    torch.cuda.set_device(0)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda u16: dev(u16.view(np.int16)).view(torch.bfloat16)

    # ------------------------------------------------------------------ decode
    cfg = synth.CONFIGS[1]
    b, L, r, heads, d = cfg.b, cfg.L, cfg.r, cfg.heads, cfg.d
    t0 = time.time()
    cs = synth.config_decode_case(cfg)
    log(f"[bench] generated decode inputs ({cfg.name}) in {time.time() - t0:.1f}s")
    C0 = bf(cs.C)
    cache_bytes = b * L * r * 2                       # one r-wide bf16 latent per cached token
    step_bytes = cache_bytes + 2 * r * heads * d * 2 + 2 * b * heads * d * 2
    n_copies = copies_for(step_bytes, args.copies)
    copies = [C0] + [C0.clone() for _ in range(n_copies - 1)]
    qv, Wk, Wv = bf(cs.q), bf(cs.Wu_k), bf(cs.Wu_v)
    O = torch.empty((b, heads, d), dtype=torch.bfloat16, device="cuda")
    ws_bytes = q.qsvd_decode_workspace_bytes(b, L, r, heads, d, q.BF16, args.splits)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    splits = args.splits or q.qsvd_decode_default_splits(b, L, r, heads, d, q.BF16)

    def step(i):
        q.qsvd_decode_attn(qv, q.BF16, copies[i % len(copies)], q.BF16, None, 0, Wk, Wv, q.BF16,
                           None, None, b, L, r, heads, d, cs.softmax_scale, args.splits, O,
                           q.BF16, ws, ws_bytes)

    step_stats = {}
    ms = timed(step, args.steps, args.warmup, step_stats)
    # per-kernel times: a pass of the same steps with a launch-boundary event per kernel
    kern, kern_pass_ms = kernel_times(q, torch, step, args.steps)
    log(f"[bench] decode step {ms * 1e3:.1f} us (median {step_stats['median_ms'] * 1e3:.1f}); "
        f"kernel pass {kern_pass_ms * 1e3:.1f} us/step: " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kern.items()))

    # plain device copy of a known size: its FETCH_SIZE / WRITE_SIZE counters give the
    # factor that turns the counters of the decode kernels into HBM bytes
    # The same copies, timed, give the copy ceiling (bytes read + written per second) that
    # the HBM legs are also reported against.
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = timed(lambda i: dst.copy_(src), 3, 1)
    copy_gbps = 2 * COPY_BYTES / (copy_ms * 1e-3) / 1e9
    log(f"[bench] 1 GiB device copy: {copy_ms * 1e3:.0f} us = {copy_gbps:.0f} GB/s read + written")
    del src, dst

    stream_ms = kern.get("decode_stream", float("nan"))
    achieved = cache_bytes / (stream_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(COUNTERS):
        c = json.load(open(COUNTERS))
        if c.get("decode_hip_sha256_16") == kernel_source_hash():
            traffic = c.get("hbm_bytes_per_launch")

    # ------------------------------------------------------------------ tiny float32 latency leg
    tiny = None
    if not args.no_tiny:
        tiny = tiny_leg(q, torch, synth, dev, args)

    # ------------------------------------------------------------------ explicit K/V leg
    explicit = None
    if not args.no_explicit:
        E = heads * d
        Wk_t = torch.empty((E, r), dtype=torch.bfloat16, device="cuda")
        Wv_t = torch.empty((E, r), dtype=torch.bfloat16, device="cuda")
        q.qsvd_pack_weight(Wk, q.BF16, r, E, Wk_t)
        q.qsvd_pack_weight(Wv, q.BF16, r, E, Wv_t)
        rc, rs = (dev(t) for t in synth.rope_tables(L, d))
        Oe = torch.empty((b, heads, d), dtype=torch.bfloat16, device="cuda")
        ws_e = torch.empty(q.qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d),
                           dtype=torch.uint8, device="cuda")

        def step_e(i):
            q.qsvd_decode_attn_explicit(qv, q.BF16, copies[i % len(copies)], q.BF16, Wk_t, Wv_t,
                                        q.BF16, b, L, r, heads, d, cs.softmax_scale, rc, rs, Oe,
                                        q.BF16, ws_e)

        ms_e = timed(step_e, max(args.steps // 10, 3), max(1, args.warmup // 20))
        flops = 2.0 * b * L * r * 2 * E
        tf = flops / (ms_e * 1e-3) / 1e12
        explicit = {"workload": "same decode step with K_h = C W^u_k,h and V_h = C W^u_v,h rebuilt "
                                "explicitly on chip and RoPE on keys and query "
                                "(qsvd_decode_attn_explicit)",
                    "ms_per_step": round(ms_e, 4), "tokens_per_s": round(b / (ms_e * 1e-3), 1),
                    "roofline": {"bound": "mfma", "kernel": "explicit_attn", "achieved": round(tf, 1),
                                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flops": flops,
                                 "traffic": counted_traffic("explicit_hip_sha256_16", "explicit.hip",
                                                            ["explicit_attn_kernel<true>"])},
                    "latent_path_speedup": round(ms_e / ms, 2)}
        log(f"[bench] explicit K/V + RoPE decode: {ms_e * 1e3:.1f} us/step, {tf:.0f} TFLOP/s")
        del ws_e, Wk_t, Wv_t

    # ------------------------------------------------------------------ per-head latent leg
    headwise = None
    if not args.no_headwise:
        headwise = headwise_leg(q, torch, synth, dev, bf, b, L, heads, d, args)

    # ------------------------------------------------------------------ other decode configurations
    configs = None
    if not args.no_configs:
        del copies, C0
        configs = {"w8a4_int4_cache": w8a4_leg(q, torch, np, synth, dev, bf, args),
                   "llava13b_two_pass": llava13b_leg(q, torch, synth, bf, args)}

    # ------------------------------------------------------------------ prefill
    prefill = None
    if not args.no_prefill:
        M, E, rp = 4 * 4096, 4096, 1536
        t0 = time.time()
        X = synth.to_bf16_bits(synth.prefill_activations(M, E))
        Wd_q, Wd_s = synth.down_projection_int8(E, rp, 0.5, 0.5, 128, (100400,))
        log(f"[bench] generated prefill inputs in {time.time() - t0:.1f}s")
        Xd = bf(X)
        del X
        Wt = dev(np.ascontiguousarray(Wd_q.T))
        ws_d = dev(Wd_s)
        xq = torch.empty((M, E), dtype=torch.int8, device="cuda")
        xs = torch.empty((M,), dtype=torch.float32, device="cuda")
        Cp = torch.empty((M, rp), dtype=torch.float32, device="cuda")
        cq = torch.empty((M, rp), dtype=torch.int8, device="cuda")
        csc = torch.empty((M,), dtype=torch.float32, device="cuda")
        a1 = lambda i: q.qsvd_quantize_latent(Xd, q.BF16, M, E, 128, q.I8, 0, xq, xs)
        a2 = lambda i: q.qsvd_project(xq, q.I8, xs, M, E, Wt, q.I8, ws_d, rp, Cp, q.F32)
        a3 = lambda i: q.qsvd_quantize_latent(Cp, q.F32, M, rp, 128, q.I8, 0, cq, csc)
        steps = max(args.steps // 2, 5)
        t_a1 = timed(a1, steps, args.warmup)
        t_a2 = timed(a2, steps, args.warmup)
        t_a3 = timed(a3, steps, args.warmup)
        # W4A4: int4 X (a1 with int4 codes) x int4 W^d -> fp32
        Wd_q4 = np.clip(np.rint(Wd_q.astype(np.float64) / 18.0), -7, 7).astype(np.int8)  # timing-only codes
        W4 = torch.empty((rp, E // 2), dtype=torch.uint8, device="cuda")
        q.qsvd_pack_weight(dev(Wd_q4), q.I4, E, rp, W4)
        x4 = torch.empty((M, E // 2), dtype=torch.uint8, device="cuda")
        q.qsvd_quantize_latent(Xd, q.BF16, M, E, 128, q.I4, 0, x4, xs)
        a2_4 = lambda i: q.qsvd_project(x4, q.I4, xs, M, E, W4, q.I4, ws_d, rp, Cp, q.F32)
        t_a2_4 = timed(a2_4, steps, args.warmup)
        del W4, x4
        tops = 2.0 * M * E * rp / (t_a2 * 1e-3) / 1e12
        prefill = {"workload": "X[16384][4096] int8 x W^d[4096][1536] int8 -> fp32",
                   "proj_us": round(t_a2 * 1e3, 2), "proj_tops": round(tops, 1),
                   "peak_tops": INT8_PEAK_TOPS, "frac": round(tops / INT8_PEAK_TOPS, 4),
                   "roofline": {"bound": "mfma", "kernel": "gemm_i8", "achieved": round(tops, 1),
                                "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                                "frac": round(tops / INT8_PEAK_TOPS, 4), "ops": 2.0 * M * E * rp,
                                "traffic": counted_traffic("gemm_hip_sha256_16", "gemm.hip",
                                                           ["gemm_kernel<true, false, 256, 384,"])},
                   "w4a4_proj_us": round(t_a2_4 * 1e3, 2),
                   "w4a4_proj_tops": round(2.0 * M * E * rp / (t_a2_4 * 1e-3) / 1e12, 1),
                   "rotate_quant_x_us": round(t_a1 * 1e3, 2),
                   "rotate_quant_c_us": round(t_a3 * 1e3, 2)}
        log(f"[bench] prefill: a1 {t_a1 * 1e3:.1f} us, a2 {t_a2 * 1e3:.1f} us ({tops:.0f} TOPS), "
            f"a3 {t_a3 * 1e3:.1f} us; W4A4 a2 {t_a2_4 * 1e3:.1f} us")
        if not args.no_chain:
            prefill["chain"] = chain_leg(q, torch, np, synth, xq, xs, M, E, steps=3)
        del Xd, xq, Cp, cq

    # ------------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cs, O)

    for leg in [headwise] + (list(configs.values()) if configs else []):
        if leg and leg.get("roofline", {}).get("bound") == "hbm":
            leg["roofline"]["frac_of_copy_ceiling"] = round(leg["roofline"]["achieved"] / copy_gbps, 4)

    out = {
        "metric": "decode tokens/s + HBM GB/s (E=4096,r=1536,b=16,L=8192); prefill proj TOPS",
        "value": round(b / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "latent-attention decode step, E=4096 (32x128), r=1536, b=16, "
                               "L=8192, bf16 latent cache (LLaVA-v1.5-7B shape)",
                   "global_batch": b, "seq_len": L, "rank": r, "splits": splits,
                   "cache_copies": n_copies},
        "hbm_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_stats": step_stats,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
        "kernel_pass_us_per_step": round(kern_pass_ms * 1e3, 2),
        "environment": environment(),
        "roofline": {"bound": "hbm", "kernel": "decode_stream", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": cache_bytes,
                     "copy_ceiling_gbps": round(copy_gbps, 1),
                     "frac_of_copy_ceiling": round(achieved / copy_gbps, 4)},
        "cpu_baseline": cpu,
        "tiny_fp32": tiny,
        "prefill": prefill,
        "explicit": explicit,
        "headwise": headwise,
        "configs": configs,
    }
    print(json.dumps(out), flush=True)


def chain_leg(q, torch, np, synth, xq, xs, M, E, steps):
    """24 layers: projection to r_l, H2 rotate + int8 requantise, K/V rebuild (int8 GEMM to
    2E columns, bf16 out).  Timing-only weights: seeded int8 codes with unit scales."""
    ranks = synth.c4_ranks()
    g = np.random.default_rng(7)
    layers = []
    for rl in ranks:
        Wd = dev_t(torch, np, g.integers(-127, 128, size=(int(rl), E)).astype(np.int8))
        Wkv = dev_t(torch, np, g.integers(-127, 128, size=(2 * E, int(rl))).astype(np.int8))
        sd = torch.full((int(rl),), 1e-3, device="cuda")
        skv = torch.full((2 * E,), 1e-3, device="cuda")
        layers.append((int(rl), Wd, sd, Wkv, skv))
    rmax = int(max(ranks))
    Cp = torch.empty((M, rmax), dtype=torch.float32, device="cuda")
    cq = torch.empty((M, rmax), dtype=torch.int8, device="cuda")
    csc = torch.empty((M,), dtype=torch.float32, device="cuda")
    KV = torch.empty((M, 2 * E), dtype=torch.bfloat16, device="cuda")

    def run(_):
        for rl, Wd, sd, Wkv, skv in layers:
            q.qsvd_project(xq, q.I8, xs, M, E, Wd, q.I8, sd, rl, Cp, q.F32)
            q.qsvd_quantize_latent(Cp, q.F32, M, rl, 128, q.I8, 0, cq, csc)
            q.qsvd_project(cq, q.I8, csc, M, rl, Wkv, q.I8, skv, 2 * E, KV, q.BF16)

    ms = timed(run, steps, 1)
    ops = sum(2.0 * M * E * rl + 2.0 * M * rl * 2 * E for rl in ranks)
    tops = ops / (ms * 1e-3) / 1e12
    return {"layers": len(ranks), "ms": round(ms, 3), "tops": round(tops, 1),
            "roofline": {"bound": "mfma", "kernel": "gemm_i8 (both projections of each layer; the "
                                                    "rotate + requantise steps are inside the time)",
                         "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": round(tops / INT8_PEAK_TOPS, 4), "ops": ops}}


def headwise_leg(q, torch, synth, dev, bf, b, L, heads, d, args, rk=64, rv=64):
    """Per-head latents at the decode leg's shape: C [b][L][heads][rk + rv] bf16, RoPE
    tables for L positions; the step is qsvd_decode_attn_headwise (stream + merge)."""
    t0 = time.time()
    hc = synth.headwise_case(b, L, heads, d, rk, rv, seed=7)
    log(f"[bench] generated per-head latent inputs in {time.time() - t0:.1f}s")
    C0 = bf(hc.C)
    hc.C = None
    copies = [C0] + [C0.clone() for _ in range(copies_for(C0.numel() * 2, args.copies) - 1)]
    qv, BK, BV = bf(hc.q), bf(hc.BK_t), bf(hc.BV)
    rc, rs = (dev(t) for t in synth.rope_tables(L, d))
    O = torch.empty((b, heads, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.qsvd_decode_headwise_workspace_bytes(b, L, heads, d, rk, rv, 0),
                     dtype=torch.uint8, device="cuda")
    res = {}
    for name, tables in (("rope", (rc, rs)), ("plain", (None, None))):
        def step(i):
            q.qsvd_decode_attn_headwise(qv, q.BF16, copies[i % len(copies)], q.BF16, BK, BV, q.BF16,
                                        b, L, heads, d, rk, rv, hc.softmax_scale, tables[0],
                                        tables[1], 0, O, q.BF16, ws)
        n = max(args.steps // 2, 5)
        ms = timed(step, n, args.warmup)
        kern, _ = kernel_times(q, torch, step, n)
        res[name] = (ms, kern)
    cache_bytes = b * L * heads * (rk + rv) * 2
    ms, kern = res["rope"]
    stream_ms = kern.get("headwise_stream", float("nan"))
    achieved = cache_bytes / (stream_ms * 1e-3) / 1e9
    step_bytes = cache_bytes + heads * d * (rk + rv) * 2 + 2 * b * heads * d * 2
    traffic = counted_traffic("headwise_hip_sha256_16", "headwise.hip",
                              [f"headwise_stream_kernel<{rk // 32}, {rv // 32}, true>"])
    log(f"[bench] per-head latent decode (RoPE): {ms * 1e3:.1f} us/step; kernels (us): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kern.items()) +
        f"; without RoPE {res['plain'][0] * 1e3:.1f} us/step")
    del copies, C0
    return {"workload": f"per-head latents (WSVD form), 32 heads x 128, rk = rv = {rk}, b = {b}, "
                        f"L = {L}, bf16 cache, RoPE (qsvd_decode_attn_headwise)",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(b / (ms * 1e-3), 1),
            "hbm_gbps": round(step_bytes / (ms * 1e-3) / 1e9, 1),
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "no_rope_ms_per_step": round(res["plain"][0], 4),
            "roofline": {"bound": "hbm", "kernel": "headwise_stream", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                         "algorithmic_bytes": cache_bytes}}


def counted_traffic(hash_key, source, kernels):
    """HBM bytes per step of the given kernels from the committed counter passes (FETCH_SIZE and
    WRITE_SIZE, calibrated), or None when the counters were taken on another source state."""
    if not os.path.exists(COUNTERS):
        return None
    c = json.load(open(COUNTERS))
    if c.get(hash_key) != source_hash(source):
        return None
    other = c.get("other_kernels", {})
    total = 0
    for k in kernels:
        # a name ending in "<" or "," matches the instantiations it begins
        hits = [v for n, v in other.items() if n == k or (k[-1] in "<," and n.startswith(k))]
        if len(hits) != 1:
            return None
        total += hits[0]["hbm_read_bytes"] + hits[0]["hbm_write_bytes"]
    return total


def decode_timing(q, torch, step, args):
    """Step time (HIP events around the timed steps, with block statistics) and
    per-kernel launch times (a pass with launch-boundary events)."""
    n = max(args.steps // 2, 5)
    stats = {}
    ms = timed(step, n, args.warmup, stats)
    kern, pass_ms = kernel_times(q, torch, step, n)
    stats["kernel_pass_us_per_step"] = round(pass_ms * 1e3, 2)
    return ms, kern, stats


def w8a4_leg(q, torch, np, synth, dev, bf, args):
    """W8A4 decode shape: E = 4096 (32 x 128), r = 768, b = 16, L = 8192.  The cache is the
    rotated latent C' = C H2^T of the synthetic layer, written as int4 codes with group-128
    scales by qsvd_quantize_latent (the cache write); W^u' = H2 W^u as int8 columns."""
    cfg = synth.CONFIGS[2]
    b, L, r, heads, d = cfg.b, cfg.L, cfg.r, cfg.heads, cfg.d
    t0 = time.time()
    cs = synth.decode_case(cfg.E, heads, d, r, b, L, dtype="f32", p=cfg.p, beta=synth.config_beta(cfg),
                           outlier_frac=cfg.outlier_frac, outlier_gain=cfg.outlier_gain,
                           hadamard=cfg.hadamard, seed=1000 + cfg.idx)
    log(f"[bench] generated W8A4 decode inputs ({cfg.name}) in {time.time() - t0:.1f}s")
    M = b * L
    Cf = dev(cs.C.reshape(M, r))
    cache_bytes = b * L * (r // 2 + 4 * (r // 128))
    copies = []
    for _ in range(copies_for(cache_bytes, args.copies)):
        codes = torch.empty((M, r // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((M, r // 128), dtype=torch.float32, device="cuda")
        q.qsvd_quantize_latent(Cf, q.F32, M, r, 0, q.I4, 128, codes, scales)
        copies.append((codes, scales))
    del Cf
    Wk_q, Wk_s = synth.int8_columns(np.asarray(cs.Wu_k, np.float64))
    Wv_q, Wv_s = synth.int8_columns(np.asarray(cs.Wu_v, np.float64))
    Wk, Wv, wsk, wsv = dev(Wk_q), dev(Wv_q), dev(Wk_s), dev(Wv_s)
    qv = bf(synth.to_bf16_bits(cs.q))
    O = torch.empty((b, heads, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.qsvd_decode_workspace_bytes(b, L, r, heads, d, q.I4, 0), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        codes, scales = copies[i % len(copies)]
        q.qsvd_decode_attn(qv, q.BF16, codes, q.I4, scales, 128, Wk, Wv, q.I8, wsk, wsv, b, L, r,
                           heads, d, cs.softmax_scale, 0, O, q.BF16, ws)

    ms, kern, stats = decode_timing(q, torch, step, args)
    n_copies = len(copies)
    stream_ms = kern.get("decode_stream", float("nan"))
    achieved = cache_bytes / (stream_ms * 1e-3) / 1e9
    log(f"[bench] W8A4 decode: {ms * 1e3:.1f} us/step; kernels (us): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kern.items()))
    del copies
    return {"workload": f"decode step, {cfg.name}: int4 group-128 latent cache (codes + float32 "
                        "scales), int8 W^u with per-column scales",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(b / (ms * 1e-3), 1),
            "cache_copies": n_copies, "step_stats": stats,
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "roofline": {"bound": "hbm", "kernel": "decode_stream", "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": counted_traffic("decode_hip_sha256_16", "decode.hip",
                                                    ["stream_mfma_kernel<1, 2, 4, 64,"]),
                         "algorithmic_bytes": cache_bytes}}


def llava13b_leg(q, torch, synth, bf, args):
    """13B decode shape: E = 5120 (40 x 128), r = 2304, b = 8, L = 16384, bf16 cache.  The
    library runs it as two passes (scores, then values), each reading the cache once."""
    cfg = synth.CONFIGS[3]
    b, L, r, heads, d = cfg.b, cfg.L, cfg.r, cfg.heads, cfg.d
    t0 = time.time()
    cs = synth.config_decode_case(cfg)
    log(f"[bench] generated 13B decode inputs ({cfg.name}) in {time.time() - t0:.1f}s")
    C0 = bf(cs.C)
    cs.C = None
    copies = [C0] + [C0.clone() for _ in range(copies_for(C0.numel() * 2, args.copies) - 1)]
    qv, Wk, Wv = bf(cs.q), bf(cs.Wu_k), bf(cs.Wu_v)
    O = torch.empty((b, heads, d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(q.qsvd_decode_workspace_bytes(b, L, r, heads, d, q.BF16, 0), dtype=torch.uint8,
                     device="cuda")

    def step(i):
        q.qsvd_decode_attn(qv, q.BF16, copies[i % len(copies)], q.BF16, None, 0, Wk, Wv, q.BF16,
                           None, None, b, L, r, heads, d, cs.softmax_scale, 0, O, q.BF16, ws)

    ms, kern, stats = decode_timing(q, torch, step, args)
    n_copies = len(copies)
    cache_bytes = b * L * r * 2
    stream_ms = kern.get("decode_scores", float("nan")) + kern.get("decode_values", float("nan"))
    achieved = cache_bytes / (stream_ms * 1e-3) / 1e9
    moved = 2 * cache_bytes + 2 * b * heads * L * 4    # the cache twice, S written and read
    log(f"[bench] 13B decode: {ms * 1e3:.1f} us/step; kernels (us): " +
        ", ".join(f"{k} {v * 1e3:.1f}" for k, v in kern.items()))
    del copies, C0
    return {"workload": f"decode step, {cfg.name}: two-pass stream (decode_scores, decode_values)",
            "ms_per_step": round(ms, 4), "tokens_per_s": round(b / (ms * 1e-3), 1),
            "cache_copies": n_copies, "step_stats": stats,
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()},
            "pass_bytes_gbps": round(moved / (stream_ms * 1e-3) / 1e9, 1),
            "roofline": {"bound": "hbm", "kernel": "decode_scores + decode_values",
                         "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": counted_traffic("decode_wide_hip_sha256_16", "decode_wide.hip",
                                                    ["wide_scores_kernel<3, 9>", "wide_values_kernel<3>"]),
                         "algorithmic_bytes": cache_bytes}}


def tiny_leg(q, torch, synth, dev, args):
    """Config 0, the tiny float32 layer (E = 256, 4 heads x 64, r = 96, b = 1, L = 512): a
    latency figure.  Back-to-back steps give the device time per step; single calls each
    followed by a synchronisation give the latency a caller sees (host launch included)."""
    import numpy as np
    cs = synth.config_decode_case(synth.CONFIGS[0])
    qv, C, Wk, Wv = dev(cs.q), dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v)
    O = torch.empty((cs.b, cs.heads, cs.d), dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qsvd_decode_workspace_bytes(cs.b, cs.L, cs.r, cs.heads, cs.d, q.F32, 0),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        q.qsvd_decode_attn(qv, q.F32, C, q.F32, None, 0, Wk, Wv, q.F32, None, None, cs.b, cs.L,
                           cs.r, cs.heads, cs.d, cs.softmax_scale, 0, O, q.F32, ws)

    ms = timed(step, max(args.steps, 20), max(args.warmup, 20))
    kern, _ = kernel_times(q, torch, step, 20)
    lat = []
    for i in range(50):
        t0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    lat = np.array(lat) * 1e6
    log(f"[bench] tiny fp32 decode: {ms * 1e3:.1f} us/step back to back, {np.median(lat):.1f} us "
        "per synchronised call")
    cache_bytes = cs.b * cs.L * cs.r * 4
    gbs = cache_bytes / (ms * 1e-3) / 1e9
    return {"workload": f"decode step, {synth.CONFIGS[0].name}", "us_per_step": round(ms * 1e3, 2),
            "roofline": {"bound": "hbm", "kernel": "whole step (latency bound: one launch, "
                                                   "decode_f32_fused_kernel, over a 197 KB cache)",
                         "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 6), "algorithmic_bytes": cache_bytes},
            "kernels_note": "launch-boundary times of a host-bound loop: the gap until the next "
                            "step's first launch is counted in the last kernel",
            "latency_us": {"median": round(float(np.median(lat)), 1),
                           "p10": round(float(np.percentile(lat, 10)), 1),
                           "p90": round(float(np.percentile(lat, 90)), 1)},
            "kernels_us": {k: round(v * 1e3, 2) for k, v in kern.items()}}


def dev_t(torch, np, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def cpu_baseline(cs, O):
    """The float64 oracle (explicit K and V) on whole sequences of the same decode step, one
    sequence at a time, cycling over the batch until about 10 s of CPU work; the outputs of the
    first pass are also compared with the GPU's output of the timed step."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    v = oracle.bf16_decode
    Wk, Wv = v(cs.Wu_k), v(cs.Wu_v)
    got = O.float().cpu().numpy()
    n, t0, refs = 0, time.perf_counter(), []
    while True:
        s = n % cs.b
        o = oracle.attend_explicit(v(cs.q[s:s + 1]), v(cs.C[s:s + 1]), Wk, Wv, cs.heads, cs.d,
                                   cs.softmax_scale)
        if n < cs.b:
            refs.append(o)
        n += 1
        if time.perf_counter() - t0 > 10.0:
            break
    dt = time.perf_counter() - t0
    m = len(refs)
    err = oracle.rel_l2(got[:m], np.concatenate(refs))
    log(f"[bench] cpu oracle: {n} sequence steps in {dt:.1f}s on {threads} threads; "
        f"GPU vs oracle rel-L2 {err:.2e} over {m} sequences")
    return {"value": round(n / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} sequence steps ({m} distinct of {cs.b}; all {cs.heads} heads, explicit "
                      f"K/V in float64) in {dt:.1f} s",
            "gpu_vs_oracle_rel_l2": float(f"{err:.3e}")}


if __name__ == "__main__":
    main()
