#!/usr/bin/env python3
"""Benchmark: one GPU's share of ring (context-parallel) causal GQA attention,
fwd + bwd, on MI355X.

A step is one pass of the whole path over the share: P forward ring steps with
log-sum-exp merges (fused into the forward kernel's epilogue by default;
--merge separate runs lse_merge as its own kernel), the backward preprocess, and
P backward ring steps, on
seeded synthetic inputs already resident in HBM. The default workload is the
LLaMA-3-8B-shaped share at context degree 8 (32 Q / 8 KV heads, d = 128, bf16,
global sequence 131,072 tokens, local 16,384 rows as two paired blocks of 8,192).

    python bench.py [--steps K] [--warmup W] [--config NAME] [--no-cpu-baseline]

Prints ONE JSON line. ``value`` is algorithmic (causal-effective) fwd+bwd
TFLOP/s: 14 d Hq b(S+1) flops per step (4 d Hq N forward, 10 d Hq N backward,
N = b(S+1) visible pairs per head) over the timed wall time.
"""
import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sources_sha256():
    """Hash of the HIP sources (identifies the kernels a counter profile was taken on)."""
    import hashlib
    d = os.path.join(ROOT, "ring_attention_attn_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def recorded_traffic(cfg_name):
    """HBM bytes per ring_attn_step_bwd launch from the committed counter summary,
    or None when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if kernel_sources_sha256() not in text:
        return None
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch:"):
            return float(line.split(":")[1])
    return None


def make_inputs(cfg, rank, layout="zigzag"):
    import torch
    from ring_attention_attn_amd import synth
    P, b = cfg.P, cfg.b
    blocks_of = synth.paired_blocks if layout == "zigzag" else synth.contiguous_blocks
    mine = blocks_of(P, rank)

    def dev(bits):
        if cfg.dtype == "bf16":
            return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(bits).cuda()

    q = dev(synth.blocks_tensor(cfg.seed, synth.T_Q, mine, b, cfg.hq, cfg.d, cfg.dtype))
    do = dev(synth.blocks_tensor(cfg.seed, synth.T_DO, mine, b, cfg.hq, cfg.d, cfg.dtype))
    K, V = [], []
    for j in range(P):
        blocks = blocks_of(P, j)
        K.append(dev(synth.blocks_tensor(cfg.seed, synth.T_K, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
        V.append(dev(synth.blocks_tensor(cfg.seed, synth.T_V, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
    return q, torch.stack(K), torch.stack(V), do


def cpu_baseline(cfg, rank, budget_rows):
    """The fp64 oracle on a bounded sample of the same share: one KV head group
    (Hq/Hkv query heads) and ``budget_rows`` query rows spread evenly over both
    paired blocks, forward + backward over the whole sequence. Reported in the
    metric's unit: algorithmic flops of the sample / oracle wall time."""
    import oracle
    from ring_attention_attn_amd import synth
    P, b, G = cfg.P, cfg.b, cfg.hq // cfg.hkv
    rows = np.linspace(0, 2 * b - 1, budget_rows).round().astype(np.int64)
    pos = oracle.zigzag_positions(cfg.S, P, rank)[rows]
    mine = synth.paired_blocks(P, rank)
    q = synth.blocks_tensor(cfg.seed, synth.T_Q, mine, b, cfg.hq, cfg.d, cfg.dtype)[rows, :G]
    do = synth.blocks_tensor(cfg.seed, synth.T_DO, mine, b, cfg.hq, cfg.d, cfg.dtype)[rows, :G]
    k = synth.blocks_tensor(cfg.seed, synth.T_K, range(2 * P), b, cfg.hkv, cfg.d, cfg.dtype)[:, :1]
    v = synth.blocks_tensor(cfg.seed, synth.T_V, range(2 * P), b, cfg.hkv, cfg.d, cfg.dtype)[:, :1]
    w = (lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)) if cfg.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    q, do, k, v = w(q), w(do), w(k), w(v)
    t0 = time.perf_counter()
    oracle.share_backward(q, k, v, do, pos, cfg.scale)
    dt = time.perf_counter() - t0
    flops = 14 * cfg.d * G * int(np.sum(pos + 1))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": (f"numpy fp64 oracle, fwd+bwd over the whole sequence for {budget_rows} of "
                       f"{2 * b} query rows (evenly spaced over both paired blocks) x {G} query "
                       f"heads of one KV head; rank {rank}; cpu {platform.processor() or 'x86_64'}")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="llama3_8b_cp8_128k")
    ap.add_argument("--rank", type=int, default=0, help="ring rank whose share is timed")
    ap.add_argument("--cpu-rows", type=int, default=1536)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=("zigzag", "contiguous"), default="zigzag",
                    help="rows of the share: paired blocks (the method) or one contiguous "
                         "chunk per rank (to measure the causal imbalance, rank by rank)")
    ap.add_argument("--kv-rings", choices=("one", "ab"), default="one",
                    help="one launch per ring step, or two (one per block of the KV chunk: "
                         "the block A and block B rings)")
    ap.add_argument("--merge", choices=("fused", "separate"), default="fused",
                    help="fold each forward step into the running result in the forward "
                         "kernel (fused) or with a separate lse_merge launch")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one head_permute of 1 GiB (a plain copy of known size) before the "
                         "warmup, to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from ring_attention_attn_amd import binding
    from ring_attention_attn_amd.configs import CONFIGS
    from ring_attention_attn_amd.ring import ShareRing
    binding.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.config]
    log(f"config {cfg.name}: S={cfg.S} P={cfg.P} ({cfg.inner}x{cfg.outer}) hq={cfg.hq} "
        f"hkv={cfg.hkv} d={cfg.d} {cfg.dtype} rank={args.rank}")
    q, K, V, do = make_inputs(cfg, args.rank, args.layout)
    ring = ShareRing(cfg.S, cfg.inner, cfg.outer, args.rank, cfg.hq, cfg.hkv, cfg.d, cfg.dtype,
                     merge=args.merge, layout=args.layout, kv_rings=args.kv_rings)
    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(7)   # 1 GiB
        dst = torch.empty_like(src)
        binding.head_permute(src, dst, 1 << 17, 32, 128, 4, 2, 0)   # [131072][32][128] -> [4][...]
        torch.cuda.synchronize()
        del src, dst
        log("copy probe: head_permute of 1 GiB done")
    torch.cuda.synchronize()
    log("inputs resident; warmup")
    for _ in range(args.warmup):
        ring.step(q, K, V, do)
    torch.cuda.synchronize()
    log("timed region")

    # per-launch HIP events on the stream the kernels run on (torch's current stream)
    stream = torch.cuda.current_stream()
    ev = {"fwd": [], "bwd": [], "merge": []}
    from ring_attention_attn_amd import binding as B

    def timed_step():
        for t, (j, off, desc) in enumerate(ring.launches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            fused = t > 0 and args.merge == "fused"
            o, l = (ring.o_acc, ring.lse_acc) if t == 0 or fused else (ring.o_step, ring.lse_step)
            k, v = ring._kv(K, j, off), ring._kv(V, j, off)
            e0.record(stream)
            if fused:
                B.ring_attn_step_fwd_merge(desc, q, k, v, o, l)
            else:
                B.ring_attn_step_fwd(desc, q, k, v, o, l)
            e1.record(stream)
            ev["fwd"].append((e0, e1))
            if t > 0 and not fused:
                m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                m0.record(stream)
                B.lse_merge(ring.L, ring.hq, ring.d, ring.o_acc, ring.lse_acc, ring.o_step,
                            ring.lse_step)
                m1.record(stream)
                ev["merge"].append((m0, m1))
        B.ra_bwd_delta(ring.L, ring.hq, ring.d, B.RA_BF16 if cfg.dtype == "bf16" else B.RA_F32,
                       ring.o_acc, do, ring.delta, ring.o_lowp if cfg.dtype == "bf16" else None)
        B.ra_fill_f32(ring.dq, ring.dq.numel(), 0.0)
        for j, off, desc in ring.launches:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            B.ring_attn_step_bwd(desc, q, ring._kv(K, j, off), ring._kv(V, j, off), do,
                                 ring.lse_acc, ring.delta, ring.dq, ring._kv(ring.dk, j, off),
                                 ring._kv(ring.dv, j, off))
            e1.record(stream)
            ev["bwd"].append((e0, e1))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        timed_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    fwd_flops, bwd_flops = cfg.flops(args.layout, args.rank)
    total = fwd_flops + bwd_flops
    ms = wall / args.steps * 1e3
    value = total * args.steps / wall / 1e12

    def avg_ms(pairs):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) if pairs else 0.0

    if args.merge == "fused":
        # the merge runs inside the forward launches; time the standalone kernel
        # (outside the timed steps) for its own bandwidth figure
        ring.o_step.zero_()
        ring.lse_step.zero_()
        for _ in range(6):
            m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            m0.record(stream)
            B.lse_merge(ring.L, ring.hq, ring.d, ring.o_acc, ring.lse_acc, ring.o_step,
                        ring.lse_step)
            m1.record(stream)
            ev["merge"].append((m0, m1))
        torch.cuda.synchronize()
        ev["merge"] = ev["merge"][1:]
    fwd_ms, bwd_ms, merge_ms = avg_ms(ev["fwd"]), avg_ms(ev["bwd"]), avg_ms(ev["merge"])
    # algorithmic flops per launch: each ring step carries 1/P of the share's pairs
    # (2b^2 per head per step, +b on the diagonal step); averaged over the P launches
    n_launch = len(ring.launches)   # P, or 2P with the block A / block B rings
    bwd_launch_flops = bwd_flops / n_launch
    fwd_launch_flops = fwd_flops / n_launch
    bwd_tflops = bwd_launch_flops / (bwd_ms * 1e-3) / 1e12
    fwd_tflops = fwd_launch_flops / (fwd_ms * 1e-3) / 1e12
    merge_bytes = cfg.rows * cfg.hq * (cfg.d * 4 * 3 + 4 * 3)
    out = {
        "metric": "ring-attention fwd+bwd TFLOP/s (causal-effective) and % bf16 MFMA peak, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1), rounded to bf16)",
        "config": {"workload": cfg.name, "global_seq": cfg.S, "ring": f"{cfg.inner}x{cfg.outer}",
                   "local_rows": cfg.rows, "hq": cfg.hq, "hkv": cfg.hkv, "head_dim": cfg.d,
                   "rank": args.rank, "layout": args.layout, "kv_rings": args.kv_rings,
                   "parallelism": "one GPU's share (virtual ring)"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "merge": args.merge,
        "breakdown_ms_per_launch": {"step_fwd": round(fwd_ms, 4), "step_bwd": round(bwd_ms, 4),
                                    "lse_merge": round(merge_ms, 4)},
        "step_fwd_tflops": round(fwd_tflops, 1),
        "lse_merge_gbs": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1) if merge_ms else None,
        "roofline": {"bound": "mfma", "kernel": "ring_attn_step_bwd", "achieved": round(bwd_tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(cfg.name)},
    }
    if args.layout != "zigzag":
        log("cpu baseline is taken on the paired-block share only; skipped")
    elif not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.rank, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
