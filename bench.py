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
PEAK_F32_VECTOR_TFLOPS = 157.3   # MI355X fp32 vector (published)


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


def recorded_mfma_util(cfg_name):
    """MFMA-busy share of each step kernel's cycles from the committed counter
    summary (SQ_VALU_MFMA_BUSY_CYCLES over 4 SIMDs x 256 CUs x the kernel's
    cycles), or None when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"mfma_lds_counters_{cfg_name}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    if kernel_sources_sha256() not in text:
        return None
    for line in text.splitlines():
        if line.startswith("mfma_busy_pct:"):
            return json.loads(line.split(":", 1)[1])
    return None


def _dev(cfg, bits):
    import torch
    if cfg.dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(bits).cuda()


def make_head_parallel_inputs(cfg, rank):
    """The 2D-Attention share's inputs with every head: Q and dO of the rank's
    rows [L][H][d], its own K/V chunk [L][Hkv][d], and the other chunks in head
    group 0 layout [L][Hkv/hp][d] (as the ring would deliver them)."""
    from ring_attention_attn_amd import synth
    P, b, hp = cfg.P, cfg.b, cfg.hp
    H, Hkv = cfg.hq * hp, cfg.hkv * hp
    mine = synth.paired_blocks(P, rank)
    dev = lambda x: _dev(cfg, x)
    q = dev(synth.blocks_tensor(cfg.seed, synth.T_Q, mine, b, H, cfg.d, cfg.dtype))
    do = dev(synth.blocks_tensor(cfg.seed, synth.T_DO, mine, b, H, cfg.d, cfg.dtype))
    k_own = dev(synth.blocks_tensor(cfg.seed, synth.T_K, mine, b, Hkv, cfg.d, cfg.dtype))
    v_own = dev(synth.blocks_tensor(cfg.seed, synth.T_V, mine, b, Hkv, cfg.d, cfg.dtype))
    k_rest, v_rest = [], []
    for j in range(P):
        blocks = synth.paired_blocks(P, j)
        k_rest.append(None if j == rank else dev(synth.blocks_tensor(
            cfg.seed, synth.T_K, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
        v_rest.append(None if j == rank else dev(synth.blocks_tensor(
            cfg.seed, synth.T_V, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
    return q, k_own, v_own, k_rest, v_rest, do


def make_inputs(cfg, rank, layout="zigzag"):
    import torch
    from ring_attention_attn_amd import synth
    P, b = cfg.P, cfg.b
    blocks_of = synth.paired_blocks if layout == "zigzag" else synth.contiguous_blocks
    mine = blocks_of(P, rank)
    dev = lambda x: _dev(cfg, x)

    q = dev(synth.blocks_tensor(cfg.seed, synth.T_Q, mine, b, cfg.hq, cfg.d, cfg.dtype))
    do = dev(synth.blocks_tensor(cfg.seed, synth.T_DO, mine, b, cfg.hq, cfg.d, cfg.dtype))
    K, V = [], []
    for j in range(P):
        blocks = blocks_of(P, j)
        K.append(dev(synth.blocks_tensor(cfg.seed, synth.T_K, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
        V.append(dev(synth.blocks_tensor(cfg.seed, synth.T_V, blocks, b, cfg.hkv, cfg.d, cfg.dtype)))
    return q, torch.stack(K), torch.stack(V), do


def cpu_info():
    """CPU model (from /proc/cpuinfo) and the BLAS numpy uses."""
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:
        pass
    return model, blas


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
    q = synth.blocks_tensor(cfg.seed, synth.T_Q, mine, b, G, cfg.d, cfg.dtype)[rows]
    do = synth.blocks_tensor(cfg.seed, synth.T_DO, mine, b, G, cfg.d, cfg.dtype)[rows]
    k = synth.blocks_tensor(cfg.seed, synth.T_K, range(2 * P), b, 1, cfg.d, cfg.dtype)
    v = synth.blocks_tensor(cfg.seed, synth.T_V, range(2 * P), b, 1, cfg.d, cfg.dtype)
    w = (lambda a: synth.bf16_bits_to_f32(a).astype(np.float64)) if cfg.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    q, do, k, v = w(q), w(do), w(k), w(v)
    t0 = time.perf_counter()
    oracle.share_backward(q, k, v, do, pos, cfg.scale)
    dt = time.perf_counter() - t0
    flops = 14 * cfg.d * G * int(np.sum(pos + 1))
    model, blas = cpu_info()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle", "seconds": round(dt, 3), "cpu": model, "blas": blas,
            "sample": (f"numpy fp64 oracle, fwd+bwd over the whole sequence for {budget_rows} of "
                       f"{2 * b} query rows (evenly spaced over both paired blocks) x {G} query "
                       f"heads of one KV head; rank {rank}; BLAS threads = the cores available "
                       f"({len(os.sched_getaffinity(0))})")}


class EventTimer:
    """HIP events around each library launch, on the stream the launches use."""

    def __init__(self, stream):
        import collections
        self.stream = stream
        self.ev = collections.defaultdict(list)

    def __call__(self, kind):
        import contextlib
        import torch

        @contextlib.contextmanager
        def cm():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            yield
            e1.record(self.stream)
            self.ev[kind].append((e0, e1))
        return cm()

    def avg_ms(self, kind):
        pairs = self.ev.get(kind, [])
        return float(np.mean([a.elapsed_time(b) for a, b in pairs])) if pairs else 0.0

    def total_ms(self, kind):
        return float(np.sum([a.elapsed_time(b) for a, b in self.ev.get(kind, [])]))


def gemm_reference(m=16384, n=16384, k=8192, reps=20):
    """Rate of one large bf16 GEMM by the vendor library (torch.matmul ->
    hipBLASLt) on this GPU, measured after the timed region: what a plain dense
    contraction sustains here, a practical reference beside the nominal peak."""
    import torch
    a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"value": round(2.0 * m * n * k / (ms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
            "what": f"torch.matmul bf16 {m}x{n}x{k} (vendor GEMM), sustained on this GPU"}


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
    ap.add_argument("--merge", choices=("fused", "separate", "chunks"), default="fused",
                    help="fold each forward step into the running result in the forward "
                         "kernel (fused) or with a separate lse_merge launch")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the vendor-GEMM reference rate measured after the timed region")
    ap.add_argument("--gemm-ref-only", action="store_true",
                    help="print only the vendor-GEMM reference rate (for counter runs of it)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run one head_permute of 1 GiB (a plain copy of known size) before the "
                         "warmup, to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share on one GPU; --gpus {args.gpus} is not supported "
              "(the library has no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.gemm_ref_only:
        print(json.dumps({"gemm_ref": gemm_reference()}), flush=True)
        return
    from ring_attention_attn_amd import binding
    from ring_attention_attn_amd.configs import CONFIGS
    from ring_attention_attn_amd.ring import HeadParallelShare, ShareRing
    binding.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.config]
    wrapped = bool(cfg.permute_heads) and args.layout == "zigzag"
    log(f"config {cfg.name}: S={cfg.S} P={cfg.P} ({cfg.inner}x{cfg.outer}) hq={cfg.hq} "
        f"hkv={cfg.hkv} d={cfg.d} {cfg.dtype} rank={args.rank}"
        + (f" head-parallel {cfg.hp} (head permutes in the step)" if wrapped else ""))
    ring_kw = dict(merge=args.merge, layout=args.layout, kv_rings=args.kv_rings)
    if wrapped:
        inputs = make_head_parallel_inputs(cfg, args.rank)
        share = HeadParallelShare(cfg.S, cfg.inner, cfg.outer, args.rank, cfg.hq * cfg.hp,
                                  cfg.hkv * cfg.hp, cfg.d, cfg.hp, group=0, dtype=cfg.dtype,
                                  **ring_kw)
        ring = share.ring
    else:
        inputs = make_inputs(cfg, args.rank, args.layout)
        share = ring = ShareRing(cfg.S, cfg.inner, cfg.outer, args.rank, cfg.hq, cfg.hkv, cfg.d,
                                 cfg.dtype, **ring_kw)
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
        share.step(*inputs)
    torch.cuda.synchronize()
    log("timed region")

    # per-launch HIP events on the stream the kernels run on (torch's current stream)
    stream = torch.cuda.current_stream()
    timer = EventTimer(stream)
    share.timer = timer
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        share.step(*inputs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    share.timer = None
    log(f"timed {args.steps} steps in {wall:.3f} s")

    fwd_flops, bwd_flops = cfg.flops(args.layout, args.rank)
    total = fwd_flops + bwd_flops
    ms = wall / args.steps * 1e3
    value = total * args.steps / wall / 1e12

    from ring_attention_attn_amd import binding as B
    if args.merge in ("fused", "chunks"):
        # the merge runs inside the forward launches; time the standalone kernel
        # (outside the timed steps, over all rows) for its own bandwidth figure
        ring.o_step.zero_()
        ring.lse_step.zero_()
        mt = EventTimer(stream)
        for _ in range(6):
            with mt("lse_merge"):
                B.lse_merge(ring.L, ring.hq, ring.d, ring.o_acc, ring.lse_acc, ring.o_step,
                            ring.lse_step)
        torch.cuda.synchronize()
        merge_ms = float(np.mean([a.elapsed_time(b) for a, b in mt.ev["lse_merge"][1:]]))
        merge_rows = ring.L
    else:
        merge_ms = timer.avg_ms("lse_merge")
        n_m = len(ring.launches) - 1
        merge_rows = sum(ring.merge_rows(desc)[1] for _, _, desc in ring.launches[1:]) / max(n_m, 1)
    fwd_ms, bwd_ms = timer.avg_ms("step_fwd"), timer.avg_ms("step_bwd")
    delta_ms = timer.avg_ms("bwd_delta")
    # algorithmic flops per launch: each ring step carries 1/P of the share's pairs
    # (2b^2 per head per step, +b on the diagonal step); averaged over the P launches
    n_launch = len(ring.launches)   # P, or 2P with the block A / block B rings
    # with --merge chunks the backward is one call over all steps
    chunks = args.merge == "chunks"
    roof_peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_VECTOR_TFLOPS
    bwd_launch_flops = bwd_flops if chunks else bwd_flops / n_launch
    # with --merge chunks the forward is one launch over all steps
    fwd_launch_flops = fwd_flops if chunks else fwd_flops / n_launch
    bwd_tflops = bwd_launch_flops / (bwd_ms * 1e-3) / 1e12
    fwd_tflops = fwd_launch_flops / (fwd_ms * 1e-3) / 1e12
    merge_bytes = merge_rows * cfg.hq * (cfg.d * 4 * 3 + 4 * 3)
    # D = rowsum(dO O): reads O (fp32) and dO, writes O in bf16 and D
    eb = 2 if cfg.dtype == "bf16" else 4
    delta_bytes = ring.L * cfg.hq * (cfg.d * (4 + eb + (2 if cfg.dtype == "bf16" else 0)) + 4)
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
                   "head_parallel": cfg.hp, "head_permutes_in_step": wrapped,
                   "parallelism": "one GPU's share (virtual ring)"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "merge": args.merge,
        "breakdown_ms_per_launch": {"step_fwd": round(fwd_ms, 4), "step_bwd": round(bwd_ms, 4),
                                    "lse_merge": round(merge_ms, 4),
                                    "bwd_delta": round(delta_ms, 4)},
        "step_fwd_tflops": round(fwd_tflops, 1),
        "step_bwd_tflops": round(bwd_tflops, 1),
        # the same step counted without the backward's QK^T recompute (12 d per
        # visible pair instead of 14 d), so the headline cannot be read as inflated
        "value_without_recompute": round(value * 12 / 14, 2),
        "lse_merge_gbs": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1) if merge_ms else None,
        "bwd_delta_gbs": round(delta_bytes / (delta_ms * 1e-3) / 1e9, 1) if delta_ms else None,
        # with --merge chunks the dominant call is ring_attn_bwd_chunks (its dQ
        # launch and its dK/dV launch over all chunks); the recorded counters are
        # the per-step kernels', so they are not quoted for it. The fp32
        # workload runs plain fp32 vector kernels: bounded by the fp32 vector
        # peak, not the matrix cores.
        "roofline": {"bound": "mfma" if cfg.dtype == "bf16" else "alu",
                     "kernel": "ring_attn_bwd_chunks" if chunks else "ring_attn_step_bwd",
                     "achieved": round(bwd_tflops, 1),
                     "peak": roof_peak, "unit": "TFLOP/s",
                     "frac": round(bwd_tflops / roof_peak, 4),
                     "traffic": None if chunks else recorded_traffic(cfg.name)},
    }
    util = None if chunks else recorded_mfma_util(cfg.name)
    if util is not None:
        out["mfma_busy_pct"] = util
    if wrapped:
        perm_ms = timer.total_ms("head_permute") / args.steps
        out["breakdown_ms_per_step"] = {"head_permutes": round(perm_ms, 4)}
        out["head_permute_gbs"] = round(share.permute_bytes() / (perm_ms * 1e-3) / 1e9, 1)
    if not args.no_gemm_ref:
        out["gemm_ref"] = gemm_reference()
    if args.layout != "zigzag":
        log("cpu baseline is taken on the paired-block share only; skipped")
    elif not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.rank, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
