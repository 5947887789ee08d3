"""Benchmark: Medusa decode steps on one MI355X.

One step = the whole hot path on one batch of synthetic input: heads (residual SiLU
block, vocabulary projections, per-head top-k) -> tree fill -> verifier Q/K/V ->
tree-masked attention -> verifier output -> lm_head verification + acceptance.
Inputs are resident in HBM before timing starts.  Prints one JSON line on stdout.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config 8b]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 MFMA, MI355X (vendor)
DOMINANT = "heads_vocab"        # the kernel with most of the step's bytes (A2+A3)
# HBM bytes of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, valid while
# the sources it was measured on are unchanged (their hash is recorded beside the figure)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "heads_vocab_8b_traffic.md")
KERNEL_SOURCES = ("speculative_decoding_amd/csrc/gemm.hip", "speculative_decoding_amd/csrc/common.hpp",
                  "speculative_decoding_amd/csrc/internal.hpp", "speculative_decoding_amd/build.py")
METRIC = "Medusa verify steps/s + tokens/s and achieved HBM GB/s at 8B shape, 1 GPU"

WORKLOADS = {
    "8b": "Medusa decode step, 8B-class shape: hidden 4096, vocab 128256, 4 heads with "
          "top-(10,5,4,3), 64-node sparse tree, one-layer verifier with GQA 32 q / 8 kv heads "
          "of dim 128, KV prefix 4096, batch 1",
    "mid": "Medusa decode step, 7B-class shape: hidden 4096, vocab 32000, 5 heads with "
           "top-(10,5,4,3,2), 64-node sparse tree, 32 heads of dim 128, KV prefix 1024, batch 1",
    "dense": "Medusa decode step, 8B-class shape with the dense 256-node tree "
             "(1+3+12+48+192), KV prefix 8192, batch 1",
    "batched70b": "Medusa decode step, 70B-class shape: hidden 8192, vocab 32000, 5 heads, "
                  "64-node sparse tree per sequence, GQA 64/8 x 128, batch 8, prefixes U[512,8192]",
    "tiny": "Medusa decode step, worked-example shape: hidden 256, vocab 1000, 3 heads, fp32",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, n_nodes: int, prefix_total: int) -> dict:
    """Bytes the method must move per step: every weight once, the valid KV rows, the
    gathered embedding rows (read for Q/K/V and again for the residual)."""
    es = 2 if cfg.dtype == "bf16" else 4
    H, V, K = cfg.H, cfg.V, cfg.K
    qd, kvd = cfg.Hq * cfg.d, cfg.Hkv * cfg.d
    parts = {
        "heads_ffn": K * H * H * es + K * H * es,
        "heads_vocab": K * V * H * es,
        "proxy_qkv": (qd + 2 * kvd) * H * es + cfg.B * n_nodes * H * es,
        "attention": prefix_total * 2 * kvd * es,
        "proxy_out": H * qd * es + cfg.B * n_nodes * H * es,
        "verify_lmhead": V * H * es,
    }
    parts["total"] = sum(parts.values())
    return parts


def decode_loop_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, rounds: int):
    """Rounds of the whole step plus medusa_advance, timed end to end on a copy of the
    inputs whose KV cache has room for every round (the same weights; the cache rows past
    the prefix start as zeros and fill with the accepted branches).  Emitted tokens per
    second count every accepted candidate and bonus token."""
    if rounds <= 0:
        return None
    import dataclasses
    Lcap = cfg.Lcap + rounds * (plan.max_depth + 1)
    dims = dataclasses.replace(Dims.from_config(cfg), Lcap=Lcap)

    def fresh():
        w2 = dict(w)
        for name in ("k_cache", "v_cache"):
            t = torch.zeros((cfg.B, Lcap) + tuple(w[name].shape[2:]), dtype=w[name].dtype, device=dev)
            t[:, : cfg.Lcap] = w[name]
            w2[name] = t
        w2["prefix_lens"] = w["prefix_lens"].clone()
        w2["h"] = w["h"].clone()
        return MedusaStep(dims, w2, plan, dev)

    fresh().decode(2)                       # warm-up on a throwaway state
    st = fresh()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, lens, toks, over = st.decode(rounds)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    streams = st.streams(lens, toks)
    tokens = int(sum(len(x) for x in streams))
    return {"rounds": rounds, "emitted_tokens": tokens, "seconds": sec,
            "rounds_per_s": rounds / sec, "tokens_per_s": tokens / sec,
            "mean_accept_len": float(lens.float().mean().item()),
            "overflow": int(over.max().item()),
            "note": "heads are random apart from the planted first round, so later rounds "
                    "mostly accept nothing; every round still emits its bonus token"}


# dense trees for four heads: the full product of top-(3,4,4,4), 1+3+12+48+192 = 256 nodes,
# and of top-(4,4,4,4), whose 4^4 = 256 leaf paths make 341 nodes
SWEEP_DENSE = {4: ((3, 4, 4, 4), (4, 4, 4, 4))}
SWEEP_NODES = "1,16,32,64,128,256,341"


def node_sweep(torch, M, MedusaStep, Dims, cfg, w, dev, seed: int, node_counts, steps: int,
               warmup: int):
    """Whole-step time t(N) for sparse trees of N nodes (the most accurate combinations)
    and for the dense Cartesian trees, on the workload's weights and KV prefix.  E[a](N)
    comes from the synthetic accuracy table drawn over the union of the trees' ranks; the
    predicted rate is (1 + E[a]) / t(N) per sequence."""
    import dataclasses
    import numpy as np
    from speculative_decoding_amd import budget
    from synth.gen import accuracy_table
    dense = SWEEP_DENSE.get(cfg.K, ())
    s = tuple(max([a] + [ds[k] for ds in dense]) for k, a in enumerate(cfg.s))
    scfg = dataclasses.replace(cfg, s=s, tree_s=s)
    acc = accuracy_table(scfg, seed)
    dims = Dims.from_config(scfg)
    n_cands = sum(int(np.prod(s[:d])) for d in range(1, len(s) + 1))
    counts = [n for n in node_counts if 1 <= n <= min(n_cands + 1, M.MEDUSA_MAX_NODES)]

    def timed(plan):
        plan.upload(dev)
        st = MedusaStep(dims, w, plan, dev)
        st.heads(bootstrap_root=True)
        for _ in range(warmup):
            st.run(bootstrap_root=False, keep_u=False)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.run(bootstrap_root=False, keep_u=False)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    pts = budget.curve(acc, s, counts, step_seconds=timed, dense=dense)
    top = budget.best(pts)
    sparse = {p.nodes: p for p in pts if p.kind == "sparse"}
    dense256 = next((p for p in pts if p.kind == "dense" and p.nodes == 256), None)
    out = {"tree_s": list(s), "steps_per_point": steps,
           "accuracy": "synthetic per-head rank accuracies 0.8*0.8^k*0.6*0.4^r*U(0.9,1.1), "
                       "heads independent; E[a] is the closed form, not a measured rate",
           "points": [p.as_dict() for p in pts],
           "best": top.as_dict()}
    if dense256 is not None and 64 in sparse:
        out["sparse64_vs_dense"] = sparse[64].tokens_per_s / dense256.tokens_per_s
    return out


TYPICAL = (1.0, 0.09, 0.3)          # temperature, epsilon, delta: values chosen here


def typical_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, steps: int, warmup: int):
    """Whole steps with typical acceptance (medusa_verify_accept_typical) in place of greedy
    acceptance, on the same inputs and plan, then a pass with every launch event-timed for
    the two verification kernels."""
    st = MedusaStep(Dims.from_config(cfg), w, plan, dev, typical=TYPICAL)
    st.heads(bootstrap_root=True)
    for _ in range(warmup):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    M.medusa_profile_reset()
    M.medusa_profile_only(None)
    M.medusa_profile_enable(True)
    for _ in range(steps):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    M.medusa_profile_enable(False)
    out = {"temperature": TYPICAL[0], "epsilon": TYPICAL[1], "delta": TYPICAL[2],
           "steps": steps, "ms_per_step": 1e3 * sec, "steps_per_s": 1.0 / sec,
           "accept_len": [int(x) for x in st.accept_len.cpu()]}
    for name in ("verify_lmhead", "verify_accept"):
        ms, n = M.medusa_profile_query(name)
        if n:
            out[name + "_us"] = 1e3 * ms / n
    return out


ROPE_BASE = 10000.0


def rope_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, steps: int, warmup: int):
    """Whole steps with rotary positions on the verifier's q and k (medusa_rope after the
    projections), on the same inputs and plan; then a pass with the rotation event-timed."""
    import dataclasses
    st = MedusaStep(dataclasses.replace(Dims.from_config(cfg), rope_base=ROPE_BASE), w, plan, dev)
    st.heads(bootstrap_root=True)
    for _ in range(warmup):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    M.medusa_profile_reset()
    M.medusa_profile_only("rope")
    M.medusa_profile_enable(True)
    for _ in range(steps):
        st.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    M.medusa_profile_enable(False)
    ms, n = M.medusa_profile_query("rope")
    return {"base": ROPE_BASE, "steps": steps, "ms_per_step": 1e3 * sec, "steps_per_s": 1.0 / sec,
            "rope_us": 1e3 * ms / n if n else None}


def clock_probe(torch, M, reps: int = 3):
    """Shader clock under MFMA load on every SIMD (medusa_clock_probe): shader-clock ticks
    over 100 MHz ticks of one workgroup's run; the median of `reps` runs, in MHz."""
    ticks = torch.zeros(2, dtype=torch.int64, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    vals = []
    for _ in range(reps + 1):
        M.medusa_clock_probe(ticks, sink)
        torch.cuda.synchronize()
        t = ticks.cpu().tolist()
        if t[1] > 0:
            vals.append(100.0 * t[0] / t[1])
    vals = vals[1:] or vals
    return sorted(vals)[len(vals) // 2] if vals else None


def hbm_probe(torch, M, buf, reps: int = 10):
    """Read ceiling of this GPU: medusa_hbm_read_probe streaming `buf` (the heads' weights)
    `reps` times, timed with events on the current stream."""
    sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    nbytes = M.medusa_hbm_probe_bytes(buf.numel() * buf.element_size())
    M.medusa_hbm_read_probe(buf, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        M.medusa_hbm_read_probe(buf, sink)
    b.record()
    torch.cuda.synchronize()
    sec = a.elapsed_time(b) * 1e-3 / reps
    return {"gbps": nbytes / sec / 1e9, "bytes_per_launch": nbytes, "launches": reps,
            "avg_us": sec * 1e6}


def step_percentiles(torch, step, steps: int):
    """Per-step durations from events around each step (a pass of its own)."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        step.run(bootstrap_root=False, keep_u=False)
        b.record()
    torch.cuda.synchronize()
    us = np.array([1e3 * a.elapsed_time(b) for a, b in ev])
    return {"median": float(np.median(us)), "p10": float(np.percentile(us, 10)),
            "p90": float(np.percentile(us, 90)), "steps": steps}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(config_name: str):
    """Bytes per launch of the dominant kernel from the committed counter summary, or None
    when there is none for this workload or the kernel sources changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, re.M))
    if fields.get("workload") != config_name or fields.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_info():
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def cpu_baseline(inp, oplan, reps: int = 3) -> dict:
    """The oracle, as it stands, on whole steps of the same workload (host cores): one
    warm-up step, then the median of `reps` timed steps."""
    import statistics
    import oracle
    res = oracle.step(inp, oplan)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.step(inp, oplan)
        times.append(time.perf_counter() - t0)
    dt = statistics.median(times)
    cores, model = cpu_info()
    return {"value": 1.0 / dt, "unit": "steps/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"whole steps (all parts) of the same workload and seed, fp64 numpy: "
                      f"one warm-up, median of {reps} ({dt:.1f} s each); host {model}, "
                      f"{cores} cores visible",
            "seconds_per_step": dt, "accept_len": [int(a) for a in res.accept_len]}


def attention_only(args) -> int:
    """medusa_tree_attention alone at one workload's shapes: its plan, heads, head dim,
    prefix lengths and cache capacity, on seeded random bf16 inputs.  Both launches are
    event-timed by the library's profiler over `--attention-calls` calls after five
    warm-up calls."""
    import torch

    from speculative_decoding_amd import medusa as M
    from synth import get_config
    from synth.gen import _prefix_lens, accuracy_table

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    plan = (M.medusa_tree_plan_full(cfg.tree_s) if cfg.tree == "full" else
            M.medusa_tree_plan_from_accuracy(accuracy_table(cfg, args.seed), cfg.tree_s, cfg.n_nodes))
    plan.upload(dev)
    B, N, Hq, Hkv, d, Lcap = cfg.B, plan.n_nodes, cfg.Hq, cfg.Hkv, cfg.d, cfg.Lcap
    lens = [int(x) for x in _prefix_lens(cfg, args.seed)]
    g = torch.Generator(device=dev).manual_seed(args.seed)
    mk = lambda *shape: torch.randn(*shape, device=dev, generator=g).to(torch.bfloat16)
    q, kt, vt = mk(B, N, Hq, d), mk(B, N, Hkv, d), mk(B, N, Hkv, d)
    kc, vc = mk(B, Lcap, Hkv, d), mk(B, Lcap, Hkv, d)
    L = torch.as_tensor(lens, device=dev, dtype=torch.int32)
    out = torch.empty(B, N, Hq, d, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.medusa_attention_workspace(plan, "bf16", B, Hq, Hkv, d, Lcap),
                     dtype=torch.uint8, device=dev)

    def call():
        M.medusa_tree_attention(plan, "bf16", B, Hq, Hkv, d, Lcap, 0.0, q, kt, vt, kc, vc, L, out, ws)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    M.medusa_profile_reset()
    M.medusa_profile_enable(True)
    for _ in range(args.attention_calls):
        call()
    torch.cuda.synchronize()
    M.medusa_profile_enable(False)
    tile_ms, tile_n = M.medusa_profile_query("attn_partial")
    merge_ms, merge_n = M.medusa_profile_query("attn_combine")
    tile_us, merge_us = 1e3 * tile_ms / tile_n, 1e3 * merge_ms / merge_n
    keys = sum(min(x, Lcap) for x in lens) + B * N
    flop = 4.0 * N * Hq * d * keys                     # scores and value sums, every (row, key)
    kv_bytes = 2 * 2 * d * Hkv * sum(min(x, Lcap) for x in lens)
    print(json.dumps({
        "metric": "tree attention alone (medusa_tree_attention)", "config": args.config,
        "library": os.path.relpath(_lib_path(), ROOT), "B": B, "nodes": N, "Hq": Hq, "Hkv": Hkv, "d": d,
        "prefix": lens, "calls": args.attention_calls, "tile_us": tile_us, "merge_us": merge_us,
        "gflop": flop / 1e9, "tflops": flop / (tile_us + merge_us) / 1e6,
        "mfma_frac": flop / (tile_us + merge_us) / 1e6 / MFMA_PEAK_TFLOPS,
        "kv_bytes": kv_bytes, "workspace_bytes": ws.numel()}))
    return 0


def _lib_path() -> str:
    from speculative_decoding_amd import _lib
    return _lib.LIB_PATH


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="8b", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--loop-rounds", type=int, default=32,
                    help="also time this many rounds of the decode loop (step + advance) on a "
                         "copy of the inputs whose KV cache has room for them (0: skip)")
    ap.add_argument("--sweep-nodes", default=SWEEP_NODES,
                    help="comma-separated sparse tree sizes for the node-budget sweep, timed "
                         "after the main measurement (empty: skip)")
    ap.add_argument("--sweep-steps", type=int, default=40)
    ap.add_argument("--typical-steps", type=int, default=100,
                    help="whole steps timed with typical acceptance, and again with rotary "
                         "positions (0: skip both)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run an elementwise kernel that reads and writes this many MiB once before "
                         "the timed region (known sizes to calibrate rocprofv3 byte counters)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time medusa_tree_attention alone at this workload's shapes on seeded "
                         "random bf16 inputs and print one JSON line of its own (not the step metric)")
    ap.add_argument("--attention-calls", type=int, default=50)
    ap.add_argument("--lib", default=None,
                    help="load this libmedusa.so instead of the in-tree build (a build of an "
                         "earlier revision, for before / after counters; with --attention-only)")
    args = ap.parse_args()
    if args.lib:
        from speculative_decoding_amd import _lib
        _lib.use_library(args.lib)
    if args.attention_only:
        return attention_only(args)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from speculative_decoding_amd import medusa as M
    from speculative_decoding_amd.step import Dims, MedusaStep, device_weights
    from synth import get_config, make_inputs

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 1
    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    patch = os.path.join(ROOT, "tests", "golden", "plants", f"{cfg.name}_s{args.seed}.json")
    t0 = time.perf_counter()
    inp = make_inputs(cfg, args.seed, patch=patch if os.path.exists(patch) else None)
    log(f"[bench] generated {cfg.name} seed {args.seed} in {time.perf_counter() - t0:.1f} s "
        f"(planted: {os.path.exists(patch)})")
    w = device_weights(inp, dev)
    if cfg.tree == "full":
        plan = M.medusa_tree_plan_full(cfg.tree_s)
    else:
        plan = M.medusa_tree_plan_from_accuracy(inp.acc, cfg.tree_s, cfg.n_nodes)
    plan.upload(dev)
    n_nodes = plan.n_nodes
    step = MedusaStep(Dims.from_config(cfg), w, plan, dev)
    torch.cuda.synchronize()
    log(f"[bench] uploaded; tree {n_nodes} nodes, depth {plan.max_depth}")

    # bootstrap root (not part of a steady-state step: there the root is the previous bonus)
    step.heads(bootstrap_root=True)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)       # a fill kernel: writes n
        dst = torch.empty_like(src)
        torch.add(src, 1, out=dst)                                # a kernel reading n, writing n
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {n} bytes read and written")
        del src, dst

    # timed region: exactly K steps; the dominant kernel's launches are bracketed by HIP
    # events on their own stream (two event records per step)
    M.medusa_profile_reset()
    M.medusa_profile_only(DOMINANT)
    M.medusa_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    M.medusa_profile_enable(False)
    dom_ms, dom_n = M.medusa_profile_query(DOMINANT)
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")

    # per-kernel breakdown from a separate pass of the same steps with every launch timed
    # (event records add a few microseconds per launch; this pass is not the timed region)
    M.medusa_profile_reset()
    M.medusa_profile_only(None)
    M.medusa_profile_enable(True)
    for _ in range(args.steps):
        step.run(bootstrap_root=False, keep_u=False)
    torch.cuda.synchronize()
    M.medusa_profile_enable(False)
    kernels = {}
    for name in ("heads_ffn", "heads_vocab", "heads_merge", "build_tree", "proxy_qkv",
                 "attn_partial", "attn_combine", "proxy_out", "verify_lmhead", "verify_accept"):
        ms, n = M.medusa_profile_query(name)
        if n:
            kernels[name] = {"avg_us": 1e3 * ms / n, "launches": n}

    step_us = step_percentiles(torch, step, args.steps)
    sclk = clock_probe(torch, M)
    probe = hbm_probe(torch, M, w["w2"])
    log(f"[bench] probe {probe['gbps']:.0f} GB/s; step median {step_us['median']:.1f} us")
    res = step.results()
    loop = decode_loop_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, args.loop_rounds)
    typical = None
    if args.typical_steps > 0:
        log("[bench] typical acceptance")
        typical = typical_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, args.typical_steps,
                               max(3, args.typical_steps // 10))
    rope = None
    if args.typical_steps > 0:
        log("[bench] rotary positions")
        rope = rope_rate(torch, M, MedusaStep, Dims, cfg, w, plan, dev, args.typical_steps,
                         max(3, args.typical_steps // 10))
    sweep = None
    counts = [int(x) for x in args.sweep_nodes.split(",") if x.strip()]
    if counts:
        log(f"[bench] node-budget sweep over {counts}")
        sweep = node_sweep(torch, M, MedusaStep, Dims, cfg, w, dev, args.seed, counts,
                           args.sweep_steps, max(3, args.sweep_steps // 5))
    props = torch.cuda.get_device_properties(dev)
    device = {"name": props.name, "cus": props.multi_processor_count,
              "arch": getattr(props, "gcnArchName", ""), "hbm_gib": round(props.total_memory / 2**30),
              "sclk_mhz_mfma_load": None if sclk is None else round(sclk, 1)}
    a = [int(x) for x in res["accept_len"]]
    prefix_total = int(np.minimum(inp.prefix_lens, cfg.Lcap).sum())
    ab = algorithmic_bytes(cfg, n_nodes, prefix_total)
    sec = elapsed / args.steps
    steps_per_s = 1.0 / sec
    expect_a = plan.expected_accept(inp.acc)
    mean_a = float(np.mean(a))
    roof = None
    if dom_n:
        hv = 1e3 * dom_ms / dom_n
        achieved = ab[DOMINANT] / (hv * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": measured_traffic(cfg.name),
                "kernel": DOMINANT, "frac_of_probe": achieved / probe["gbps"],
                "bytes_per_launch": ab[DOMINANT], "avg_us": hv, "launches": dom_n}
    out = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * sec,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic (seeded draws, planted head ranks; no trained weights)",
        "config": {"workload": WORKLOADS[cfg.name], "name": cfg.name, "seed": args.seed,
                   "batch": cfg.B, "tree_nodes": n_nodes, "prefix": cfg.L or list(map(int, inp.prefix_lens))},
        "tokens_per_s": steps_per_s * cfg.B * (1.0 + mean_a),
        "tokens_per_s_expected": steps_per_s * cfg.B * (1.0 + expect_a),
        "accept_len": a,
        "expected_accept_len": expect_a,
        "hbm_gbps": ab["total"] / sec / 1e9,
        "hbm_frac": ab["total"] / sec / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": ab["total"],
        "step_us": step_us,
        "hbm_probe": probe,
        "roofline": roof,
        "kernels": kernels,
        "decode_loop": loop,
        "node_sweep": sweep,
        "typical": typical,
        "rope": rope,
        "device": device,
        "kernels_note": "per-kernel averages from a second pass of the same steps with every "
                        "launch event-timed (not the timed region)",
    }
    if not args.no_cpu_baseline:
        import oracle
        from tests.planting import plan_for
        log("[bench] timing the CPU oracle on one step")
        out["cpu_baseline"] = cpu_baseline(inp, plan_for(cfg, inp.acc))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
