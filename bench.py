#!/usr/bin/env python3
"""Benchmark of one pi0.5-shape action-expert decision on one MI355X.

A "step" of this benchmark is one whole decision: S = 10 flow-matching Euler
steps of the 18-layer expert over 10 action rows attending to a 768-token
prefix K/V cache, replayed from the library's captured HIP graph.  Inputs
(weights, prefix K/V, noise) are synthetic and seeded, and resident in HBM
before the timed region starts.

--workload pi05_expert_w8a16 runs the same decision on the 8-bit weight tier
(int8 codes per output column for every layer projection, bf16 activations;
the tier's instance of the persistent decision kernel).
--workload va_chunk_bf16 (256-row video-action chunk over a 4096-row cache,
8 layers x 5 steps) or wam_dit_bf16 (DiT-style step over 4128 tokens, 4
blocks) measures the large-token plan instead; those are MFMA-bound, so their
roofline is the dominant GEMM's TFLOP/s against the bf16 dense peak.
--workload prefix_prefill_bf16 times the prefix prefill (18 causal layers of
width 2048 over 768 tokens in an 800-row bucket, writing the K/V cache), one
phx_expert_prefill call per step.
--multi-kernel runs the pi0.5 decision (bf16 or the 8-bit tier) on the
captured multi-kernel graph instead of the persistent decision kernel.
--timeline prints, instead of the benchmark line, the persistent kernel's
critical path per phase of a layer-step (from its per-workgroup timeline).

Prints ONE JSON line (see --help for the knobs).  Besides the wall-clock
figure it carries:
  * "roofline": the dominant kernel's algorithmic bytes per launch divided by
    its average launch duration, timed here with HIP events on the stream the
    kernel runs on, against MI355X's 8 TB/s HBM peak;
  * "cpu_baseline": the CPU oracle timed on a bounded sample of the same
    workload on this host's cores, and on one thread (a reported baseline,
    not the target);
  * measured ceilings beside the spec peaks: a 4 GiB device copy for the
    HBM-bound lines, a library 8192^3 bf16 GEMM for the MFMA-bound ones.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--workload NAME]
       [--multi-kernel] [--timeline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import phx_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix peak
WORKLOAD = "pi05_expert_bf16"
BATCH_WORKLOADS = ("rollout_b16_bf16",)
W8_WORKLOADS = ("pi05_expert_w8a16",)
TOKEN_WORKLOADS = ("va_chunk_bf16", "wam_dit_bf16")
PREFILL_WORKLOADS = ("prefix_prefill_bf16",)
PROFILES = os.path.join(ROOT, "profiles")
# HBM counter records of the decision kernel, per workload (its bf16 and 8-bit instances)
TRAFFIC_FILES = {WORKLOAD: os.path.join(PROFILES, "traffic_pi05_expert_bf16.json"),
                 "pi05_expert_w8a16": os.path.join(PROFILES, "traffic_pi05_expert_w8a16.json")}


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg: dict) -> dict:
    """Bytes one decision must move at least once per Euler step: every
    weight matrix of the step loop, the valid prefix K/V rows of every layer,
    and the fp32 modulation rows the norms read."""
    esz = 2 if cfg["dtype"] == "bf16" else 4
    D, A, F = cfg["width"], cfg["state_dim"], cfg["mlp_hidden"]
    H, KVH, Dh, NL = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["layers"]
    qkv = (H + 2 * KVH) * Dh
    w_layer = (D * qkv + H * Dh * D + D * 2 * F + F * D) * esz
    if int(cfg.get("flags", 0)) & 8:  # the 8-bit tier: one byte per code plus a float scale per column
        w_layer = (D * qkv + H * Dh * D + D * 2 * F + F * D) + 4 * (qkv + D + 2 * F + D)
    w_step = NL * w_layer + 2 * A * D * esz
    lens = phx_inputs.prefix_lengths(cfg)
    kv_step = int(sum(2 * NL * int(L) * KVH * Dh * esz for L in lens))
    mod_step = (2 * NL + 1) * 2 * D * 4
    S = cfg["steps"]
    return dict(weights_per_step=w_step, kv_per_step=kv_step, mod_per_step=mod_step,
                per_decision=S * (w_step + kv_step + mod_step))


def token_flops(cfg: dict) -> dict:
    """Algorithmic FLOPs and bytes of one large-token decision: every GEMM
    (2 per multiply-add) and attention (QK^T and PV over prefix + chunk keys),
    and every weight, valid cache row and modulation row once per step."""
    D, A, F, M = cfg["width"], cfg["state_dim"], cfg["mlp_hidden"], cfg["rows"]
    H, KVH, Dh, NL, S = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["layers"], cfg["steps"]
    dit = cfg.get("block", "decoder") == "dit"
    L = int(phx_inputs.prefix_lengths(cfg)[0])
    qkv, hd = (H + 2 * KVH) * Dh, H * Dh
    up = F if dit else 2 * F
    gemm_layer = 2 * M * (D * qkv + hd * D + D * up + F * D)
    attn_layer = 4 * M * (L + M) * hd
    io = 0 if dit else 2 * 2 * M * A * D
    w_step = 2 * (NL * (D * qkv + hd * D + D * up + F * D) + (0 if dit else 2 * A * D))
    kv_step = 2 * 2 * NL * L * KVH * Dh
    mod_step = 4 * (NL * 6 * D if dit else (2 * NL + 1) * 2 * D)
    return dict(flops_per_decision=S * (NL * (gemm_layer + attn_layer) + io),
                gemm_flops_per_decision=S * (NL * gemm_layer + io), attn_flops_per_decision=S * NL * attn_layer,
                bytes_per_decision=S * (w_step + kv_step + mod_step))


def node_flops(cfg: dict, kind: int) -> int:
    """FLOPs of one launch of a large-token plan kernel kind."""
    from flow_matching_action_decision_amd.binding import PHX_NODE as K
    D, A, F, M = cfg["width"], cfg["state_dim"], cfg["mlp_hidden"], cfg["rows"]
    H, KVH, Dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    dit = cfg.get("block", "decoder") == "dit"
    L = int(phx_inputs.prefix_lengths(cfg)[0])
    return {K["IN_PROJ"]: 2 * M * A * D, K["QKV"]: 2 * M * D * (H + 2 * KVH) * Dh,
            K["ATTENTION"]: 4 * M * (L + M) * H * Dh, K["OUT_PROJ_RESID"]: 2 * M * H * Dh * D,
            K["GATEUP"]: 2 * M * D * (F if dit else 2 * F), K["DOWN_PROJ_RESID"]: 2 * M * F * D,
            K["OUT_EULER"]: 2 * M * D * A}.get(kind, 0)


DECISION_KERNEL_SOURCES = ("phx_decide.hip", "phx_decide.h")
TOKEN_KERNEL_SOURCES = ("phx_tokens.hip", "phx_tokens.h")


def kernel_source_hash(files=DECISION_KERNEL_SOURCES) -> str:
    """Hash of the sources of the timed kernel (its code and launch shape)."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "flow_matching_action_decision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_hash: str, name: str = WORKLOAD):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILES[name]) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash:
        return None
    return t.get("bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo), and the
    logical cores the process may run on."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    name = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 0
    return f"{name} ({n} logical cores available)"


def omp_threads() -> int:
    import ctypes
    try:
        return int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except OSError:
        return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(cfg: dict, inp: dict, budget_s: float) -> dict:
    """Time the oracle, unchanged, on a bounded sample: the first s Euler
    steps of the same decision (s chosen so the sample takes about budget_s),
    scaled to ms per full decision."""
    import oracle
    lib = oracle.load()
    probe = dict(cfg, steps=1)
    t0 = time.perf_counter()
    oracle.decide(probe, inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=lib)
    t1 = time.perf_counter()
    per_step = t1 - t0
    s = int(max(1, min(cfg["steps"], budget_s // max(per_step, 1e-9))))
    if s > 1:
        t0 = time.perf_counter()
        oracle.decide(dict(cfg, steps=s), inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=lib)
        t1 = time.perf_counter()
        per_step = (t1 - t0) / s
    cores = omp_threads()
    one = one_thread_step_s(cfg, inp, lib)
    return {"value": round(per_step * cfg["steps"] * 1e3, 1), "unit": "ms/decision", "cores": cores,
            "kind": "oracle",
            "sample": f"first {s} of {cfg['steps']} Euler steps of the same {cfg['layers']}-layer decision "
                      f"(double-precision oracle, OpenMP), scaled to a full decision",
            **({"value_1_thread": round(one * cfg["steps"] * 1e3, 1),
                "sample_1_thread": "first Euler step on one OpenMP thread, scaled to a full decision"}
               if one is not None else {})}


def one_thread_step_s(cfg: dict, inp: dict, lib):
    """Seconds of one Euler step of the oracle on a single OpenMP thread (the
    process's OpenMP runtime is set to one thread and then restored), or None
    where the runtime cannot be reached."""
    import ctypes
    import oracle
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
    except OSError:
        return None
    before = int(gomp.omp_get_max_threads())
    gomp.omp_set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.decide(dict(cfg, steps=1), inp["weights"], inp["kv_k"], inp["kv_v"], inp["lens"], inp["noise"], lib=lib)
        return time.perf_counter() - t0
    finally:
        gomp.omp_set_num_threads(before)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default=WORKLOAD,
                    choices=(WORKLOAD,) + BATCH_WORKLOADS + W8_WORKLOADS + TOKEN_WORKLOADS + PREFILL_WORKLOADS)
    ap.add_argument("--steps", type=int, default=200, help="timed decisions")
    ap.add_argument("--warmup", type=int, default=20, help="untimed decisions before the timed region")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--kernel-reps", type=int, default=50, help="timed launches of the dominant kernel")
    ap.add_argument("--multi-kernel", action="store_true",
                    help="pi05_expert_bf16 or pi05_expert_w8a16 on the captured multi-kernel graph (2 + 6 NL "
                         "launches per Euler step) instead of the persistent decision kernel")
    ap.add_argument("--timeline", action="store_true",
                    help="pi05_expert_bf16 on the persistent kernel with its phase timeline on: prints one JSON "
                         "line of per-phase critical-path microseconds instead of the benchmark line")
    ap.add_argument("--bf16-act", action="store_true",
                    help="large-token workloads: plain bf16 GEMM activations (PHX_FLAG_BF16_ACT) instead of the "
                         "plan's default (paired for the DiT-style step and the prefill)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device-to-device copy of 256 MiB (a kernel of known traffic, to scale "
                         "profiler byte counters against)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decision path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only (WORLD_SIZE > 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (the decision runs only in the HIP library)", file=sys.stderr)
        sys.exit(1)
    from flow_matching_action_decision_amd.expert import Expert
    from flow_matching_action_decision_amd import binding

    if args.multi_kernel and args.workload != WORKLOAD and args.workload not in W8_WORKLOADS:
        print("--multi-kernel applies to pi05_expert_bf16 and pi05_expert_w8a16 (the other workloads have one "
              "execution path)", file=sys.stderr)
        sys.exit(2)
    if args.timeline:
        if args.workload != WORKLOAD or args.multi_kernel:
            print("--timeline applies to pi05_expert_bf16 on the persistent kernel", file=sys.stderr)
            sys.exit(2)
        return bench_timeline(args)
    if args.workload in TOKEN_WORKLOADS:
        return bench_tokens(args)
    if args.workload in PREFILL_WORKLOADS:
        return bench_prefill(args)
    name = args.workload
    cfg = phx_inputs.workload(name)
    log(f"bench: generating inputs for {name}")
    inp = phx_inputs.make_inputs(cfg, args.seed)
    ab = algorithmic_bytes(cfg)

    mk = bool(args.multi_kernel)
    log("bench: creating handle")
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=binding.PHX_FLAG_MULTI_KERNEL if mk else 0)
    keep = ex.load_all(inp)
    noise = torch.from_numpy(inp["noise"]).cuda()
    out = torch.empty_like(noise)
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        ex.decide(noise, out)
    torch.cuda.synchronize()

    # timed region: K decisions back to back
    log(f"bench: timing {args.steps} decisions")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for a, b in ev:
        a.record(stream)
        ex.decide(noise, out)
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = np.array([a.elapsed_time(b) for a, b in ev])
    ms = total_ms / args.steps
    log(f"bench: {ms:.4f} ms/decision (p50 {np.percentile(per, 50):.4f}, p95 {np.percentile(per, 95):.4f})")
    # a decision call returns once enqueued; the status word says the last one ran to its end
    assert ex.status() == 0, "the last timed decision gave up waiting (persistent kernel status)"

    # dominant kernel: duration of its launches, timed with HIP events on the
    # stream it runs on
    dom = ex.time_dominant_kernel(args.kernel_reps)
    # the persistent decision kernel (bf16 or the 8-bit tier's instance), else the multi-kernel graph (the
    # rollout batch, --multi-kernel); the committed counter records cover the persistent kernel
    persistent = dom["name"] == "decision_kernel"
    kernel_hash = kernel_source_hash(DECISION_KERNEL_SOURCES if persistent
                                     else ("phx_kernels.hip", "phx_internal.h") + TOKEN_KERNEL_SOURCES)
    traffic = measured_traffic(kernel_hash, name) if persistent and name in TRAFFIC_FILES else None
    achieved = dom["bytes_per_launch"] / (dom["ms_per_launch"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom["name"], "bytes_per_launch": dom["bytes_per_launch"],
                "us_per_launch": round(dom["ms_per_launch"] * 1e3, 3), "kernel_hash": kernel_hash}

    # execution-state capsule: snapshot, restore and fork of the declared state
    # regions, each timed with HIP events on the handle's stream
    capsule = capsule_timing(ex, Expert, cfg, inp, stream, flags=binding.PHX_FLAG_MULTI_KERNEL if mk else 0)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    first = out.cpu().numpy()
    assert np.all(np.isfinite(first)), "non-finite actions"
    nk = ex.kernels_per_decision()
    del keep
    ex.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, inp, args.cpu_budget_s)
        cpu["cpu_model"] = cpu_model()

    hbm_gbs = ab["per_decision"] / (ms * 1e-3) / 1e9
    copy_gbs = measured_copy_gbs()
    lens = [int(L) for L in inp["lens"]]
    w8 = name in W8_WORKLOADS
    batch = name in BATCH_WORKLOADS
    if w8:
        metric = ("ms/decision (pi0.5-shape, 18L x 10 steps, 8-bit weight tier" + (", multi-kernel graph" if mk else "")
                  + ") + % peak HBM GB/s, 1 GPU")
    elif mk:
        metric = "ms/decision (pi0.5-shape, 18L x 10 steps, multi-kernel graph) + % peak HBM GB/s, 1 GPU"
    elif batch:
        metric = f"ms/decision ({name}: {cfg['batch']} requests, 18L x 10 steps) + % peak HBM GB/s, 1 GPU"
    else:
        metric = "ms/decision (pi0.5-shape, 18L x 10 steps) + % peak HBM GB/s, 1 GPU"
    line = {
        "metric": metric,
        "value": round(ms, 4), "unit": "ms/decision", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) bf16 prefix K/V, N(0,1) noise)",
        "config": {"workload": name, "layers": cfg["layers"], "euler_steps": cfg["steps"],
                   "action_rows": cfg["rows"], "prefix_len": lens[0] if cfg["batch"] == 1 else lens, "width": cfg["width"],
                   "heads": f"{cfg['n_heads']}x{cfg['head_dim']} / {cfg['n_kv_heads']} kv",
                   "mlp_hidden": cfg["mlp_hidden"], "batch": cfg["batch"],
                   **({"weights": "int8 codes per output column (layer projections), bf16 in/out projections"}
                      if w8 else {}),
                   **({"path": "multi-kernel graph"} if mk else {}),
                   **({"gemm_activations": "QKV, gate/up and down inputs paired bf16 (hi + lo)"} if batch and not mk and not w8 else {})},
        "decisions_per_s": round(1000.0 / ms, 1),
        "p50_ms": round(float(np.percentile(per, 50)), 4), "p95_ms": round(float(np.percentile(per, 95)), 4),
        **({"requests_per_s": round(1000.0 * cfg["batch"] / ms, 1),
            "ms_per_request_amortised": round(ms / cfg["batch"], 4)} if cfg["batch"] > 1 else {}),
        "algorithmic_bytes_per_decision": ab["per_decision"],
        "hbm_gbs": round(hbm_gbs, 1), "hbm_frac_of_peak": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "hbm_copy_gbs": round(copy_gbs, 1), "hbm_frac_of_copy": round(hbm_gbs / copy_gbs, 4),
        "kernels_per_decision": nk,
        "capsule": capsule,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def measured_copy_gbs(gib: int = 4, reps: int = 50, warm: int = 10) -> float:
    """Device-to-device copy bandwidth of this GPU: a `gib` GiB buffer copied
    into another, best of `reps` after `warm` untimed copies; read plus
    written bytes over the time (a practical ceiling beside the 8 TB/s spec)."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(warm):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    best_ms = min(a.elapsed_time(b) for a, b in ev)
    del src, dst
    torch.cuda.empty_cache()
    return 2.0 * n / (best_ms * 1e-3) / 1e9


def measured_gemm_tflops(n: int = 8192, reps: int = 20, warm: int = 5) -> float:
    """Dense bf16 GEMM rate of this GPU through the vendor library (torch.matmul,
    n x n x n), best of `reps` after `warm`: a practical ceiling beside the
    2.5 PFLOP/s spec."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    for _ in range(warm):
        torch.matmul(a, b)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for e0, e1 in ev:
        e0.record(stream)
        torch.matmul(a, b)
        e1.record(stream)
    torch.cuda.synchronize()
    best_ms = min(e0.elapsed_time(e1) for e0, e1 in ev)
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / (best_ms * 1e-3) / 1e12


PHASES = ("qkv", "attention", "merge", "out_proj", "out_proj_allreduce", "gate_up", "down", "down_allreduce")


def bench_timeline(args):
    """Critical path of the persistent decision kernel, phase by phase.

    The handle records, per workgroup, when its compute waves finished each
    phase of each layer-step (a 100 MHz counter).  A phase's critical time is
    how far the latest workgroup's stamp moved past the previous phase's
    latest stamp, averaged over the interior layer-steps (Euler steps 1..S-2,
    layers 2..NL-3), away from the ramp at the start and the drain at the
    end.  Also reported: per phase, how long after the previous phase's
    latest stamp the first and the median workgroup finish it."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert
    from flow_matching_action_decision_amd import binding

    cfg = phx_inputs.workload(WORKLOAD)
    inp = phx_inputs.make_inputs(cfg, args.seed)
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=binding.PHX_FLAG_TIMELINE)
    keep = ex.load_all(inp)
    noise = torch.from_numpy(inp["noise"]).cuda()
    out = torch.empty_like(noise)
    stream = torch.cuda.current_stream()
    for _ in range(max(args.warmup, 1)):
        ex.decide(noise, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    ex.decide(noise, out)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    tl = np.asarray(ex.timeline(), dtype=np.int64)
    del keep
    ex.close()
    S, NL = cfg["steps"], cfg["layers"]
    crit = np.zeros(len(PHASES))
    first = np.zeros(len(PHASES))
    median = np.zeros(len(PHASES))
    n = 0
    for k in range(1, S - 1):
        base = 1 + k * (2 + len(PHASES) * NL)
        for l in range(2, NL - 2):
            e = base + 1 + len(PHASES) * l
            prev = tl[:, e - 1].max()
            for p in range(len(PHASES)):
                col = tl[:, e + p]
                crit[p] += col.max() - prev
                first[p] += col.min() - prev
                median[p] += np.median(col) - prev
                prev = col.max()
            n += 1
    to_us = 0.01 / n  # 100 MHz ticks, averaged
    line = {"workload": WORKLOAD, "kernel": "decision_kernel", "ms_per_decision_with_timeline": round(ms, 4),
            "layer_steps_averaged": n,
            "critical_us": {p: round(float(c * to_us), 2) for p, c in zip(PHASES, crit)},
            "critical_us_per_layer_step": round(float(crit.sum() * to_us), 2),
            "first_finish_after_previous_us": {p: round(float(c * to_us), 2) for p, c in zip(PHASES, first)},
            "median_finish_after_previous_us": {p: round(float(c * to_us), 2) for p, c in zip(PHASES, median)}}
    print(json.dumps(line), flush=True)


def capsule_timing(ex, Expert, cfg: dict, inp: dict, stream, reps: int = 20, flags: int = 0) -> dict:
    """Average ms of a capsule snapshot, a restore into the same handle and a
    fork into a second handle of the same plan (restore on a fresh handle)."""
    import torch
    cap = ex.capsule_save()
    torch.cuda.synchronize()

    def timed(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return float(sum(a.elapsed_time(b) for a, b in ev) / reps)

    snap = timed(lambda: ex.capsule_save(cap))
    rest = timed(lambda: ex.capsule_restore(cap))
    other = Expert(cfg, inp["weights"], inp["weights_bits"], flags=flags)
    try:
        fork = timed(lambda: other.capsule_restore(cap))
    finally:
        other.close()
    return {"bytes": int(cap.numel()), "regions": [r["name"] for r in ex.capsule_regions()],
            "snapshot_ms": round(snap, 4), "restore_ms": round(rest, 4), "fork_ms": round(fork, 4)}


def bench_tokens(args):
    """The large-token workloads: decision time, per-kind kernel breakdown,
    and the dominant GEMM against the MFMA bf16 peak."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert

    name = args.workload
    cfg = phx_inputs.workload(name)
    dit = cfg.get("block", "decoder") == "dit"
    log(f"bench: generating inputs for {name}")
    inp = phx_inputs.make_inputs(cfg, args.seed)
    fl = token_flops(cfg)
    log("bench: creating handle")
    from flow_matching_action_decision_amd import binding
    tflags = binding.PHX_FLAG_BF16_ACT if args.bf16_act else 0
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=tflags)
    keep = ex.load_all(inp)
    noise = torch.from_numpy(inp["noise"]).cuda()
    out = torch.empty_like(noise)
    stream = torch.cuda.current_stream()
    steps = min(args.steps, 50)
    warm = min(args.warmup, 5)
    for _ in range(warm):
        ex.decide(noise, out)
    torch.cuda.synchronize()
    log(f"bench: timing {steps} decisions")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in ev:
        a.record(stream)
        ex.decide(noise, out)
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    per = np.array([a.elapsed_time(b) for a, b in ev])
    log(f"bench: {ms:.4f} ms/decision")

    # per-kind breakdown over the first step's launches, and the dominant kind by FLOPs
    nodes = ex.nodes()
    first = [i for i, n in enumerate(nodes) if n["step"] == 0]
    t = ex.time_nodes(first, reps=max(3, min(args.kernel_reps, 10)))
    kinds = {}
    # matrix-core work of the paired-activation GEMMs (the DiT-style block's default) beyond the algorithmic FLOPs
    paired = dit and not args.bf16_act
    paired_extra = 0
    for i, tm in zip(first, t):
        n = nodes[i]
        k = kinds.setdefault(n["name"], dict(kind=n["kind"], launches=0, ms=0.0, flops=0))
        k["launches"] += 1
        k["ms"] += tm
        k["flops"] += node_flops(cfg, n["kind"])
        if paired and n["kind"] in (binding.PHX_NODE["QKV"], binding.PHX_NODE["GATEUP"],
                                    binding.PHX_NODE["DOWN_PROJ_RESID"]):
            paired_extra += node_flops(cfg, n["kind"])
    for nm, k in sorted(kinds.items(), key=lambda kv: -kv[1]["ms"]):
        tf = k["flops"] / (k["ms"] * 1e-3) / 1e12 if k["flops"] else 0.0
        log(f"  {nm:24s} x{k['launches']:3d}  {k['ms'] * 1e3 / k['launches']:9.1f} us/launch  {tf:7.1f} TFLOP/s")
    dom_name = max(kinds, key=lambda nm: kinds[nm]["flops"])
    dk = kinds[dom_name]
    us = dk["ms"] * 1e3 / dk["launches"]
    f_launch = dk["flops"] // dk["launches"]
    achieved = f_launch / (us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None, "kernel": dom_name,
                "flops_per_launch": f_launch, "us_per_launch": round(us, 3),
                "kernel_hash": kernel_source_hash(TOKEN_KERNEL_SOURCES)}
    res = out.cpu().numpy()
    assert np.all(np.isfinite(res)), "non-finite output"
    history = None
    if not dit:
        # history update: commit the decided chunk into the cache (event-timed on the stream); the
        # handle's state is restored from a capsule afterwards
        cap = ex.capsule_save()
        reps = 8
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            ex.commit_chunk(out[0])
            b.record(stream)
        torch.cuda.synchronize()
        cm = [a.elapsed_time(b) for a, b in ev]
        ex.capsule_restore(cap)
        torch.cuda.synchronize()
        history = {"commit_ms": round(float(np.mean(cm)), 4), "commits": reps,
                   "rows_per_commit": cfg["rows"], "window": cfg["capacity"],
                   "history_rows": f"{int(phx_inputs.prefix_lengths(cfg)[0])} -> "
                                   f"{min(cfg['capacity'], int(phx_inputs.prefix_lengths(cfg)[0]) + reps * cfg['rows'])}"}
        del cap
    nk = ex.kernels_per_decision()
    del keep
    ex.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_tokens(cfg, inp, fl)
        cpu["cpu_model"] = cpu_model()

    tflops = fl["flops_per_decision"] / (ms * 1e-3) / 1e12
    hbm = fl["bytes_per_decision"] / (ms * 1e-3) / 1e9
    gemm_tf = measured_gemm_tflops()
    line = {
        "metric": f"ms/decision ({name}) + % of MFMA bf16 peak, 1 GPU",
        "value": round(ms, 4), "unit": "ms/decision", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) bf16 cache, N(0,1) state)",
        "config": {"workload": name, "block": "dit" if dit else "decoder", "layers": cfg["layers"],
                   "euler_steps": cfg["steps"], "rows": cfg["rows"],
                   "prefix_len": int(phx_inputs.prefix_lengths(cfg)[0]), "width": cfg["width"],
                   "heads": f"{cfg['n_heads']}x{cfg['head_dim']} / {cfg['n_kv_heads']} kv",
                   "mlp_hidden": cfg["mlp_hidden"],
                   "gemm_activations": "QKV, gate/up and down inputs paired bf16 (hi + lo)" if paired_extra else "bf16"},
        "decisions_per_s": round(1000.0 / ms, 2),
        "mfma_flops_executed_per_decision": fl["flops_per_decision"] + paired_extra * cfg["steps"],
        "p50_ms": round(float(np.percentile(per, 50)), 4), "p95_ms": round(float(np.percentile(per, 95)), 4),
        "flops_per_decision": fl["flops_per_decision"], "tflops": round(tflops, 1),
        "mfma_frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "library_gemm_tflops": round(gemm_tf, 1), "mfma_frac_of_library_gemm": round(tflops / gemm_tf, 4),
        "algorithmic_bytes_per_decision": fl["bytes_per_decision"], "hbm_gbs": round(hbm, 1),
        "kernels_per_decision": nk, "history_update": history, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_tokens(cfg: dict, inp: dict, fl: dict) -> dict:
    """Time the oracle, unchanged, on a bounded slice of the same workload
    (one layer of one step for the chunk; one block over 528 tokens for the
    DiT-style step) and scale by the FLOP ratio to a whole decision."""
    import oracle
    lib = oracle.load()
    if cfg.get("block", "decoder") == "dit":
        sc = dict(cfg, layers=1, rows=528)
        x = inp["noise"][0, :528]
        wsl = phx_inputs.weight_slices(cfg)
        ssl = phx_inputs.weight_slices(sc)
        w = np.empty(phx_inputs.weight_count(sc), dtype=np.float32)
        for nm, (off, shape) in ssl.items():
            if nm == "W_mod":
                o2, sh2 = wsl["W_mod"]
                w[off:off + int(np.prod(shape))] = inp["weights"][o2:o2 + int(np.prod(shape))]
            else:
                o2, _ = wsl[nm]
                w[off:off + int(np.prod(shape))] = inp["weights"][o2:o2 + int(np.prod(shape))]
        t0 = time.perf_counter()
        oracle.dit(sc, w, x, lib=lib)
        dt_s = time.perf_counter() - t0
        what = "one block over 528 of the 4128 tokens"
    else:
        sc = dict(cfg, layers=1, steps=1)
        wsl = phx_inputs.weight_slices(cfg)
        ssl = phx_inputs.weight_slices(sc)
        w = np.empty(phx_inputs.weight_count(sc), dtype=np.float32)
        for nm, (off, shape) in ssl.items():
            n = int(np.prod(shape))
            o2, _ = wsl[nm]
            w[off:off + n] = inp["weights"][o2:o2 + n]
        t0 = time.perf_counter()
        oracle.decide(sc, w, inp["kv_k"][:, :1], inp["kv_v"][:, :1], inp["lens"], inp["noise"], lib=lib)
        dt_s = time.perf_counter() - t0
        what = "one layer of one Euler step (with the in- and out-projections)"
    fs = token_flops(sc)["flops_per_decision"]
    return {"value": round(dt_s * fl["flops_per_decision"] / fs * 1e3, 1), "unit": "ms/decision",
            "cores": omp_threads(), "kind": "oracle",
            "sample": f"{what} (double-precision oracle, OpenMP), scaled by FLOPs to a full decision"}


def prefill_flops(cfg: dict, n: int) -> dict:
    """Algorithmic work of one prefill over n tokens: every GEMM on the n token
    rows (the last layer only its QKV: nothing after it reaches the cache),
    causal attention (QK^T and PV over keys 0..i for token i), and bytes: the
    weights used once, the token rows read, the cache written."""
    D, F = cfg["width"], cfg["mlp_hidden"]
    H, KVH, Dh, NL = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["layers"]
    qkv, hd, kvd = (H + 2 * KVH) * Dh, H * Dh, KVH * Dh
    rest = hd * D + D * 2 * F + F * D
    gemm = 2 * n * (NL * D * qkv + (NL - 1) * rest)
    attn = (NL - 1) * 4 * hd * (n * (n + 1) // 2)
    byts = 2 * (NL * D * qkv + (NL - 1) * rest) + n * D * 4 + 2 * NL * n * kvd * 2
    return dict(flops=gemm + attn, gemm_flops=gemm, attn_flops=attn, bytes=byts)


def prefill_node_flops(cfg: dict, kind: int, n: int) -> int:
    """FLOPs of one launch of a prefill kernel kind over n tokens."""
    from flow_matching_action_decision_amd.binding import PHX_NODE as K
    D, F = cfg["width"], cfg["mlp_hidden"]
    H, KVH, Dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    return {K["QKV"]: 2 * n * D * (H + 2 * KVH) * Dh, K["ATTENTION"]: 4 * H * Dh * (n * (n + 1) // 2),
            K["OUT_PROJ_RESID"]: 2 * n * H * Dh * D, K["GATEUP"]: 2 * n * D * 2 * F,
            K["DOWN_PROJ_RESID"]: 2 * n * F * D}.get(kind, 0)


def bench_prefill(args):
    """The prefix prefill: time per phx_expert_prefill call (token rows in,
    every layer's K/V out), per-kind kernel breakdown, and the dominant GEMM
    against the MFMA bf16 peak."""
    import torch
    from flow_matching_action_decision_amd.expert import Expert

    name = args.workload
    cfg = phx_inputs.workload(name)
    n = int(phx_inputs.prefix_lengths(cfg)[0])
    log(f"bench: generating inputs for {name}")
    inp = phx_inputs.make_inputs(cfg, args.seed)
    fl = prefill_flops(cfg, n)
    log("bench: creating handle")
    from flow_matching_action_decision_amd import binding
    ex = Expert(cfg, inp["weights"], inp["weights_bits"], flags=binding.PHX_FLAG_BF16_ACT if args.bf16_act else 0)
    x = torch.from_numpy(np.ascontiguousarray(inp["noise"][0])).cuda()
    kvd = cfg["n_kv_heads"] * cfg["head_dim"]
    k = torch.empty((cfg["layers"], n, kvd), dtype=torch.int16, device="cuda")
    v = torch.empty_like(k)
    stream = torch.cuda.current_stream()
    steps = min(args.steps, 50)
    warm = min(args.warmup, 5)
    for _ in range(warm):
        ex.prefill(x, n, k, v)
    torch.cuda.synchronize()
    log(f"bench: timing {steps} prefills")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for a, b in ev:
        a.record(stream)
        ex.prefill(x, n, k, v)
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / steps
    per = np.array([a.elapsed_time(b) for a, b in ev])
    log(f"bench: {ms:.4f} ms/prefill")

    nodes = ex.nodes()
    idx = list(range(len(nodes)))
    t = ex.time_nodes(idx, reps=max(3, min(args.kernel_reps, 10)))
    kinds = {}
    for i, tm in zip(idx, t):
        nd = nodes[i]
        kk = kinds.setdefault(nd["name"], dict(kind=nd["kind"], launches=0, ms=0.0, flops=0))
        kk["launches"] += 1
        kk["ms"] += tm
        kk["flops"] += prefill_node_flops(cfg, nd["kind"], n)
    for nm, kk in sorted(kinds.items(), key=lambda kv: -kv[1]["ms"]):
        tf = kk["flops"] / (kk["ms"] * 1e-3) / 1e12 if kk["flops"] else 0.0
        log(f"  {nm:24s} x{kk['launches']:3d}  {kk['ms'] * 1e3 / kk['launches']:9.1f} us/launch  {tf:7.1f} TFLOP/s")
    dom_name = max(kinds, key=lambda nm: kinds[nm]["flops"])
    dk = kinds[dom_name]
    us = dk["ms"] * 1e3 / dk["launches"]
    f_launch = dk["flops"] // dk["launches"]
    achieved = f_launch / (us * 1e-6) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None, "kernel": dom_name,
                "flops_per_launch": f_launch, "us_per_launch": round(us, 3),
                "kernel_hash": kernel_source_hash(TOKEN_KERNEL_SOURCES)}
    kh = _bf16_bits_to_f32(k)
    assert np.all(np.isfinite(kh)), "non-finite cache"
    nk = ex.kernels_per_decision()
    ex.close()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline_prefill(cfg, inp, fl)
        cpu["cpu_model"] = cpu_model()

    tflops = fl["flops"] / (ms * 1e-3) / 1e12
    gemm_tf = measured_gemm_tflops()
    line = {
        "metric": f"ms/prefill ({name}) + % of MFMA bf16 peak, 1 GPU",
        "value": round(ms, 4), "unit": "ms/prefill", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,0.02) bf16 weights and gains, N(0,1) token rows)",
        "config": {"workload": name, "block": "prefill", "layers": cfg["layers"], "tokens": n,
                   "bucket_rows": cfg["rows"], "width": cfg["width"],
                   "heads": f"{cfg['n_heads']}x{cfg['head_dim']} / {cfg['n_kv_heads']} kv",
                   "mlp_hidden": cfg["mlp_hidden"], "mask": "causal",
                   "gemm_activations": "bf16" if args.bf16_act else "QKV, gate/up and down inputs paired bf16 (hi + lo)"},
        "prefills_per_s": round(1000.0 / ms, 2),
        "p50_ms": round(float(np.percentile(per, 50)), 4), "p95_ms": round(float(np.percentile(per, 95)), 4),
        "flops_per_prefill": fl["flops"], "tflops": round(tflops, 1),
        "mfma_frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "library_gemm_tflops": round(gemm_tf, 1), "mfma_frac_of_library_gemm": round(tflops / gemm_tf, 4),
        "algorithmic_bytes_per_prefill": fl["bytes"], "hbm_gbs": round(fl["bytes"] / (ms * 1e-3) / 1e9, 1),
        "kernels_per_prefill": nk, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def _bf16_bits_to_f32(t) -> np.ndarray:
    u = t.cpu().numpy().view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def cpu_baseline_prefill(cfg: dict, inp: dict, fl: dict) -> dict:
    """Time the oracle, unchanged, on a bounded sample of the prefill (the
    first two layers over the first 64 tokens) and scale by the FLOP ratio to
    the whole prefill."""
    import oracle
    lib = oracle.load()
    n = 64
    sc = dict(cfg, layers=2)
    wsl = phx_inputs.weight_slices(cfg)
    ssl = phx_inputs.weight_slices(sc)
    w = np.empty(phx_inputs.weight_count(sc), dtype=np.float32)
    for nm, (off, shape) in ssl.items():
        m = int(np.prod(shape))
        o2, _ = wsl[nm]
        w[off:off + m] = inp["weights"][o2:o2 + m]
    t0 = time.perf_counter()
    oracle.prefill(sc, w, inp["noise"][0], n, lib=lib)
    dt_s = time.perf_counter() - t0
    fs = prefill_flops(sc, n)["flops"]
    return {"value": round(dt_s * fl["flops"] / fs * 1e3, 1), "unit": "ms/prefill", "cores": omp_threads(),
            "kind": "oracle",
            "sample": f"the first two layers over the first {n} tokens (double-precision oracle, OpenMP), "
                      f"scaled by FLOPs to the whole prefill"}


if __name__ == "__main__":
    main()
