"""Benchmark of the GDN recurrent decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one layer's call of the hot path over one batch of seeded synthetic input that is
already resident in HBM: gdn_decode_step for the decode workloads (state read once, T tokens,
state written once), gdn_conv_gate_decode for the fused one, gdn_decode_verify for the verify
rounds, and gdn_prefill for the prompt workload (`--sequential` runs that workload through
gdn_decode_step instead; its roofline prices the recurrence's flop against the fp32 matrix
peak, as the chunked form is bound by arithmetic, not HBM). Layer buffers (state, inputs,
outputs) are rotated so that the state a step reads was not left in the 256 MB MALL by the
previous step. W untimed steps, then K timed steps between two device synchronisations; the
HIP events that time them are recorded on the stream the kernels are launched on.

Prints ONE JSON line. `value` is microseconds per layer step (lower is better); `roofline`
prices the kernel's algorithmic bytes per launch against MI355X's 8 TB/s HBM peak; `traffic`
is the measured HBM bytes per launch from a committed rocprofv3 counter summary, or null if
the kernel source changed since it was taken; `cpu_baseline` times the fp64 oracle on a
bounded sample of the same workload on the host.

The low-rank window workloads (`lowrank_*`) time gdn_lowrank_decode_step.

`--workload copy_<MB>` instead times a plain device-to-device copy of that many MB (torch's
copy kernel), the calibration used for the counter-based traffic and the practical
read+write bandwidth ceiling.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN decode µs/layer + achieved HBM GB/s (% roofline), B=256 H=48 128×128"
DEFAULT_WORKLOAD = "decode_b256_h48_d128_t1"
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "gated_deltanet_recurrent_02_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("gdn_kernels.hip", "gdn_launch.h")]
PREFILL_SOURCES = [os.path.join(_CSRC, f)
                   for f in ("gdn_prefill.hip", "gdn_prefill_launch.h", "gdn_launch.h")]
LOWRANK_SOURCES = [os.path.join(_CSRC, f)
                   for f in ("gdn_lowrank.hip", "gdn_lowrank_launch.h", "gdn_launch.h")]


def code_text(src: str) -> str:
    """C++ source without its comments, whitespace runs collapsed: what the compiler sees,
    so that editing a comment does not count as changing a kernel. String and character
    literals are kept verbatim."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(prefill: bool = False, lowrank: bool = False) -> str:
    """Hash of the code a workload runs: the kernel sources (decode, prefill or low-rank
    window kernels) as code_text, plus the compiler flags they are built with."""
    from gated_deltanet_recurrent_02_amd import build as gdn_build
    h = hashlib.sha256()
    for p in (PREFILL_SOURCES if prefill else LOWRANK_SOURCES if lowrank else KERNEL_SOURCES):
        with open(p, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    h.update(" ".join(gdn_build.HIPFLAGS).encode())
    return h.hexdigest()[:16]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--state-dtype", default="f32", choices=["f32", "bf16", "f16"])
    ap.add_argument("--layers", type=int, default=0, help="layer buffers rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle sample time")
    ap.add_argument("--cpu-threads", type=int, default=1,
                    help="host threads for the oracle sample (sequences split over a pool)")
    ap.add_argument("--graph-groups", type=int, default=7, help="graph-replay groups (0 = skip)")
    ap.add_argument("--graph-replays", type=int, default=400, help="launches per graph replay")
    ap.add_argument("--sequential", action="store_true",
                    help="prompt workloads: time gdn_decode_step (token by token) instead of gdn_prefill")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------- bytes


def algorithmic_bytes(spec: dict, state_dtype: str) -> int:
    """Bytes the step must move once: state read + written, per-token vectors, outputs."""
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    sb = 4 if state_dtype == "f32" else 2
    if spec.get("lowrank"):
        # the window read once (U, K, weights, pos); the slots written (one per token, at most
        # r), every weight and pos written back; the per-token vectors and o
        r, ab = spec["r"], 4 if spec["act"] == "f32" else 2
        read = B * H * (2 * r * D * sb + 4 * r + 4)
        write = B * H * (min(T, r) * 2 * D * sb + 4 * r + 4)
        return read + write + B * T * H * (3 * D * ab + 8 + D * ab)
    state = 2 * B * H * D * D * sb
    if spec.get("verify"):
        from gated_deltanet_recurrent_02_amd import synth
        ab = 4 if spec["act"] == "f32" else 2
        n_acc = int(synth.accepted_prefix(B, T).sum())  # committed tokens over the batch
        new = B * T * H * (3 * D * ab + 8 + D * ab + D * 4)       # q k v, gates, o, dk_out
        prev = n_acc * H * (D * ab + 4 + D * 4)                    # k, alpha, dk of the prefix
        return state + new + prev + B * 4
    if spec.get("fused"):
        C = 3 * H * D
        return (state + B * T * C * 2          # qkv in
                + 2 * B * C * 3 * 2            # conv state read + write
                + C * 4 * 4                    # conv weights
                + 2 * B * T * H * 4            # gate logits
                + B * T * H * D * 2)           # o
    ab = 4 if spec["act"] == "f32" else 2
    return state + B * T * H * (3 * D * ab + 8 + D * ab)


def flops(spec: dict) -> int:
    """Arithmetic of the recurrence: u = S k, S q (2 x 2D^2), update (2D^2), k.q, delta, o.
    On the low-rank window: K k, K q (2 x 2rD), k.q, the two sums over slots (2 x 2rD)."""
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    if spec.get("lowrank"):
        return B * H * T * (8 * spec["r"] * D + 6 * D)
    return B * H * T * (6 * D * D + 6 * D)


def read_traffic(workload: str, state_dtype: str, prefill: bool = False, lowrank: bool = False):
    """Measured HBM bytes per launch from profiles/traffic_<workload>_<state>.txt, if the
    kernel source still hashes to the value recorded there; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}_{state_dtype}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(prefill, lowrank):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- GPU timing


def time_gpu(args, spec, workload):
    import torch

    import gated_deltanet_recurrent_02_amd as gdn
    from gated_deltanet_recurrent_02_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fused = spec.get("fused", False)
    lowrank = spec.get("lowrank", False)
    state_keys = ("U", "K", "c", "pos") if lowrank else ("state",)
    x = synth.workload_inputs(workload, state_dtype=args.state_dtype)
    x_B, x_T = x["B"], x["T"]
    state_bytes = sum(x[n].numel() * x[n].element_size() for n in state_keys)
    layer_bytes = sum(v.numel() * v.element_size() for v in x.values() if isinstance(v, torch.Tensor))
    L = args.layers or max(1, math.ceil(2 * MALL_BYTES / layer_bytes))
    L = min(L, 64)
    print(f"[bench] {workload} state={args.state_dtype} layers={L} "
          f"state_bytes={state_bytes} layer_bytes={layer_bytes}", file=sys.stderr, flush=True)
    layers = []
    for i in range(L):
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        if i > 0:  # every layer has its own state; copies of the same draw are enough
            for n in state_keys:
                g[n] = g[n].clone()
        if fused:
            g["o"] = torch.empty((x["B"], x["T"], x["H"], x["D"]), dtype=torch.bfloat16, device=dev)
        else:
            g["o"] = torch.empty_like(g["v"])
        layers.append(g)
    del x

    if spec.get("verify"):
        n_acc = synth.accepted_prefix(x_B, x_T).to(dev)
        for g in layers:
            g["dk"] = [torch.zeros(g["v"].shape, dtype=torch.float32, device=dev) for _ in range(2)]
            g["i"] = 0

        def step(g):
            # each round commits the previous round's accepted prefix (same token tensors)
            j = g["i"] & 1
            gdn.decode_verify(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"],
                              prev=(n_acc, g["k"], g["alpha"], g["dk"][1 - j]), o=g["o"],
                              dk_out=g["dk"][j])
            g["i"] += 1
    elif spec.get("prefill") and not args.sequential:
        ws = gdn.prefill_workspace(layers[0]["q"], layers[0]["v"])  # launches are serialised

        def step(g):
            gdn.prefill(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], o=g["o"],
                        workspace=ws)
    elif lowrank:
        def step(g):
            gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                    g["c"], g["pos"], o=g["o"])
    elif fused:
        def step(g):
            gdn.conv_gate_decode(g["qkv"], g["conv_state"], g["conv_w"], g["conv_b"], g["a_logit"],
                                 g["b_logit"], g["state"], o=g["o"])
    else:
        def step(g):
            gdn.decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], o=g["o"])

    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        step(layers[i % L])
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(layers[i % L])
    end.record(stream)
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)

    extra = {}
    if args.graph_groups > 0:
        # The same launches replayed from a HIP graph: median over groups of the mean per
        # launch, each group one replay of `graph_replays` captured launches.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.graph_replays):
                step(layers[i % L])
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(args.graph_groups):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(torch.cuda.current_stream(dev))
            g.replay()
            e1.record(torch.cuda.current_stream(dev))
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / args.graph_replays)
        per.sort()
        extra["graph_median_us"] = per[len(per) // 2] * 1e3
        # spread over the groups: nearest-rank 10th and 90th percentiles of the group means
        extra["graph_p10_us"] = per[max(0, math.ceil(0.1 * len(per)) - 1)] * 1e3
        extra["graph_p90_us"] = per[max(0, math.ceil(0.9 * len(per)) - 1)] * 1e3
        extra["graph_protocol"] = f"median of {args.graph_groups} graph replays x {args.graph_replays} launches"
        del g
    # Plain device copy of the same number of state bytes: the read+write ceiling of this machine.
    src = layers[0][state_keys[0]]
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(50):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    nb = 2 * src.numel() * src.element_size()
    extra["copy_gbps_same_bytes"] = nb / (e0.elapsed_time(e1) / 50 * 1e-3) / 1e9
    return ms_total / args.steps, L, extra


def time_copy(args, mb: int):
    import torch
    dev = torch.device("cuda:0")
    n = (mb << 20) // 4
    L = max(2, math.ceil(2 * MALL_BYTES / (n * 4)))
    src = [torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(L)]
    dst = [torch.empty_like(s) for s in src]
    for i in range(args.warmup):
        dst[i % L].copy_(src[i % L])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        dst[i % L].copy_(src[i % L])
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / args.steps, 2 * n * 4


# ----------------------------------------------------------------------------- CPU baseline


def cpu_baseline(spec: dict, workload: str, state_dtype: str, target_s: float, threads: int = 1):
    """The fp64 oracle, untuned, on a bounded sample: the first few sequences of the same
    workload (all heads), repeated until about `target_s` seconds; scaled to one layer. With
    threads > 1 the sample's sequences are split over a thread pool (the C oracle runs outside
    the GIL), one oracle call per sequence."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from gated_deltanet_recurrent_02_amd import synth

    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    Bs = max(1, min(B, max(8, threads)))
    threads = max(1, min(threads, Bs))  # one sequence per call: no more threads than sequences
    Ts = T
    if spec.get("prefill"):  # the oracle's time is linear in T: a prefix of one prompt
        Bs, Ts = 1, min(T, 256)
    x = synth.workload_inputs(workload, state_dtype=state_dtype, B=Bs, T=Ts)
    f = lambda t: t.double().numpy()
    if spec.get("lowrank"):
        names = ("q", "k", "v", "alpha", "beta", "U", "K", "c")
        full = {n: f(x[n]) for n in names}
        full["pos"] = x["pos"].numpy()
        one = lambda sl: oracle.gdn_lowrank_decode(*(full[n][sl] for n in names + ("pos",)))
    elif spec.get("fused"):
        names = ("qkv", "conv_state", "a_logit", "b_logit", "state")
        full = {n: f(x[n]) for n in names}
        w = f(x["conv_w"])
        one = lambda sl: oracle.gdn_conv_gate_decode(
            full["qkv"][sl], full["conv_state"][sl], w, None, full["a_logit"][sl],
            full["b_logit"][sl], full["state"][sl], H=H, dk=D, dv=D)
    else:
        names = ("q", "k", "v", "alpha", "beta", "state")
        full = {n: f(x[n]) for n in names}
        one = lambda sl: oracle.gdn_decode(*(full[n][sl] for n in names))
    if threads == 1:
        run = lambda: one(slice(0, Bs))
    else:
        pool = ThreadPoolExecutor(threads)
        run = lambda: list(pool.map(one, [slice(b, b + 1) for b in range(Bs)]))
    oracle.load()
    run()
    reps, t0 = 0, time.perf_counter()
    while True:
        run()
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
    per_rep = el / reps
    us_per_layer = per_rep * (B / Bs) * (T / Ts) * 1e6
    scaled = f"{B}/{Bs}" + (f" x {T}/{Ts} tokens" if Ts != T else "")
    how = "single-thread" if threads == 1 else f"{threads} threads (one sequence per call)"
    return {"value": us_per_layer, "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"{Bs} of {B} sequences x {H} heads (D={D}, T={Ts} of {T}), fp64 "
                      f"{how} C oracle, {reps} repetitions in {el:.1f} s, scaled by {scaled}",
            "host_cpus": os.cpu_count()}


# ----------------------------------------------------------------------------- main


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no cross-GPU step; see the sharding note in the design document)",
              file=sys.stderr)
        return 2

    if args.workload.startswith("copy_"):
        mb = int(args.workload.split("_", 1)[1])
        ms, nbytes = time_copy(args, mb)
        gbps = nbytes / (ms * 1e-3) / 1e9
        print(json.dumps({"metric": "device copy GB/s (read + write)", "value": gbps, "unit": "GB/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                          "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
                          "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                          "config": {"workload": args.workload, "bytes_per_copy": nbytes}}))
        return 0

    from gated_deltanet_recurrent_02_amd import synth
    spec = dict(synth.WORKLOADS[args.workload])
    chunked = bool(spec.get("prefill")) and not args.sequential
    lowrank = bool(spec.get("lowrank"))
    ms, L, extra = time_gpu(args, spec, args.workload)
    us = ms * 1e3
    nbytes = algorithmic_bytes(spec, args.state_dtype)
    gbps = nbytes / (ms * 1e-3) / 1e9
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    act = "bf16" if spec.get("fused") else spec["act"]
    line = {
        "metric": METRIC, "value": us, "unit": "us/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "dk": D, "dv": D, "T": T,
                   "state_dtype": args.state_dtype, "act_dtype": act,
                   "entry_point": ("gdn_conv_gate_decode" if spec.get("fused") else
                                   "gdn_lowrank_decode_step" if lowrank else
                                   "gdn_decode_verify" if spec.get("verify") else
                                   "gdn_prefill" if spec.get("prefill") and not args.sequential else
                                   "gdn_decode_step"),
                   "layers_rotated": L, **({"r": spec["r"]} if lowrank else {})},
        "achieved_gbps": gbps,
        "seq_tokens_per_s": B * T / (ms * 1e-3),
        "us_per_token_48_layers": us * 48,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS,
                     "traffic": read_traffic(args.workload, args.state_dtype, chunked, lowrank),
                     "algorithmic_bytes_per_launch": nbytes,
                     "kernel_source_sha256_16": kernel_source_hash(chunked, lowrank)},
        "gflops": flops(spec) / (ms * 1e-3) / 1e9,
    }
    line.update(extra)
    line["frac_of_copy_bw"] = gbps / extra["copy_gbps_same_bytes"]
    if chunked:
        # The chunked form is bound by fp32 matrix-core arithmetic, not by HBM: price the
        # recurrence's flops (per token and head: S k, S q and the rank-1 update, 6 D^2) against
        # the fp32 MFMA peak. The time is the whole call (prep kernel + state kernel).
        tf = flops(spec) / (ms * 1e-3) / 1e12
        line["roofline_hbm"] = line["roofline"]
        line["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_FP32_MFMA_TFLOPS,
                            "unit": "TFLOP/s", "frac": tf / PEAK_FP32_MFMA_TFLOPS,
                            "traffic": line["roofline_hbm"]["traffic"],
                            "algorithmic_flops_per_launch": flops(spec),
                            "timed": "whole gdn_prefill call (prep + state kernels)"}
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(spec, args.workload, args.state_dtype, args.cpu_seconds,
                                            args.cpu_threads)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
