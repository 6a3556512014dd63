"""Benchmark of the GDN recurrent decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--state-dtype S]
                    [--no-cpu-baseline] [--no-extra]
    python bench.py --profile-commands --workload NAME [--state-dtype S] [--profile-root DIR]
    python bench.py --summarize DIR --workload NAME [--state-dtype S]

A step is one layer's call of the hot path over one batch of seeded synthetic input that is
already resident in HBM: gdn_decode_step for the decode workloads (state read once, T tokens,
state written once), gdn_conv_gate_decode for the fused one, gdn_decode_verify for the verify
rounds, gdn_prefill for the prompt workload (`--sequential` runs that workload through
gdn_decode_step instead) and gdn_lowrank_decode_step for the low-rank window workloads. Layer
buffers (state, inputs, outputs) are rotated so that the state a step reads was not left in
the 256 MB MALL by the previous step. W untimed steps, the last of them queued behind a device
synchronisation so that the GPU is already busy when the first timed step starts, then K timed
steps; the HIP events that time them are recorded on the stream the kernels are launched on,
and a device synchronisation closes the timed region. Before that, the same launches are
replayed from a HIP graph (median of 7 groups x 400 launches), which also brings the GPU's
clocks to their steady state under the workload before the timed steps.

Prints ONE JSON line. `value` is microseconds per layer step of the workload (lower is better);
`roofline` prices the dominant kernel's algorithmic bytes per launch against MI355X's 8 TB/s
HBM peak (the prompt workload: its arithmetic against the matrix-core peaks); `traffic` is the
measured HBM bytes per launch from a committed rocprofv3 counter summary, or null if the kernel
source changed since it was taken; `cpu_baseline` times the fp64 oracle on a bounded sample of
the same workload on all the host's cores and on one. The default workload's line also carries
`configs`: the other workloads (single stream, mid batch, 16-bit state, fused layer path,
multi-token, verify, prefill, low-rank window) and the in-place stream probe, each with its
own timing and roofline fraction.

Other workloads:
  copy_<MB>     a plain device-to-device copy of that many MB (torch's copy kernel): the
                calibration of the counter-based traffic figures.
  probe_<name>  the in-place stream probe (libgdn_probe.so) over the state of workload <name>:
                the decode kernels' state access pattern with no arithmetic, i.e. the
                practical ceiling of their read-modify-write stream (`--probe-variant`,
                `--probe-group` select the geometry and workgroup order).

`--profile-commands` prints the rocprofv3 command of every profiling pass the summary of a
workload is made from (one per line, `name<TAB>command`); `--summarize DIR` reads the CSV
files those commands wrote under DIR and writes profiles/<kernel>_<workload>_<state>.md and
profiles/traffic_<workload>_<state>.txt.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN decode µs/layer + achieved HBM GB/s (% roofline), B=256 H=48 128×128"
DEFAULT_WORKLOAD = "decode_b256_h48_d128_t1"
PEAK_HBM_GBPS = 8000.0
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
MAX_ROTATION_BYTES = 16 << 30    # device memory the rotated layer buffers may take
HOST_CPU_SHARE = 16              # host cores one GPU's jobs may use
PROFILES = os.path.join(ROOT, "profiles")
_PKG = os.path.join(ROOT, "gated_deltanet_recurrent_02_amd")
_CSRC = os.path.join(_PKG, "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in ("gdn_kernels.hip", "gdn_launch.h")]
PREFILL_SOURCES = [os.path.join(_CSRC, f)
                   for f in ("gdn_prefill.hip", "gdn_prefill_launch.h", "gdn_launch.h")]
LOWRANK_SOURCES = [os.path.join(_CSRC, f)
                   for f in ("gdn_lowrank.hip", "gdn_lowrank_launch.h", "gdn_launch.h")]
PROBE_SOURCES = [os.path.join(_CSRC, "gdn_stream_probe.hip")]
PROBE_LIBRARY = os.path.join(_PKG, "libgdn_probe.so")

# Extra workloads timed with the default one: (label, workload, state dtype).
EXTRA_CONFIGS = [
    ("single_stream_b1_f32", "decode_b1_h48_d128_t1", "f32"),
    # the same single stream over 48 layers (one token's pass through a 48-layer model: 151 MB
    # of state, which the 256 MB MALL can hold) and hot (one layer, cache-resident), labelled
    ("single_stream_b1_f32_48_layers", "decode_b1_h48_d128_t1", "f32", {"layers": 48}),
    ("single_stream_b1_f32_hot", "decode_b1_h48_d128_t1", "f32", {"layers": 1}),
    ("mid_batch_b64_f32", "decode_b64_h48_d128_t1", "f32"),
    ("bottleneck_b256_bf16_state", "decode_b256_h48_d128_t1", "bf16"),
    ("fused_b256_t4_f32", "fused_b256_h48_d128_t4", "f32"),
    ("decode_b256_t4_f32", "decode_b256_h48_d128_t4", "f32"),
    ("verify_b256_t4_f32", "verify_b256_h48_d128_t4", "f32"),
    # bf16 states with bf16 activations take the chunk form for these calls
    ("decode_b256_t4_bf16_state", "decode_b256_h48_d128_t4", "bf16"),
    ("verify_b256_t4_bf16_state", "verify_b256_h48_d128_t4", "bf16"),
    ("prefill_b4_t4096_f32", "prefill_b4_h48_d128_t4096", "f32"),
    ("lowrank_b256_r16_t1_f32", "lowrank_b256_h48_d128_r16_t1", "f32"),
    ("lowrank_b256_r16_t4_bf16", "lowrank_b256_h48_d128_r16_t4", "bf16"),
    ("lowrank_b256_r32_t8_bf16", "lowrank_b256_h48_d128_r32_t8", "bf16"),
    ("stream_probe_b256_f32", "probe_decode_b256_h48_d128_t1", "f32"),
    # the fastest in-place stream geometry of a sweep over 11 geometries x 5 XCD orders
    # (4 rows per one-wave workgroup, runs of 2 tiles per XCD)
    ("stream_probe_best_b256_f32", "probe_decode_b256_h48_d128_t1", "f32", {"probe_variant": 4, "probe_group": 2}),
]


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


def workload_kind(workload: str, sequential: bool = False) -> str:
    """decode | fused | verify | prefill (chunked) | lowrank | probe | copy."""
    if workload.startswith("copy_"):
        return "copy"
    if workload.startswith("probe_"):
        return "probe"
    from gated_deltanet_recurrent_02_amd import synth
    spec = synth.WORKLOADS[workload]
    for k in ("fused", "verify", "lowrank"):
        if spec.get(k):
            return k
    if spec.get("prefill") and not sequential:
        return "prefill"
    return "decode"


def kernel_source_hash(kind: str = "decode") -> str:
    """Hash of the code a workload runs: its kernel sources as code_text, plus the compiler
    flags they are built with."""
    from gated_deltanet_recurrent_02_amd import build as gdn_build
    srcs = {"prefill": PREFILL_SOURCES, "lowrank": LOWRANK_SOURCES,
            "probe": PROBE_SOURCES}.get(kind, KERNEL_SOURCES)
    h = hashlib.sha256()
    for p in srcs:
        with open(p, encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    h.update(" ".join(gdn_build.HIPFLAGS).encode())
    return h.hexdigest()[:16]


ENTRY_POINTS = {"decode": "gdn_decode_step", "fused": "gdn_conv_gate_decode",
                "verify": "gdn_decode_verify", "prefill": "gdn_prefill",
                "lowrank": "gdn_lowrank_decode_step", "probe": "gdn_stream_probe"}
KERNEL_NAMES = {"decode": ["gdn_decode_"], "fused": ["gdn_conv_gate_decode_kernel"],
                "verify": ["gdn_verify_"],
                "prefill": ["gdn_prefill_prep_kernel", "gdn_prefill_state_kernel"],
                "lowrank": ["gdn_lowrank_"], "probe": ["gdn_stream_probe_kernel"]}
PROFILE_PREFIX = {"decode": "gdn_decode_kernel", "fused": "gdn_conv_gate_decode_kernel",
                  "verify": "gdn_verify_kernel", "prefill": "gdn_prefill",
                  "lowrank": "gdn_lowrank_kernel", "probe": "gdn_stream_probe_kernel"}


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--state-dtype", default="f32", choices=["f32", "bf16", "f16"])
    ap.add_argument("--layers", type=int, default=0, help="layer buffers rotated (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload: skip the extra configs")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle sample time")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads for the all-cores oracle sample (0 = the host's share)")
    ap.add_argument("--graph-groups", type=int, default=7, help="graph-replay groups (0 = skip)")
    ap.add_argument("--graph-replays", type=int, default=400, help="launches per graph replay")
    ap.add_argument("--sequential", action="store_true",
                    help="prompt workloads: time gdn_decode_step (token by token) instead of gdn_prefill")
    ap.add_argument("--probe-variant", type=int, default=-1,
                    help="probe_ workloads: geometry (-1 = that of the base workload's one-token "
                         "decode: 0 for a 4-byte state, 2 for a 2-byte state)")
    ap.add_argument("--probe-group", type=int, default=0,
                    help="probe_ workloads: consecutive tiles per XCD (0 = the decode kernel's own "
                         "order: 4 from 8192 heads and 16 below for a 4-byte state, 1 for 2-byte)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="write profiles/ summaries from the rocprofv3 CSVs under DIR")
    ap.add_argument("--profile-commands", action="store_true",
                    help="print the rocprofv3 passes of --workload and exit")
    ap.add_argument("--profile-root", default="gpurun_out",
                    help="--profile-commands: directory the passes write to")
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


def probe_bytes(spec: dict, state_dtype: str) -> int:
    """The probe moves the base workload's state once each way and nothing else."""
    sb = 4 if state_dtype == "f32" else 2
    return 2 * spec["B"] * spec["H"] * spec["D"] * spec["D"] * sb


def flops(spec: dict) -> int:
    """Arithmetic of the recurrence: u = S k, S q (2 x 2D^2), update (2D^2), k.q, delta, o.
    On the low-rank window: K k, K q (2 x 2rD), k.q, the two sums over slots (2 x 2rD)."""
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    if spec.get("lowrank"):
        return B * H * T * (8 * spec["r"] * D + 6 * D)
    return B * H * T * (6 * D * D + 6 * D)


PREFILL_CHUNK = 16


def prefill_matrix_flop(spec: dict) -> dict:
    """Matrix-core arithmetic one gdn_prefill call issues (bf16 activations, chunks of 16
    tokens taken in pairs, D = dk = dv), per head and chunk:
      K S'^T on three bf16 parts of S', Q S'^T on two     (3 + 2) x 16 x D x D x 2   bf16
      the state update on three bf16 parts of its factors 3 x D x 16 x D x 2         bf16
      K Q^T, the prep's K K^T, and per pair K1 K0^T and Q1 K0^T (one per chunk)
                                                          3 x 16 x 16 x D x 2        bf16
      T Z, P Delta, and per pair the two corrections through Delta0 (one per chunk)
                                                          3 x 16 x 16 x D x 2        fp32
    Returns bf16 and fp32 flop per call."""
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    C = PREFILL_CHUNK
    chunks = B * H * math.ceil(T / C)
    bf16 = chunks * ((3 + 2) * C * D * D * 2 + 3 * D * C * D * 2 + 3 * C * C * D * 2)
    f32 = chunks * (3 * C * C * D * 2)
    return {"bf16": bf16, "f32": f32}


def read_traffic(workload: str, state_dtype: str, kind: str):
    """Measured HBM bytes per launch from profiles/traffic_<workload>_<state>.txt, if the
    kernel source still hashes to the value recorded there; else None."""
    path = os.path.join(PROFILES, f"traffic_{workload}_{state_dtype}.txt")
    if not os.path.exists(path):
        return None
    kv = read_kv(path)
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(kind):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_kv(path: str) -> dict:
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


# ----------------------------------------------------------------------------- GPU timing


def _probe_lib():
    import ctypes
    if not os.path.exists(PROBE_LIBRARY):
        raise ImportError(f"{PROBE_LIBRARY} is missing: build it with "
                          "`python -m gated_deltanet_recurrent_02_amd.build`")
    L = ctypes.CDLL(PROBE_LIBRARY)
    L.gdn_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_uint32, ctypes.c_void_p]
    L.gdn_stream_probe.restype = ctypes.c_int
    return L


def time_gpu(args, workload: str, state_dtype: str, copy_ceiling: bool = False) -> dict:
    """Time `args.steps` launches of a workload after `args.warmup` untimed ones, plus the
    graph-replay protocol. Returns ms per step, layers rotated and the graph statistics."""
    import ctypes

    import torch

    import gated_deltanet_recurrent_02_amd as gdn
    from gated_deltanet_recurrent_02_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kind = workload_kind(workload, args.sequential)
    if kind == "probe":
        base = workload[len("probe_"):]
        spec = synth.WORKLOADS[base]
        heads = spec["B"] * spec["H"]
        dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[state_dtype]
        x = {"state": torch.empty((spec["B"], spec["H"], spec["D"], spec["D"]), dtype=dt)}
        x["state"].view(torch.uint8 if dt != torch.float32 else torch.int32).random_(0, 100)
        state_keys = ("state",)
    else:
        spec = synth.WORKLOADS[workload]
        x = synth.workload_inputs(workload, state_dtype=state_dtype)
        state_keys = ("U", "K", "c", "pos") if kind == "lowrank" else ("state",)
    state_bytes = sum(x[n].numel() * x[n].element_size() for n in state_keys)
    layer_bytes = sum(v.numel() * v.element_size() for v in x.values() if isinstance(v, torch.Tensor))
    L = args.layers or max(1, math.ceil(2 * MALL_BYTES / layer_bytes))
    L = max(1, min(L, MAX_ROTATION_BYTES // layer_bytes, 1024))
    print(f"[bench] {workload} state={state_dtype} layers={L} "
          f"state_bytes={state_bytes} layer_bytes={layer_bytes}", file=sys.stderr, flush=True)
    layers = []
    for i in range(L):
        g = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
        if i > 0:  # every layer has its own state; copies of the same draw are enough
            for n in state_keys:
                g[n] = g[n].clone()
        if kind == "fused":
            g["o"] = torch.empty((x["B"], x["T"], x["H"], x["D"]), dtype=torch.bfloat16, device=dev)
        elif kind != "probe":
            g["o"] = torch.empty_like(g["v"])
        layers.append(g)
    x_B, x_T = spec["B"], spec["T"]
    del x

    if kind == "probe":
        plib = _probe_lib()
        variant = args.probe_variant if args.probe_variant >= 0 else (0 if state_dtype == "f32" else 2)
        group = args.probe_group or (1 if variant == 2 else (4 if heads >= 8192 else 16))

        def step(g):
            st = g["state"]
            rc = plib.gdn_stream_probe(ctypes.c_void_p(st.data_ptr()), st.numel() * st.element_size(),
                                       heads, variant, group,
                                       ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
            if rc != 0:
                raise RuntimeError(f"gdn_stream_probe failed ({rc})")
    elif kind == "verify":
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
    elif kind == "prefill":
        ws = gdn.prefill_workspace(layers[0]["q"], layers[0]["v"])  # launches are serialised

        def step(g):
            gdn.prefill(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], o=g["o"],
                        workspace=ws)
    elif kind == "lowrank":
        def step(g):
            gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                    g["c"], g["pos"], o=g["o"])
    elif kind == "fused":
        def step(g):
            gdn.conv_gate_decode(g["qkv"], g["conv_state"], g["conv_w"], g["conv_b"], g["a_logit"],
                                 g["b_logit"], g["state"], o=g["o"])
    else:
        def step(g):
            gdn.decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], o=g["o"])

    stream = torch.cuda.current_stream(dev)
    out = {"layers": L}
    if args.graph_groups > 0:
        # The same launches replayed from a HIP graph: median over groups of the mean per
        # launch, each group one replay of `graph_replays` captured launches. Run first, so
        # that the GPU's clocks have settled under this load before the timed steps below.
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
        out["graph_median_us"] = per[len(per) // 2] * 1e3
        # spread over the groups: nearest-rank 10th and 90th percentiles of the group means
        out["graph_p10_us"] = per[max(0, math.ceil(0.1 * len(per)) - 1)] * 1e3
        out["graph_p90_us"] = per[max(0, math.ceil(0.9 * len(per)) - 1)] * 1e3
        out["graph_protocol"] = f"median of {args.graph_groups} graph replays x {args.graph_replays} launches"
        del g
    # Warm-up: all but the last `pre` steps, a device synchronisation, then `pre` steps queued
    # right before the start event, so the first timed step starts on a busy GPU (no idle gap
    # while the host issues it).
    pre = min(args.warmup, 2)
    for i in range(args.warmup - pre):
        step(layers[i % L])
    torch.cuda.synchronize()
    for i in range(args.warmup - pre, args.warmup):
        step(layers[i % L])
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(layers[(args.warmup + i) % L])
    end.record(stream)
    torch.cuda.synchronize()
    out["ms"] = start.elapsed_time(end) / args.steps

    if copy_ceiling:
        # Plain device copy of the same number of state bytes: the read+write ceiling of a copy.
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
        out["copy_gbps_same_bytes"] = nb / (e0.elapsed_time(e1) / 50 * 1e-3) / 1e9
        del dst
    del layers
    torch.cuda.empty_cache()
    return out


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


def measure(args, workload: str, state_dtype: str, copy_ceiling: bool = False) -> dict:
    """Time a workload and price it: µs per step, algorithmic GB/s and the roofline object."""
    from gated_deltanet_recurrent_02_amd import synth
    kind = workload_kind(workload, args.sequential)
    t = time_gpu(args, workload, state_dtype, copy_ceiling)
    ms = t["ms"]
    if kind == "probe":
        spec = synth.WORKLOADS[workload[len("probe_"):]]
        nbytes = probe_bytes(spec, state_dtype)
    else:
        spec = synth.WORKLOADS[workload]
        nbytes = algorithmic_bytes(spec, state_dtype)
    gbps = nbytes / (ms * 1e-3) / 1e9
    r = {"workload": workload, "state_dtype": state_dtype, "kind": kind, "spec": spec,
         "entry_point": ENTRY_POINTS[kind], "us": ms * 1e3, "ms": ms, "layers": t["layers"],
         "gbps": gbps, "nbytes": nbytes,
         "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": gbps / PEAK_HBM_GBPS,
                      "traffic": read_traffic(workload, state_dtype, kind),
                      "algorithmic_bytes_per_launch": nbytes,
                      "kernel_source_sha256_16": kernel_source_hash(kind)}}
    r.update({k: v for k, v in t.items() if k not in ("ms", "layers")})
    if kind == "prefill":
        # The chunked form is bound by matrix-core and vector issue, not by HBM. The method's
        # arithmetic (6 D^2 per token and head: S k, S q and the rank-1 update) is priced
        # against the fp32 matrix peak (the precision the results carry) and against the bf16
        # dense peak of the instructions that actually run; the matrix-core flop the chunked
        # form issues (three bf16 parts per fp32 operand) against the bf16 peak as well.
        sec = ms * 1e-3
        tf = flops(spec) / sec / 1e12
        mf = prefill_matrix_flop(spec)
        issued_bf16 = mf["bf16"] / sec / 1e12
        r["roofline_hbm"] = r["roofline"]
        r["roofline"] = {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_MFMA_TFLOPS,
                         "unit": "TFLOP/s", "frac": tf / PEAK_BF16_MFMA_TFLOPS,
                         "traffic": r["roofline_hbm"]["traffic"],
                         "algorithmic_flops_per_launch": flops(spec),
                         "frac_of_fp32_matrix_peak": tf / PEAK_FP32_MFMA_TFLOPS,
                         "issued_bf16_flops_per_launch": mf["bf16"],
                         "issued_bf16_tflops": issued_bf16,
                         "issued_frac_of_bf16_peak": issued_bf16 / PEAK_BF16_MFMA_TFLOPS,
                         "issued_fp32_flops_per_launch": mf["f32"],
                         "timed": "whole gdn_prefill call (prep + state kernels)"}
    return r


# ----------------------------------------------------------------------------- CPU baseline


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, HOST_CPU_SHARE))


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
        threads = 1
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
    pool = None
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
    if pool is not None:
        pool.shutdown()
    per_rep = el / reps
    us_per_layer = per_rep * (B / Bs) * (T / Ts) * 1e6
    scaled = f"{B}/{Bs}" + (f" x {T}/{Ts} tokens" if Ts != T else "")
    how = "single-thread" if threads == 1 else f"{threads} threads (one sequence per call)"
    return {"value": us_per_layer, "unit": "us/layer", "cores": threads, "kind": "oracle",
            "sample": f"{Bs} of {B} sequences x {H} heads (D={D}, T={Ts} of {T}), fp64 "
                      f"{how} C oracle, {reps} repetitions in {el:.1f} s, scaled by {scaled}",
            "host_cpus": os.cpu_count()}


# ----------------------------------------------------------------------------- profiles


def profile_commands(workload: str, state_dtype: str, root: str = "gpurun_out") -> list:
    """The rocprofv3 passes a profile summary is made from, as (name, shell command). Each
    command runs committed files only; the CSVs land under `root`."""
    tag = f"{workload}_{state_dtype}"
    b = f"python bench.py --workload {workload} --state-dtype {state_dtype} --no-cpu-baseline --no-extra"
    short = f"{b} --steps 5 --warmup 1 --graph-groups 0"

    def pmc(name, counters, cmd=short, out="k"):
        return (name, f"rocprofv3 --pmc {counters} -d {root}/prof_{name}_{tag} -o {out} "
                      f"--output-format csv -- {cmd}")

    return [
        ("bench", f"{b} > {root}/bench_{tag}.log"),
        ("trace", f"rocprofv3 --kernel-trace --stats -d {root}/prof_trace_{tag} -o k "
                  f"--output-format csv -- {b} --steps 200 --warmup 20"),
        pmc("fetch", "FETCH_SIZE"),
        pmc("write", "WRITE_SIZE"),
        pmc("req", "TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum "
                   "TCC_EA0_WRREQ_64B_sum"),
        pmc("wreq", "TCC_EA0_WRREQ_sum TCC_EA0_RDREQ_sum"),
        pmc("sq", "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_ACTIVE_INST_VALU "
                  "SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE"),
        pmc("vb", "VALUBusy MfmaUtil"),
    ]


def copy_calibration_commands(root: str = "gpurun_out") -> list:
    c = "python bench.py --workload copy_805 --steps 5 --warmup 1"
    return [("copy_fetch", f"rocprofv3 --pmc FETCH_SIZE -d {root}/prof_copy_fetch -o copy --output-format csv -- {c}"),
            ("copy_write", f"rocprofv3 --pmc WRITE_SIZE -d {root}/prof_copy_write -o copy --output-format csv -- {c}")]


COPY_CAL_BYTES = ((805 << 20) // 4) * 4   # bytes read (= bytes written) by one copy_805 copy


def _rows(path: str) -> list:
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counters(path: str, names: list) -> dict:
    """Per kernel (matched by substring) and counter: the mean value over its dispatches, the
    dispatch count, and the kernel's register/LDS resources."""
    out = {}
    if not os.path.exists(path):
        return out
    for r in _rows(path):
        for k in names:
            if k in r["Kernel_Name"]:
                d = out.setdefault(k, {"values": {}, "res": {}})
                d["values"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                d["res"] = {"vgpr": r.get("VGPR_Count"), "agpr": r.get("Accum_VGPR_Count"),
                            "sgpr": r.get("SGPR_Count"), "lds": r.get("LDS_Block_Size"),
                            "wg": r.get("Workgroup_Size"), "grid": r.get("Grid_Size")}
    for d in out.values():
        d["n"] = {c: len(v) for c, v in d["values"].items()}
        d["mean"] = {c: statistics.mean(v) for c, v in d["values"].items()}
    return out


def _copy_counter(path: str) -> float | None:
    """Mean counter value of the largest kernel in a copy calibration run."""
    if not os.path.exists(path):
        return None
    by = {}
    for r in _rows(path):
        by.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return max(statistics.mean(v) for v in by.values()) if by else None


def summarize(root: str, workload: str, state_dtype: str, out_dir: str = PROFILES) -> str:
    """Write profiles/<kernel>_<workload>_<state>.md (and traffic_<workload>_<state>.txt when
    the traffic passes are present) from the CSVs the profile_commands passes wrote under
    `root`. Returns the summary's path."""
    from gated_deltanet_recurrent_02_amd import synth
    kind = workload_kind(workload)
    names = KERNEL_NAMES[kind]
    tag = f"{workload}_{state_dtype}"
    cmds = dict(profile_commands(workload, state_dtype, "gpurun_out"))
    cal = dict(copy_calibration_commands("gpurun_out"))
    spec = synth.WORKLOADS[workload[len("probe_"):] if kind == "probe" else workload]
    alg = probe_bytes(spec, state_dtype) if kind == "probe" else algorithmic_bytes(spec, state_dtype)
    lines = [f"# {workload}, {state_dtype} state: {ENTRY_POINTS[kind]} on MI355X", ""]
    # kernel trace
    trace = {}
    tp = os.path.join(root, f"prof_trace_{tag}", "k_kernel_stats.csv")
    for r in _rows(tp):
        for k in names:
            if k in r["Name"]:
                trace[k] = r
    missing = [k for k in names if k not in trace]
    if missing:
        raise ValueError(f"{tp}: no row for {missing}")
    import re
    disp = {}
    for k in names:
        m = re.search(r"(gdn_\w+?)(<|\()", trace[k]["Name"])
        disp[k] = m.group(1) if m else k
    lines += ["Kernels: " + "; ".join(f"`{trace[k]['Name']}`" for k in names), "",
              "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              f"Command: `{cmds['trace']}`", "",
              "| kernel | calls | average ns | min ns | max ns | stddev ns |", "|---|---|---|---|---|---|"]
    avg_ns = 0.0
    for k in names:
        r = trace[k]
        avg_ns += float(r["AverageNs"])
        lines.append(f"| {disp[k]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} | {float(r['StdDev']):.0f} |")
    lines.append("")
    per_launch_gbps = alg / (avg_ns * 1e-9) / 1e9
    lines.append(f"Per launch{' (sum of the kernels)' if len(names) > 1 else ''}: {avg_ns / 1e3:.1f} us; "
                 f"{alg} algorithmic bytes / that time = {per_launch_gbps:.0f} GB/s, "
                 f"{100 * per_launch_gbps / PEAK_HBM_GBPS:.1f}% of 8 TB/s.")
    bl = os.path.join(root, f"bench_{tag}.log")
    if os.path.exists(bl):
        js = [ln for ln in open(bl) if ln.startswith("{")]
        if js:
            b = json.loads(js[-1])
            lines += ["", f"`{cmds['bench'].split(' > ')[0]}` on the same build: {b['value']:.1f} us per "
                          f"launch (HIP events over {b['steps']} launches after {b['warmup']}), "
                          f"{b['achieved_gbps']:.0f} GB/s algorithmic, "
                          f"{100 * b['achieved_gbps'] / PEAK_HBM_GBPS:.1f}% of 8 TB/s; graph median "
                          f"{b.get('graph_median_us', float('nan')):.1f} us "
                          f"({b.get('graph_protocol', '')}); layers rotated {b['config'].get('layers_rotated')}."]
            if kind == "prefill":
                rf = b["roofline"]
                lines.append(f"Matrix-core view: {rf['achieved']:.1f} TFLOP/s of the method's arithmetic "
                             f"= {100 * rf['frac']:.1f}% of the 2.5 PFLOP/s bf16 dense peak "
                             f"({100 * rf['frac_of_fp32_matrix_peak']:.1f}% of the fp32 matrix peak); "
                             f"issued bf16 matrix flop {rf['issued_bf16_tflops']:.0f} TFLOP/s "
                             f"= {100 * rf['issued_frac_of_bf16_peak']:.1f}% of the bf16 peak.")
    lines.append("")
    # HBM traffic: FETCH_SIZE / WRITE_SIZE with the copy calibration
    fe = _counters(os.path.join(root, f"prof_fetch_{tag}", "k_counter_collection.csv"), names)
    wr = _counters(os.path.join(root, f"prof_write_{tag}", "k_counter_collection.csv"), names)
    cf = _copy_counter(os.path.join(root, "prof_copy_fetch", "copy_counter_collection.csv"))
    cw = _copy_counter(os.path.join(root, "prof_copy_write", "copy_counter_collection.csv"))
    hbm = None
    if all(k in fe and k in wr for k in names) and cf and cw:
        fscale = COPY_CAL_BYTES / (cf * 1024)
        wscale = COPY_CAL_BYTES / (cw * 1024)
        lines += ["## HBM traffic (rocprofv3 --pmc FETCH_SIZE, WRITE_SIZE; one counter per run)", "",
                  "Commands:", f"- `{cmds['fetch']}`", f"- `{cmds['write']}`",
                  f"- `{cal['copy_fetch']}`", f"- `{cal['copy_write']}`", "",
                  f"Calibration: one device copy of {COPY_CAL_BYTES} bytes reads FETCH_SIZE {cf:.1f} KiB "
                  f"and WRITE_SIZE {cw:.1f} KiB per dispatch, so bytes = FETCH_SIZE x {fscale:.4f} KiB "
                  f"and WRITE_SIZE x {wscale:.4f} KiB.", "",
                  "| kernel | FETCH_SIZE KiB (dispatches) | WRITE_SIZE KiB (dispatches) | scaled bytes |",
                  "|---|---|---|---|"]
        hbm = 0.0
        fk = wk = 0.0
        for k in names:
            f_ = fe[k]["mean"]["FETCH_SIZE"]
            w_ = wr[k]["mean"]["WRITE_SIZE"]
            fk += f_
            wk += w_
            by = f_ * 1024 * fscale + w_ * 1024 * wscale
            hbm += by
            lines.append(f"| {disp[k]} | {f_:.1f} ({fe[k]['n']['FETCH_SIZE']}) | {w_:.1f} "
                         f"({wr[k]['n']['WRITE_SIZE']}) | {by:.0f} |")
        lines += ["", f"Measured HBM bytes per launch {hbm:.0f} vs algorithmic {alg} "
                      f"({100 * (hbm / alg - 1):+.1f}%).", ""]
    # by request size
    rq = _counters(os.path.join(root, f"prof_req_{tag}", "k_counter_collection.csv"), names)
    wq = _counters(os.path.join(root, f"prof_wreq_{tag}", "k_counter_collection.csv"), names)
    req_bytes = None
    if all(k in rq and k in wq for k in names):
        lines += ["## HBM traffic by request size (rocprofv3 --pmc TCC_EA0_* request counters)", "",
                  "Commands:", f"- `{cmds['req']}`", f"- `{cmds['wreq']}`", "",
                  "Bytes read = 32 x RDREQ_32B + 64 x RDREQ_64B + 128 x RDREQ_128B; bytes written = "
                  "64 x WRREQ_64B + 32 x (WRREQ - WRREQ_64B). No calibration factor enters.", "",
                  "| kernel | RDREQ (32B / 64B / 128B) | RDREQ total | WRREQ (64B of total) | bytes read | bytes written |",
                  "|---|---|---|---|---|---|"]
        req_bytes = 0.0
        for k in names:
            m, n_ = rq[k]["mean"], wq[k]["mean"]
            r32, r64, r128 = (m["TCC_EA0_RDREQ_32B_sum"], m["TCC_EA0_RDREQ_64B_sum"],
                              m["TCC_EA0_RDREQ_128B_sum"])
            w64, wtot, rtot = m["TCC_EA0_WRREQ_64B_sum"], n_["TCC_EA0_WRREQ_sum"], n_["TCC_EA0_RDREQ_sum"]
            rb = 32 * r32 + 64 * r64 + 128 * r128
            wb = 64 * w64 + 32 * (wtot - w64)
            req_bytes += rb + wb
            lines.append(f"| {disp[k]} | {r32:.0f} / {r64:.0f} / {r128:.0f} | {rtot:.0f} | {w64:.0f} of "
                         f"{wtot:.0f} | {rb:.0f} | {wb:.0f} |")
        lines += ["", f"By request size: {req_bytes:.0f} bytes per launch vs algorithmic {alg} "
                      f"({100 * (req_bytes / alg - 1):+.1f}%).", ""]
    # instruction counters
    sq = _counters(os.path.join(root, f"prof_sq_{tag}", "k_counter_collection.csv"), names)
    vb = _counters(os.path.join(root, f"prof_vb_{tag}", "k_counter_collection.csv"), names)
    if all(k in sq for k in names):
        lines += ["## Instruction counters (rocprofv3 --pmc)", "", "Commands:", f"- `{cmds['sq']}`",
                  f"- `{cmds['vb']}`", "",
                  "GRBM_GUI_ACTIVE is summed over the 8 XCDs (/8 = cycles of the dispatch). VALU busy = "
                  "SQ_ACTIVE_INST_VALU / (256 CUs x cycles); MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
                  "(1024 SIMDs x cycles); the derived VALUBusy and MfmaUtil are rocprofv3's own figures.", "",
                  "| kernel | waves | VALU instrs / wave | MFMA instrs / wave | VALU busy % | MFMA busy % | "
                  "wait / wave cycles | VALUBusy | MfmaUtil | VGPR (AGPR) | SGPR | LDS B | wg size |",
                  "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
        for k in names:
            m = sq[k]["mean"]
            waves = m["SQ_WAVES"]
            cyc = m["GRBM_GUI_ACTIVE"] / 8
            v = vb.get(k, {}).get("mean", {})
            res = sq[k]["res"]
            lines.append(
                f"| {disp[k]} | {waves:.0f} | {m['SQ_INSTS_VALU'] / waves:.1f} | {m['SQ_INSTS_MFMA'] / waves:.1f} | "
                f"{100 * m['SQ_ACTIVE_INST_VALU'] / (256 * cyc):.1f} | "
                f"{100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cyc):.1f} | "
                f"{m['SQ_WAIT_INST_ANY'] / max(1.0, m['SQ_WAVE_CYCLES']):.2f} | "
                f"{v.get('VALUBusy', float('nan')):.1f} | {v.get('MfmaUtil', float('nan')):.1f} | "
                f"{res['vgpr']} ({res['agpr']}) | {res['sgpr']} | {res['lds']} | {res['wg']} |")
        lines.append("")
    os.makedirs(out_dir, exist_ok=True)
    # a decode or verify workload runs one of two kernels (token by token, or the chunk form):
    # the file is named for the one that ran
    prefix = disp[names[0]] if kind in ("decode", "verify") else PROFILE_PREFIX[kind]
    path = os.path.join(out_dir, f"{prefix}_{tag}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines).rstrip() + "\n")
    if hbm is not None:
        with open(os.path.join(out_dir, f"traffic_{tag}.txt"), "w") as f:
            f.write(f"# HBM traffic per launch of the {workload} kernels ({state_dtype} state), from\n"
                    f"# rocprofv3 FETCH_SIZE/WRITE_SIZE scaled by a device-copy calibration.\n"
                    f"workload: {workload}\nstate_dtype: {state_dtype}\n"
                    f"kernel_source_sha256_16: {kernel_source_hash(kind)}\n"
                    f"hbm_bytes_per_launch: {hbm:.0f}\n"
                    + (f"request_size_bytes_per_launch: {req_bytes:.0f}\n" if req_bytes else "")
                    + f"algorithmic_bytes_per_launch: {alg}\nkernel_avg_ns: {avg_ns:.0f}\n")
    return path


# ----------------------------------------------------------------------------- main


def _config_entry(r: dict, cpu: dict | None = None) -> dict:
    e = {"workload": r["workload"], "state_dtype": r["state_dtype"],
         "entry_point": r["entry_point"], "us": r["us"],
         "graph_median_us": r.get("graph_median_us"), "gbps": r["gbps"],
         "frac": r["gbps"] / PEAK_HBM_GBPS, "algorithmic_bytes": r["nbytes"],
         "layers_rotated": r["layers"], "traffic": r["roofline"]["traffic"]}
    if r["kind"] == "prefill":
        rf = r["roofline"]
        e.update({"tflops": rf["achieved"], "frac_bf16_mfma": rf["frac"],
                  "frac_fp32_mfma": rf["frac_of_fp32_matrix_peak"],
                  "issued_frac_bf16_mfma": rf["issued_frac_of_bf16_peak"]})
    return e


def main(argv=None):
    args = parse_args(argv)
    if args.profile_commands:
        for name, cmd in profile_commands(args.workload, args.state_dtype, args.profile_root):
            print(f"{name}\t{cmd}")
        for name, cmd in copy_calibration_commands(args.profile_root):
            print(f"{name}\t{cmd}")
        return 0
    if args.summarize:
        print(summarize(args.summarize, args.workload, args.state_dtype))
        return 0
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

    headline = args.workload == DEFAULT_WORKLOAD and args.state_dtype == "f32"
    r = measure(args, args.workload, args.state_dtype, copy_ceiling=True)
    spec, kind = r["spec"], r["kind"]
    B, H, D, T = spec["B"], spec["H"], spec["D"], spec["T"]
    act = "bf16" if spec.get("fused") else spec.get("act", "none")
    if kind == "probe":
        act = "none"
    line = {
        "metric": METRIC, "value": r["us"], "unit": "us/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "dk": D, "dv": D, "T": T,
                   "state_dtype": args.state_dtype, "act_dtype": act,
                   "entry_point": r["entry_point"], "layers_rotated": r["layers"],
                   **({"r": spec["r"]} if kind == "lowrank" else {}),
                   **({"probe_variant": args.probe_variant, "probe_group": args.probe_group}
                      if kind == "probe" else {})},
        "achieved_gbps": r["gbps"],
        "seq_tokens_per_s": B * T / (r["ms"] * 1e-3),
        "us_per_token_48_layers": r["us"] * 48,
        "roofline": r["roofline"],
        "gflops": flops(spec) / (r["ms"] * 1e-3) / 1e9,
    }
    for k in ("roofline_hbm", "graph_median_us", "graph_p10_us", "graph_p90_us", "graph_protocol",
              "copy_gbps_same_bytes"):
        if k in r:
            line[k] = r[k]
    line["frac_of_copy_bw"] = r["gbps"] / r["copy_gbps_same_bytes"]
    if headline and not args.no_extra:
        configs = {}
        for label, wl, sdt, *over in EXTRA_CONFIGS:
            try:
                a2 = argparse.Namespace(**{**vars(args), **(over[0] if over else {})})
                configs[label] = _config_entry(measure(a2, wl, sdt))
                if over:
                    configs[label].update(over[0])
            except Exception as e:  # a failing extra config must not hide the headline line
                configs[label] = {"workload": wl, "state_dtype": sdt, "error": repr(e)[:300]}
            print(f"[bench] {label}: {json.dumps(configs[label])[:200]}", file=sys.stderr, flush=True)
        line["configs"] = configs
        probe = configs.get("stream_probe_b256_f32", {})
        if "us" in probe:
            line["frac_of_same_pattern_probe"] = probe["us"] / r["us"]
        best = configs.get("stream_probe_best_b256_f32", {})
        if "us" in best:
            line["frac_of_best_stream_probe"] = best["us"] / r["us"]
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        if kind == "probe":
            line["cpu_baseline"] = None
        else:
            n = args.cpu_threads or host_cores()
            cb = cpu_baseline(spec, args.workload, args.state_dtype, args.cpu_seconds, n)
            if cb["cores"] != 1:
                cb["single_thread"] = cpu_baseline(spec, args.workload, args.state_dtype,
                                                   args.cpu_seconds, 1)
            line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
