#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer on one MI355X.

Default workload: batch-1 decode through the GLM-5.2-shaped layer (H 6144,
I 2048, 256 routed experts top-8 with 8 groups keeping 4, rsf 2.5, router
bias N(0, 0.01), one shared expert; packed int4 weights with per-row fp32
scales; Q8_0 activations; logits computed from the fp32 gate).  Eight
independent layer instances (8 x 4.87 GB) are resident and step s uses
instance s mod 8 with its own token, so no step re-reads another step's
weights out of the 256 MB Infinity Cache.

A "step" is one full layer forward on one token.  The K timed steps are
captured into one HIP graph (launch overhead out of the way) and replayed
once between two synchronisations.  The same K steps are then launched
eagerly on the current stream through coli_moe_forward_profiled, whose
kernel launches each record a start and a stop hipEvent
(hipExtLaunchKernelGGL); those give each kernel's average execution time,
including that of the dominant kernel used for the roofline figure (decode:
the single fused kernel; union batches: the gate/up kernel).  Prints ONE JSON
line on stdout; details go to stderr.

  python bench.py [--steps K] [--warmup W] [--workload decode|verify3|prefill512]

``--workload fp8convert`` measures the checkpoint converter's step on the
device: one GLM-5.2 expert (gate and up 2048 x 6144, down 6144 x 2048) of
128x128 block-scaled FP8 E4M3 codes requantised into the packed container
(int4 unless --bits says otherwise) per step, over 16 resident experts.

``--workload gemvf32`` measures the f32-activation variant of the expert
GEMV (codes times row scale against binary32 activations, one token) on
GLM-5.2 gate-shaped (2048 x 6144) and down-shaped (6144 x 2048) matrices.

``--workload stack`` measures instead a 40-layer stack of such layers resident
in HBM (40 x 257 int4 experts, ~195 GB) decoded one token at a time, with a
Zipf-like expert popularity per layer and expert top-p 0.7; its bytes per
step are those of the experts the routing actually kept.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
MFMA_MIN_DEFAULT = 8  # the library's default mfma_min_tokens (routed experts) ...
MFMA_ALL_TOKENS = 64  # ... in batches below this size; from it on, every routed expert
MFMA_MIN_SHARED_DEFAULT = 64  # and for the shared expert
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _hip():
    """The HIP runtime torch loaded (shared with libcoli_moe.so)."""
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    L = ctypes.CDLL(path or "libamdhip64.so.7")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    L.hipGetLastError.argtypes = []
    return L


WORKLOADS = {
    # name: (tokens per step, logits supplied?, correlation of supplied logits)
    "decode": (1, False, 0.0),
    "verify3": (3, True, 0.0),
    "prefill512": (512, True, 0.0),
    # the small layer (H 256, I 128, 16 int8 experts top-2): latency only
    "tiny": (4, False, 0.0),
}


def expert_bytes(s) -> dict:
    """Algorithmic bytes of one expert (packed codes + fp32 row scales)."""
    H, I, b = s.hidden, s.inter, s.bits
    gate_up = 2 * (I * H * b // 8 + I * 4)
    down = H * I * b // 8 + H * 4
    return {"gate_up": gate_up, "down": down, "total": gate_up + down}


# sources each counted kernel is built from (its .hip file and the headers
# it includes)
KERNEL_SOURCES = {
    "k_decode_fused": ["decode.hip", "actq.hpp", "device.hpp", "ffn_common.hpp", "kernels.hpp",
                       "select.hpp"],
    "k_small_fused": ["decode.hip", "actq.hpp", "device.hpp", "ffn_common.hpp", "kernels.hpp",
                      "select.hpp"],
    "k_gateup_mfma": ["mfma.hip", "device.hpp", "ffn_common.hpp", "kernels.hpp"],
    "k_down_mfma": ["mfma.hip", "device.hpp", "ffn_common.hpp", "kernels.hpp"],
}


def kernel_sources_sha256(kernel: str = "k_decode_fused") -> str:
    """Hash of the sources a kernel is built from and of the ABI header: a
    stored counter measurement applies only to the kernel it was taken on."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(root, "quantized_moe_coli_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel)
    if names is None:
        names = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".hpp")))
    files = [os.path.join(csrc, f) for f in sorted(names)]
    files.append(os.path.join(root, "include", "coli_moe.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of the dominant kernel from rocprofv3 FETCH_SIZE and
    WRITE_SIZE runs (profiles/traffic_<workload>.json, scaled by a copy of
    known size), or None if absent or taken on other kernel sources."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if (not kernel.startswith(rec.get("kernel", "?"))
            or rec.get("sources_sha256") != kernel_sources_sha256(rec["kernel"])):
        return None
    return int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])


def summarize_counters(fetch_csv: str, write_csv: str, kernel: str, calib_mib: int,
                       commands: list) -> dict:
    """Traffic record of `kernel` from two rocprofv3 counter CSVs (FETCH_SIZE,
    then WRITE_SIZE; KiB per dispatch): the kernel's mean per dispatch, each
    scaled by what the same counter reads for the largest device-to-device
    copy in the run (the calibration copy of calib_mib MiB, which must read
    and write calib_mib * 1024 KiB)."""
    import csv

    def per_kernel(path):
        vals, copy = [], 0.0
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r.get("Kernel_Name") or r.get("Kernel-Name") or ""
                v = float(r.get("Counter_Value") or r.get("Counter-Value") or 0.0)
                if kernel in name:
                    vals.append(v)
                elif "copyBuffer" in name:
                    copy = max(copy, v)
        if not vals or copy <= 0:
            raise SystemExit(f"{path}: no {kernel} dispatches or no calibration copy")
        return sum(vals) / len(vals), copy, len(vals)

    known_kib = calib_mib * 1024.0
    f_mean, f_copy, n_f = per_kernel(fetch_csv)
    w_mean, w_copy, n_w = per_kernel(write_csv)
    f_scale, w_scale = known_kib / f_copy, known_kib / w_copy
    return {
        "kernel": kernel,
        "sources_sha256": kernel_sources_sha256(kernel),
        "fetch_bytes_per_launch": int(round(f_mean * 1024 * f_scale)),
        "write_bytes_per_launch": int(round(w_mean * 1024 * w_scale)),
        "fetch_kib_mean": round(f_mean, 1), "write_kib_mean": round(w_mean, 1),
        "copy_fetch_kib": round(f_copy, 1), "copy_write_kib": round(w_copy, 1),
        "fetch_scale": round(f_scale, 5),
        "write_scale": round(w_scale, 5),
        "dispatches": [n_f, n_w],
        "commands": commands,
    }


def main() -> int:
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters FETCH.csv WRITE.csv KERNEL CALIB_MIB "cmd1" "cmd2"
        rec = summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]),
                                 sys.argv[6:])
        print(json.dumps(rec, indent=1))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--instances", type=int, default=8)
    ap.add_argument("--workload", choices=list(WORKLOADS) + ["stack", "tiered", "guard",
                                                          "fp8convert", "gemvf32", "timeline"],
                    default="decode")
    ap.add_argument("--layers", type=int, default=None,
                    help="stack workload: layers resident (default 40); tiered workload: "
                         "layers whose experts sit in the pinned host tier (default 12: one "
                         "process may pin 64 GiB on the measured host, 12 x 4.84 GB)")
    ap.add_argument("--slots", type=int, default=None,
                    help="tiered workload: HBM expert slots per layer (default 64); guard "
                         "workload: run on the tiered stack with this many slots")
    ap.add_argument("--pin", type=int, default=16,
                    help="tiered workload: slots per layer pinned from the learned usage")
    ap.add_argument("--accept", type=str, default="0.3,0.6,0.9",
                    help="guard workload: per-draft acceptance rates to simulate")
    ap.add_argument("--draft", type=int, default=2, help="guard workload: drafts per verify")
    ap.add_argument("--bits", type=int, choices=(8, 4, 2), default=None,
                    help="weight container of the GLM-5.2-shaped layer (default int4)")
    ap.add_argument("--mfma-min", type=int, default=0,
                    help="layer's mfma_min_tokens (0: the library default)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per step with logits computed from the gate (overrides the "
                         "workload's batch; 1 = decode; with --workload stack: tokens per "
                         "step through the stack, e.g. 3 for MTP verify batches)")
    ap.add_argument("--rho", type=float, default=None,
                    help="verify3/prefill512: correlation of the supplied logits across the "
                         "batch (0: independent tokens; near 1: few unique experts)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one untimed device-to-device copy of this many MiB after the "
                         "warm-up (the known-size reference for hardware byte counters)")
    ap.add_argument("--stacked", action="store_true",
                    help="gemvf32 workload: one launch over the 16 experts' gate-shaped rows "
                         "stacked (32768 x 6144) and one over their down-shaped rows (98304 x 2048)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the oracle's timed CPU sample (0 disables it)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this "
              "build runs the layer on a single MI355X; multi-GPU sharding is a design "
              "note, not a measured path.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs

    torch.cuda.set_device(0)
    if args.workload == "stack":
        return stack_main(args)
    if args.workload == "tiered":
        return tiered_main(args)
    if args.workload == "guard":
        return guard_main(args)
    if args.workload == "fp8convert":
        return fp8_main(args)
    if args.workload == "gemvf32":
        return gemv_f32_main(args)
    if args.workload == "timeline":
        return timeline_main(args)
    dev = "cuda"
    s = inputs.TINY if args.workload == "tiny" else inputs.GLM
    if args.bits is not None:
        s = s.with_(bits=args.bits)
    T, supplied, rho = WORKLOADS[args.workload]
    if args.tokens > 0:
        T, supplied, rho = args.tokens, False, 0.0
    if args.rho is not None and supplied:
        rho = args.rho
    default_run = (args.bits in (None, 4) and args.tokens == 0 and args.workload != "tiny"
                   and args.mfma_min == 0)
    label = args.workload if default_run else (f"{args.workload}_int{s.bits}_T{T}" +
                                               (f"_mfma{args.mfma_min}" if args.mfma_min else ""))
    if supplied and rho != 0.0:
        label += f"_rho{rho:g}"
    K, W, NI = args.steps, args.warmup, args.instances
    cfg = B.router_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, 0.0, 1)

    t0 = time.time()
    layers = []
    for li in range(NI):
        L = B.MoeLayer.empty(s.hidden, s.inter, s.bits, cfg, dev)
        L.gate_w.copy_(inputs.gate_weight(s, li, dev))
        L.gate_bias.copy_(inputs.gate_bias(s, li, dev))
        for e in range(s.n_experts + 1):
            g, u, d = inputs.expert_weights(s, li, e, dev)
            L.pack_expert(e, g, u, d)
            del g, u, d
        L.mfma_min_tokens = args.mfma_min
        layers.append(L)
        torch.cuda.synchronize()
    log(f"[bench] {NI} layer instances packed in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB resident)")

    n_x = max(K, W)
    xs = torch.stack([inputs.tokens(s, 1, st, T, dev) for st in range(n_x)])  # [n_x, T, H]
    lgs = None
    if supplied:
        lgs = torch.stack([inputs.correlated_logits(1000 + st, T, s.n_experts, rho, device=dev)
                           for st in range(n_x)])
    ys = torch.empty(n_x, T, s.hidden, device=dev)
    ws = B.workspace(layers[0], T)
    cls = [L.c_struct() for L in layers]

    def step(st, stream_events=None):
        li = st % NI
        lin = lgs[st] if lgs is not None else None
        if stream_events is None:
            B.coli_moe_forward(layers[li], xs[st], ys[st], ws, logits_in=lin, c_layer=cls[li])
        else:
            B.coli_moe_forward_profiled(layers[li], xs[st], ys[st], ws, stream_events,
                                        logits_in=lin, c_layer=cls[li])

    # warm-up (eager, untimed)
    for st in range(W):
        step(st)
    torch.cuda.synchronize()
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # headline: the K timed steps captured into one HIP graph, replayed once
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for st in range(K):
                step(st)
    torch.cuda.synchronize()
    g.replay()  # one untimed replay of the captured steps
    torch.cuda.synchronize()

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    g.replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    del g

    # kernel durations: the same K steps launched eagerly on the current
    # stream; each launch of the front, gate/up and down kernels records a
    # start and a stop hipEvent itself (hipExtLaunchKernelGGL)
    hip = _hip()
    n_ev = 10
    evs = []
    for _ in range(K * n_ev):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e.value)
    torch.cuda.synchronize()
    e0 = time.perf_counter()
    for st in range(K):
        step(st, evs[st * n_ev:(st + 1) * n_ev])
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - e0

    def el(a, b):
        v = ctypes.c_float()
        rc = hip.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            hip.hipGetLastError()
            return float("nan")
        return v.value

    # decode and batches of 2-4 tokens: one fused kernel; larger unions:
    # front, gate/up and down on the dot-product path, gate/up and down on
    # the matrix cores
    n_k = 1 if T == 1 else 5
    stage = np.array([[el(evs[st * n_ev + 2 * i], evs[st * n_ev + 2 * i + 1]) for i in range(n_k)]
                      for st in range(K)])  # ms
    # a small batch that ran as one kernel records only the first events
    single = T == 1 or (T <= 4 and not np.isfinite(stage[:, 1:]).any())
    if single:
        stage = stage[:, :1]
        n_k = 1
    # the last kernel that ran (the matrix-core kernels are skipped for
    # batches below mfma_min tokens)
    last = n_k - 1 if np.isfinite(stage[:, n_k - 1]).all() else min(n_k - 1, 2)
    span = np.array([el(evs[st * n_ev], evs[st * n_ev + 2 * last + 1]) for st in range(K)])
    eager_ms = el(evs[0], evs[(K - 1) * n_ev + 2 * last + 1])
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    hip.hipGetLastError()

    ms_per_step = total_ms / K
    tokens_per_s = T * K / (total_ms / 1e3)
    eb = expert_bytes(s)
    gate_bytes = 0 if supplied else s.n_experts * s.hidden * 4

    # algorithmic bytes: the unique experts each step reads (+ the shared
    # one); in a union batch, experts with at least mfma_min tokens (and the
    # shared expert when T >= mfma_min) run on the matrix cores
    mfma_min = layers[0].mfma_min_tokens or (1 if T >= MFMA_ALL_TOKENS else MFMA_MIN_DEFAULT)
    shared_min = layers[0].mfma_min_tokens or MFMA_MIN_SHARED_DEFAULT
    if T == 1:
        uniq = np.full(K, s.top_k, dtype=np.float64)
        n_mfma = np.zeros(K)
    else:
        uniq, n_mfma = [], []
        for st in range(K):
            idx = torch.empty(T, s.top_k, dtype=torch.int32, device=dev)
            if lgs is not None:
                B.coli_moe_route(cfg, lgs[st], layers[st % NI].gate_bias, idx,
                                 torch.empty(T, s.top_k, device=dev))
            else:  # computed logits: the layer's own routing of this step
                B.coli_moe_forward(layers[st % NI], xs[st], torch.empty_like(ys[st]), ws,
                                   idx_out=idx, c_layer=cls[st % NI])
            cnt = torch.bincount(idx[idx >= 0].long(), minlength=s.n_experts)
            uniq.append(int((cnt > 0).sum()))
            n_mfma.append(int((cnt >= mfma_min).sum()) + (1 if T >= shared_min else 0))
        uniq = np.array(uniq, dtype=np.float64)
        n_mfma = np.array(n_mfma, dtype=np.float64)
    act_bytes = T * s.hidden * 4 * 2  # x in, y out
    layer_bytes = (uniq + 1) * eb["total"] + gate_bytes + act_bytes
    avg = stage.mean(axis=0)
    layer_gbps = float(np.mean(layer_bytes)) / (ms_per_step * 1e-3) / 1e9
    if single:  # the dominant (only) kernel is the fused kernel
        dom_name = ("k_decode_fused (the whole layer for one token)" if T == 1 else
                    f"k_small_fused (the whole layer for the {T}-token batch)")
        dom_ms = float(avg[0])
        dom_bytes = float(np.mean(layer_bytes))
    else:
        # each kernel's bytes: the expert weights of the slots it runs
        n_dot = uniq + 1 - n_mfma
        kbytes = {1: n_dot * eb["gate_up"], 2: n_dot * eb["down"],
                  3: n_mfma * eb["gate_up"], 4: n_mfma * eb["down"]}
        knames = {1: "k_gateup_union (gate/up dot-product GEMV + SwiGLU + Q8_0 of h)",
                  2: "k_down_union (down dot-product GEMV)",
                  3: "k_gateup_mfma (gate/up on the int8 matrix cores + SwiGLU + Q8_0 of h)",
                  4: "k_down_mfma (down on the int8 matrix cores)"}
        dom = max((1, 2, 3, 4), key=lambda i: np.nan_to_num(avg[i]))
        avg = np.nan_to_num(avg)
        dom_name = knames[dom]
        dom_ms = float(avg[dom])
        dom_bytes = float(np.mean(kbytes[dom]))
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9
    log(f"[bench] {label}: {K} steps in {total_ms:.3f} ms (wall {wall * 1e3:.1f} ms): "
        f"{ms_per_step * 1e3:.2f} us/step, {tokens_per_s:.0f} tokens/s")
    log(f"[bench] eager pass with kernel events: {eager_ms / K * 1e3:.2f} us/step (host wall "
        f"{eager_wall / K * 1e6:.2f} us/step), first-kernel start to last-kernel end "
        f"{np.mean(span) * 1e3:.2f} us")
    if single:
        log(f"[bench] kernel mean (us): {'k_decode_fused' if T == 1 else 'k_small_fused'} "
            f"{avg[0] * 1e3:.2f}")
    else:
        gbs = {i: float(np.mean(kbytes[i])) / (avg[i] * 1e-3) / 1e9 for i in (1, 2, 3, 4)}
        log(f"[bench] kernel means (us): front {avg[0] * 1e3:.2f}; dot-product path gate/up "
            f"{avg[1] * 1e3:.2f} ({gbs[1]:.0f} GB/s), down {avg[2] * 1e3:.2f} ({gbs[2]:.0f} GB/s); "
            f"matrix cores gate/up {avg[3] * 1e3:.2f} ({gbs[3]:.0f} GB/s), down {avg[4] * 1e3:.2f} "
            f"({gbs[4]:.0f} GB/s); experts on the matrix cores/step {n_mfma.mean():.1f}")
    log(f"[bench] unique experts/step {uniq.mean():.1f}; layer bytes/step "
        f"{np.mean(layer_bytes) / 1e6:.2f} MB -> {layer_gbps:.0f} GB/s "
        f"({100 * layer_gbps / HBM_PEAK_GBPS:.1f}% of HBM peak); dominant kernel "
        f"{dom_gbps:.0f} GB/s")

    result = {
        "metric": "MoE-layer tokens/s (int4 top-8/256 decode)" if (T == 1 and default_run) else
                  f"MoE-layer tokens/s ({label})",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{s.bits}xint8->int32,fp32-scale",
        "data": "synthetic",
        "config": {
            "workload": (("GLM-5.2 routed-MoE layer" if s is not inputs.TINY and args.workload != "tiny"
                          else "small routed-MoE layer") +
                         (" batch-1 decode" if T == 1 else f" {T}-token union batch"
                          + (" in one kernel" if single else "")) +
                         f": H {s.hidden}, I {s.inter}, {s.n_experts} experts top-{s.top_k} "
                         + (f"({s.n_group} groups keep {s.topk_group}, rsf {s.rsf}) " if s.n_group > 1
                            else f"(rsf {s.rsf}) ")
                         + f"+ 1 shared, {'packed ' if s.bits < 8 else ''}int{s.bits} per-row fp32 "
                         "scale, Q8_0 activations" + (", logits from the fp32 gate" if not supplied
                                                       else f", logits supplied (correlation "
                                                            f"{rho:g} across the batch)")),
            "tokens_per_step": T,
            "layer_instances": NI,
            "unique_experts_per_step": {"mean": round(float(uniq.mean()), 2),
                                        "min": int(uniq.min()), "max": int(uniq.max())},
            "launch": "one HIP graph of the K timed steps",
            "kernel_us": ({("k_decode_fused" if T == 1 else "k_small_fused"): round(float(avg[0]) * 1e3, 3)}
                          if single else
                          {"front": round(float(avg[0]) * 1e3, 3),
                           "gate_up_dot": round(float(avg[1]) * 1e3, 3),
                           "down_dot": round(float(avg[2]) * 1e3, 3),
                           "gate_up_mfma": round(float(avg[3]) * 1e3, 3),
                           "down_mfma": round(float(avg[4]) * 1e3, 3)}),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom_name,
            "achieved": round(dom_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(label, dom_name),
            "avg_launch_us": round(dom_ms * 1e3, 3),
            "bytes_per_launch": int(dom_bytes),
        },
        "layer_roofline": {
            "bound": "hbm",
            "achieved": round(layer_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
            "bytes_per_step": int(np.mean(layer_bytes)),
        },
    }

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(s, layers[0], xs, lgs, ys, NI, args.cpu_seconds, T)
    print(json.dumps(result), flush=True)
    return 0


def cpu_model() -> str:
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def timed_samples(run_one, budget_s, n_samples=3):
    """Rates of `n_samples` back-to-back samples that share `budget_s`: each
    sample calls `run_one()` (which returns its own timed seconds and units
    done) until its share is spent, at least once.  Returns the per-sample
    (units, seconds)."""
    out = []
    for i in range(n_samples):
        units, spent = 0, 0.0
        while True:
            dt, du = run_one()
            spent += dt
            units += du
            if spent >= budget_s / n_samples:
                break
        out.append((units, spent))
        log(f"[bench] cpu baseline sample {i + 1}/{n_samples}: {units:g} units in {spent:.2f} s")
    return out


def cpu_baseline(s, layer0, xs, lgs, ys, NI, budget_s, T):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    steps that use layer instance 0, one forward call at a time, first on one
    thread and then on every thread the oracle's OpenMP runtime starts by
    default (the host's share of cores), half the budget each, as three
    samples per thread count whose median rate is reported.  The oracle packs
    the experts it needs from the same fp32 draws with its own code (untimed,
    once per step) and each thread count gets one untimed warm call."""
    import numpy as np

    import oracle
    from quantized_moe_coli_amd import inputs

    li = 0
    ocfg = oracle.make_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, 0.0, 1)
    gate_w = inputs.gate_weight(s, li, "cuda").cpu().numpy()
    bias = inputs.gate_bias(s, li, "cuda").cpu().numpy()
    cache, prepared = {}, {}

    def expert(e):
        if e not in cache:
            g, u, d = (t.cpu().numpy() for t in inputs.expert_weights(s, li, e, "cuda"))
            cache[e] = oracle.Expert.from_float(s.bits, g, u, d)
        return cache[e]

    def prepare(st):
        if st not in prepared:
            x = xs[st].cpu().numpy()
            lin = lgs[st].cpu().numpy() if lgs is not None else None
            lg = oracle.logits(x, gate_w) if lin is None else lin
            idx, _ = oracle.route(ocfg, lg, bias)
            exps = [None] * s.n_experts
            for e in set(idx.ravel().tolist()):
                if e >= 0:
                    exps[e] = expert(e)
            L = oracle.Layer(s.hidden, s.inter, s.bits, ocfg, exps, expert(s.n_experts), gate_w, bias)
            prepared[st] = (L, x, lin, ys[st].cpu().numpy().astype(np.float64))
        return prepared[st]

    steps = list(range(0, xs.shape[0], NI))
    state = {"i": 0, "err": 0.0}

    def run_one():
        st = steps[state["i"] % len(steps)]
        state["i"] += 1
        L, x, lin, y = prepare(st)
        t0 = time.perf_counter()
        y_r, _, _, _ = oracle.moe_forward(L, x, lin)
        dt = time.perf_counter() - t0
        err = np.abs(y - y_r).max(axis=1) / np.maximum(np.abs(y_r).max(axis=1), 1e-30)
        state["err"] = max(state["err"], float(err.max()))
        return dt, T

    n_all = oracle.num_threads()
    legs = {}
    for n in (1, n_all):
        if n in legs:
            continue
        oracle.set_num_threads(n)
        L, x, lin, _ = prepare(steps[0])
        oracle.moe_forward(L, x, lin)  # untimed warm call
        samples = timed_samples(run_one, budget_s / 2)
        rates = sorted(u / t for u, t in samples)
        legs[n] = {"threads": n, "value": round(float(np.median(rates)), 4),
                   "samples": [round(r, 4) for r in rates],
                   "calls": int(sum(u for u, _ in samples) // T),
                   "seconds": round(sum(t for _, t in samples), 2)}
        log(f"[bench] oracle on {n} thread(s): median {legs[n]['value']} tokens/s over "
            f"samples {legs[n]['samples']} ({legs[n]['calls']} calls)")
    oracle.set_num_threads(n_all)
    log(f"[bench] GPU outputs of the timed steps within {state['err']:.2e} (rel. to max |y|) "
        f"of the oracle")
    return {
        "value": legs[n_all]["value"],
        "unit": "tokens/s",
        "cores": n_all,
        "kind": "oracle",
        "cpu": cpu_model(),
        "single_thread": legs[1],
        "all_threads": legs[n_all],
        "sample": f"forward calls of {T} token(s) on layer instance 0 (steps 0, {NI}, "
                  f"{2 * NI}, ... in turn), on 1 thread and on {n_all}; per thread count "
                  f"three back-to-back samples of ~{budget_s / 6:.1f} s of timed calls, "
                  f"median rate; GPU outputs of the same steps agree to {state['err']:.1e}",
    }


TRACE_NAMES = {1: "entry", 2: "logit slices done", 3: "x quantised", 4: "shared rows done",
               5: "selection begins", 6: "scores read", 7: "selection done",
               8: "routed gate/up item done", 9: "down item begins", 10: "down item h ready",
               11: "down item done", 12: "exit"}


def timeline_main(args) -> int:
    """Where the single-kernel decode's time goes: the timeline build of the
    library records every workgroup's phase and item boundaries
    (s_memrealtime, 10 ns ticks) on the default decode workload; each step's
    times are taken from its first workgroup's entry, and the medians over
    the steps of each phase's first / median / last workgroup are reported.
    Beside it, the plain streaming read of as many bytes (the practical HBM
    ceiling for a kernel with no routing and no dependencies) over 8
    distinct buffers, timed with hip events."""
    import numpy as np
    import torch

    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs

    dev = "cuda"
    s = inputs.GLM if args.bits is None else inputs.GLM.with_(bits=args.bits)
    NI, K = args.instances, max(8, min(args.steps, 64))
    cfg = B.router_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, 0.0, 1)
    layers = []
    for li in range(NI):
        L = B.MoeLayer.empty(s.hidden, s.inter, s.bits, cfg, dev)
        L.gate_w.copy_(inputs.gate_weight(s, li, dev))
        L.gate_bias.copy_(inputs.gate_bias(s, li, dev))
        for e in range(s.n_experts + 1):
            g, u, d = inputs.expert_weights(s, li, e, dev)
            L.pack_expert(e, g, u, d)
            del g, u, d
        layers.append(L)
    torch.cuda.synchronize()
    cls = [L.c_struct() for L in layers]
    xs = [inputs.tokens(s, 1, st, 1, dev) for st in range(K + 8)]
    y = torch.empty(1, s.hidden, device=dev)
    ws = B.workspace(layers[0], 1)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    trace = torch.zeros(8 * n_cu, B.TRACE_RECORDS, 2, dtype=torch.int64, device=dev)
    for st in range(8):  # warm-up
        B.coli_debug_decode_trace(layers[st % NI], xs[st], y, ws, trace, c_layer=cls[st % NI])
    torch.cuda.synchronize()
    rows = {}  # name -> list over steps of (first, median, last) in us
    kern = []
    for st in range(K):
        trace.zero_()
        li = (8 + st) % NI
        grid = B.coli_debug_decode_trace(layers[li], xs[8 + st], y, ws, trace, c_layer=cls[li])
        torch.cuda.synchronize()
        r = trace[:grid].cpu().numpy()
        code = (r[:, :, 0] >> 48) & 0xFFFF
        tm = r[:, :, 1].astype(np.float64)
        t0 = tm[code == 1].min()
        rel = (tm - t0) / 100.0  # 100 MHz ticks -> us
        kern.append(rel[code == 12].max())
        for c, nm in TRACE_NAMES.items():
            v = rel[code == c]
            if v.size:
                rows.setdefault(nm, []).append((v.min(), np.median(v), v.max(), v.size))
    table = {nm: {"first": round(float(np.median([x[0] for x in v])), 2),
                  "median": round(float(np.median([x[1] for x in v])), 2),
                  "last": round(float(np.median([x[2] for x in v])), 2),
                  "records": int(np.median([x[3] for x in v]))}
             for nm, v in rows.items()}
    log(f"[bench] timeline of the single-kernel decode (int{s.bits}, grid {grid}, medians over {K} "
        f"steps; us from the first workgroup's entry)")
    for nm in TRACE_NAMES.values():
        if nm in table:
            t = table[nm]
            log(f"[bench]   {nm:26s} first {t['first']:6.2f}  median {t['median']:6.2f}  "
                f"last {t['last']:6.2f}  ({t['records']} records)")
    eb = expert_bytes(s)
    step_bytes = 9 * eb["total"] + s.n_experts * s.hidden * 4 + 2 * s.hidden * 4
    # plain streaming read of the same bytes, 8 distinct buffers
    nbytes = (step_bytes + 15) // 16 * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(8)]
    for b in bufs:
        b.fill_(1)
    out = torch.empty(8 * n_cu, dtype=torch.int32, device=dev)
    for b in bufs:
        B.coli_debug_stream_read(b, out)
    torch.cuda.synchronize()
    reps = 200
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        B.coli_debug_stream_read(bufs[i % 8], out)
    stop.record()
    torch.cuda.synchronize()
    stream_us = start.elapsed_time(stop) / reps * 1e3
    big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    big.fill_(1)
    B.coli_debug_stream_read(big, out)
    torch.cuda.synchronize()
    start.record()
    for i in range(20):
        B.coli_debug_stream_read(big, out)
    stop.record()
    torch.cuda.synchronize()
    big_us = start.elapsed_time(stop) / 20 * 1e3
    kernel_us = float(np.median(kern))
    log(f"[bench] decode kernel (trace build, median over steps) {kernel_us:.2f} us for "
        f"{step_bytes / 1e6:.2f} MB")
    log(f"[bench] plain streaming read of {nbytes / 1e6:.2f} MB: {stream_us:.2f} us "
        f"({nbytes / stream_us / 1e3:.0f} GB/s); of 1 GiB: {big_us:.1f} us "
        f"({(1 << 30) / big_us / 1e3:.0f} GB/s)")
    print(json.dumps({
        "metric": "single-kernel decode timeline (us from the first workgroup's entry)",
        "workload": f"GLM-5.2 layer batch-1 decode, int{s.bits}, {NI} layer instances",
        "grid": grid, "steps": K, "phases": table,
        "kernel_us": round(kernel_us, 2),
        "stream_ceiling": {"bytes": nbytes, "us": round(stream_us, 2),
                           "GBps": round(nbytes / stream_us / 1e3, 1),
                           "GiB_us": round(big_us, 1),
                           "GiB_GBps": round((1 << 30) / big_us / 1e3, 1)},
    }), flush=True)
    return 0


def _kernel_events(hip, n):
    evs = []
    for _ in range(n):
        e = ctypes.c_void_p()
        if hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        evs.append(e.value)
    return evs


def stack_main(args) -> int:
    """The multi-layer decode: every step feeds a fresh token through all
    resident layers (h <- h + MoE_l(rmsnorm(h))), one HIP graph per step
    replayed on the token.  With --tokens T > 1 every step is instead a
    T-token batch (an MTP verify: the current token and T - 1 drafts) that
    each layer runs as one batch union."""
    import numpy as np
    import torch

    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs, stack

    dev = "cuda"
    K, W, NL = args.steps, args.warmup, args.layers or 40
    T = max(1, args.tokens)
    t0 = time.time()
    stk = stack.build(NL)
    s = stk.s
    log(f"[bench] stack: {NL} layers packed in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB resident)")
    n_x = max(K, W, 1)
    xs = torch.stack([inputs.tokens(s, stack.token_seed(), t, T, dev) for t in range(n_x)])
    ws = B.workspace(stk.layers[0], T)
    h = torch.empty(T, s.hidden, device=dev)
    y = torch.empty(T, s.hidden, device=dev)
    idx_g = torch.empty(NL, T, s.top_k, dtype=torch.int32, device=dev)
    w_g = torch.empty(NL, T, s.top_k, device=dev)
    for t in range(W):
        h.copy_(xs[t])
        stack.step(stk, h, ws, y, idx_g, w_g)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            stack.step(stk, h, ws, y, idx_g, w_g)
    torch.cuda.synchronize()
    idx_all = torch.empty(K, NL, T, s.top_k, dtype=torch.int32, device=dev)

    def run_steps():
        for t in range(K):
            h.copy_(xs[t])
            g.replay()
            idx_all[t].copy_(idx_g)

    run_steps()  # one untimed pass
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record()
    run_steps()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    del g

    # kernel durations: an eager pass over the first steps, every layer's
    # launches recording start and stop events (T = 1: the fused decode
    # kernel; T = 2-4: the fused small-batch kernel; larger T: front, gate/up
    # and down on the dot-product path, gate/up and down on the matrix cores)
    hip = _hip()
    KP = min(K, 32)
    n_ev = 2 if T == 1 else 10
    evs = _kernel_events(hip, KP * NL * n_ev)
    torch.cuda.synchronize()
    for t in range(KP):
        h.copy_(xs[t])
        for li, L in enumerate(stk.layers):
            e = evs[(t * NL + li) * n_ev:(t * NL + li + 1) * n_ev]
            B.coli_moe_forward_profiled(L, stack.rmsnorm(h), y, ws, e, c_layer=stk.c_layers[li])
            h.add_(y)
    torch.cuda.synchronize()
    def ev_ms(i, k):
        v = ctypes.c_float()
        rc = hip.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(evs[i * n_ev + 2 * k]),
                                     ctypes.c_void_p(evs[i * n_ev + 2 * k + 1]))
        return v.value if rc == 0 else float("nan")

    # a small batch that ran as one kernel records only the first events
    single = T == 1 or (T <= 4 and all(np.isnan(ev_ms(i, 1)) for i in range(KP * NL)))
    dom_k = 0 if single else 1  # the fused kernel / the dot-product gate/up kernel
    kms = [ev_ms(i, dom_k) for i in range(KP * NL)]
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    hip.hipGetLastError()
    kms = np.array(kms).reshape(KP, NL)

    idx = idx_all.cpu().numpy()  # [K, NL, T, k]
    kept = (idx >= 0).sum(axis=3)  # [K, NL, T] experts each token keeps
    uniq = np.array([[len(set(idx[t, li][idx[t, li] >= 0].tolist())) for li in range(NL)]
                     for t in range(K)])  # [K, NL] unique experts a layer reads for the batch
    ebd = expert_bytes(s)
    eb = ebd["total"]
    gate_bytes = s.n_experts * s.hidden * 4
    act_bytes = T * s.hidden * 4 * 2
    launch_bytes = (uniq + 1) * eb + gate_bytes + act_bytes  # per layer launch
    step_bytes = launch_bytes.sum(axis=1)
    ms_per_step = total_ms / K
    tokens_per_s = T * K / (total_ms / 1e3)
    gbps = float(step_bytes.mean()) / (ms_per_step * 1e-3) / 1e9
    k_avg_ms = float(np.nanmean(kms))
    if single:
        k_bytes = float(launch_bytes[:KP].mean())
        k_name = ("k_decode_fused (one layer for one token)" if T == 1 else
                  f"k_small_fused (one layer for the {T}-token batch)")
    else:  # T < 8: every slot on the dot-product path
        k_bytes = float(((uniq[:KP] + 1) * ebd["gate_up"]).mean())
        k_name = "k_gateup_union (one layer's gate/up for the batch union)"
    k_gbps = k_bytes / (k_avg_ms * 1e-3) / 1e9
    log(f"[bench] stack: {K} steps of {T} token(s) in {total_ms:.2f} ms (wall {wall * 1e3:.1f} "
        f"ms): {ms_per_step * 1e3:.1f} us/step, {tokens_per_s:.1f} tokens/s; kept experts per "
        f"token and layer {kept.mean():.2f}, unique per layer {uniq.mean():.2f}; bytes/step "
        f"{step_bytes.mean() / 1e9:.3f} GB -> {gbps:.0f} GB/s")
    log(f"[bench] {k_name.split()[0]}: {k_avg_ms * 1e3:.2f} us avg over {KP * NL} launches, "
        f"{k_bytes / 1e6:.1f} MB each -> {k_gbps:.0f} GB/s")

    result = {
        "metric": (f"MoE-stack tokens/s ({NL} int4 layers, Zipf popularity, expert top-p 0.7)"
                   if T == 1 else
                   f"MoE-stack MTP-verify tokens/s ({T}-token batches through {NL} int4 layers, "
                   "Zipf popularity, expert top-p 0.7)"),
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8->int32,fp32-scale",
        "data": "synthetic",
        "config": {
            "workload": f"{NL} GLM-5.2-shaped routed-MoE layers resident (H 6144, I 2048, 256 "
                        "experts top-8, 8 groups keep 4, rsf 2.5, + 1 shared; packed int4), "
                        "per-layer logit offsets -1.1 ln(rank+1) over a random expert ranking, "
                        "expert top-p 0.7 renormalised; "
                        + ("batch-1 decode" if T == 1 else
                           f"{T}-token MTP verify batches (the current token and {T - 1} "
                           "drafts) run as one batch union per layer"
                           + (" in one kernel" if single else ""))
                        + ", h <- h + MoE(rmsnorm(h)) between layers",
            "tokens_per_step": T,
            "layers": NL,
            "launch": "one HIP graph per step (all layers), replayed on each token",
            "kept_experts_per_layer": round(float(kept.mean()), 3),
            "unique_experts_per_layer": round(float(uniq.mean()), 3),
            # expert reads of a verify batch against T decode steps of the same tokens
            "expert_reads_vs_per_token": round(float((uniq + 1).sum() / (kept + 1).sum()), 4),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": k_name,
            "achieved": round(k_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(k_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "avg_launch_us": round(k_avg_ms * 1e3, 3),
            "bytes_per_launch": int(k_bytes),
        },
        "layer_roofline": {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "bytes_per_step": int(step_bytes.mean()),
        },
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = stack_cpu_baseline(stk, xs, ws, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


PCIE5_X16_GBPS = 63.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def _mem_available() -> int:
    with open("/proc/meminfo") as f:
        for line in f:
            if line.startswith("MemAvailable:"):
                return int(line.split()[1]) * 1024
    return 0


def tiered_main(args) -> int:
    """The stack decode with every layer's routed experts in pinned host
    memory and --slots HBM slots per layer in front of them (per-layer
    expert caches, LRU with pinned slots).  Three timed passes of --steps
    tokens: a cold start (empty caches), the same caches warmed by the
    first pass, and a restart whose caches pin, at start, the --pin experts
    per layer that the first two passes used most (the usage profile).  A
    calibration times the copy kernel alone on a repin of S-1 experts."""
    import numpy as np
    import torch

    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs, stack

    dev = "cuda"
    K, NL, S, NP = args.steps, args.layers or 12, args.slots or 64, args.pin
    s = stack.STACK_SHAPE
    eb = expert_bytes(s)["total"]
    tier_bytes = NL * s.n_experts * eb
    avail = _mem_available()
    log(f"[bench] tiered: {NL} layers, host tier {tier_bytes / 1e9:.1f} GB pinned "
        f"(MemAvailable {avail / 1e9:.1f} GB), {S} HBM slots per layer "
        f"({NL * S * eb / 1e9:.1f} GB), {NP} pinned per layer in the restart pass")
    if avail and tier_bytes > 0.8 * avail:
        print(f"host tier of {tier_bytes / 1e9:.0f} GB exceeds 80% of the host's available "
              f"memory ({avail / 1e9:.0f} GB); use fewer --layers", file=sys.stderr)
        return 2
    if not 0 <= NP < S - s.top_k + 1:
        print("--pin must leave at least top_k unpinned slots", file=sys.stderr)
        return 2
    t0 = time.time()
    st = stack.build_tiered(NL, S, log=log)
    log(f"[bench] tiered: built in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB in HBM)")
    xs = torch.stack([inputs.tokens(s, stack.token_seed(), t, 1, dev) for t in range(3 * K)])
    ws = B.workspace(st.layers[0], 1)
    h = torch.empty(1, s.hidden, device=dev)
    y = torch.empty(1, s.hidden, device=dev)
    idx_g = torch.empty(NL, 1, s.top_k, dtype=torch.int32, device=dev)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            stack.step_tiered(st, h, ws, y, idx_g)
    torch.cuda.synchronize()

    def totals():
        hs = [c.stats() for c in st.caches]
        return sum(x["hits"] for x in hs), sum(x["misses"] for x in hs), max(x["error"] for x in hs)

    def run_pass(first):
        h0, m0, _ = totals()
        kept = torch.empty(K, NL, 1, s.top_k, dtype=torch.int32, device=dev)
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for t in range(K):
            h.copy_(xs[first + t])
            g.replay()
            kept[t].copy_(idx_g)
        stop.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(stop)
        h1, m1, err = totals()
        hits, misses = h1 - h0, m1 - m0
        k = kept.cpu().numpy()
        return {"tokens_per_s": round(K / (ms / 1e3), 3), "ms_per_token": round(ms / K, 4),
                "hit_rate": round(hits / max(1, hits + misses), 4),
                "misses_per_token": round(misses / K, 3),
                "host_link_gb_per_token": round(misses * eb / K / 1e9, 4),
                "kept_experts_per_layer": round(float((k >= 0).sum(axis=3).mean()), 3),
                "cache_error": int(err)}

    for c in st.caches:
        c.init()
    cold = run_pass(0)
    log(f"[bench] tiered cold: {cold}")
    warm = run_pass(K)
    log(f"[bench] tiered warm: {warm}")
    # restart with the usage profile the two passes learned, pinned at start
    usage = [c.use_count.clone() for c in st.caches]
    for c, u, L, cl in zip(st.caches, usage, st.layers, st.c_layers):
        c.init()
        c.use_count.copy_(u)
        c.repin(L, NP, c_layer=cl)
    torch.cuda.synchronize()
    h_r, m_r, _ = totals()
    pinned = run_pass(2 * K)
    log(f"[bench] tiered restart with {NP} learned pins per layer: {pinned}")

    # host-link calibration: the copy kernel alone moving S-1 experts into an
    # emptied cache (a repin from zero usage loads experts 0 .. S-2)
    c0, L0, cl0 = st.caches[0], st.layers[0], st.c_layers[0]
    reps, cal_ms = 3, []
    for _ in range(reps):
        c0.init()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c0.repin(L0, S - 1, c_layer=cl0)
        e1.record()
        torch.cuda.synchronize()
        cal_ms.append(e0.elapsed_time(e1))
    cal_ms = float(np.median(cal_ms))
    link = (S - 1) * eb / (cal_ms * 1e-3) / 1e9
    log(f"[bench] copy kernel: {S - 1} experts ({(S - 1) * eb / 1e9:.2f} GB) host -> HBM in "
        f"{cal_ms:.2f} ms -> {link:.1f} GB/s")
    del g
    result = {
        "metric": (f"MoE-stack tokens/s through per-layer HBM expert caches over a pinned host "
                   f"tier ({NL} int4 layers, Zipf popularity, expert top-p 0.7)"),
        "value": warm["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": K,
        "ms_per_step": warm["ms_per_token"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8->int32,fp32-scale",
        "data": "synthetic",
        "config": {
            "workload": f"{NL} GLM-5.2-shaped routed-MoE layers (H 6144, I 2048, 256 experts "
                        "top-8, 8 groups keep 4, rsf 2.5, + 1 shared; packed int4), per-layer "
                        "logit offsets -1.1 ln(rank+1) over a random expert ranking, expert "
                        "top-p 0.7 renormalised, batch-1 decode; routed experts in pinned host "
                        f"memory, {S} HBM slots per layer",
            "layers": NL,
            "slots_per_layer": S,
            "hbm_slot_gb": round(NL * S * eb / 1e9, 2),
            "host_tier_gb": round(tier_bytes / 1e9, 2),
            "launch": "one HIP graph per token (all layers: logits, selection, cache update, "
                      "copies, layer), replayed",
            "value_pass": "warm",
        },
        "passes": {"cold": cold, "warm": warm, f"restart_pinned_{NP}": pinned},
        "roofline": {
            "bound": "host_link",
            "kernel": "k_cache_fill (host tier -> HBM slots)",
            "achieved": round(link, 2),
            "peak": PCIE5_X16_GBPS,
            "unit": "GB/s",
            "frac": round(link / PCIE5_X16_GBPS, 4),
            "traffic": None,
            "bytes_per_launch": int((S - 1) * eb),
            "avg_launch_us": round(cal_ms * 1e3, 1),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def guard_main(args) -> int:
    """The adaptive speculation guard on the stack decode.  A step either
    decodes one token or verifies it with --draft drafts in one batch (one
    batch union per layer); acceptance is simulated (seeded, per-draft rate
    --accept, a draft counts only if every earlier one was accepted), since
    the drafts' content needs the trained model.  Three policies per rate --
    never draft, always draft, the guard fed each step's measured GPU time --
    over the same --steps from the same start.  With --slots the stack is
    the tiered one (12 layers over pinned host memory, caches emptied before
    each policy: the cold start the guard exists for); else --layers resident
    layers."""
    import numpy as np
    import torch

    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs, stack

    dev = "cuda"
    K, D = args.steps, args.draft
    tiered = args.slots is not None and args.slots > 0
    rates = [float(v) for v in args.accept.split(",")]
    t0 = time.time()
    if tiered:
        NL = args.layers or 12
        st = stack.build_tiered(NL, args.slots, log=log)
        step_fn = lambda h, ws, y, idx: stack.step_tiered(st, h, ws, y, idx)  # noqa: E731
    else:
        NL = args.layers or 40
        st = stack.build(NL)
        step_fn = lambda h, ws, y, idx: stack.step(st, h, ws, y, idx)  # noqa: E731
    s = st.s
    log(f"[bench] guard: {NL} layers {'tiered, ' + str(args.slots) + ' slots' if tiered else 'resident'}"
        f", built in {time.time() - t0:.1f}s")
    graphs, bufs = {}, {}
    for T in (1, 1 + D):
        ws = B.workspace(st.layers[0], T)
        h = torch.empty(T, s.hidden, device=dev)
        y = torch.empty(T, s.hidden, device=dev)
        idx = torch.empty(NL, T, s.top_k, dtype=torch.int32, device=dev)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                step_fn(h, ws, y, idx)
        torch.cuda.synchronize()
        # the graph reads and writes these: they live as long as it does
        graphs[T], bufs[T] = g, (h, idx, ws, y)
    xs = {T: torch.stack([inputs.tokens(s, stack.token_seed(), t, T, dev) for t in range(K)])
          for T in (1, 1 + D)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(policy, rate):
        if tiered:
            for c in st.caches:
                c.init()
            torch.cuda.synchronize()
        rng = np.random.default_rng(1234)
        guard = B.SpecGuard(D, probe_every=16, ema=0.25) if policy == "guard" else None
        produced, total_ms, reads, drafted_steps, miss0 = 0, 0.0, 0, 0, 0
        if tiered:
            miss0 = sum(c.stats()["misses"] for c in st.caches)
        for t in range(K):
            d = D if policy == "always" else 0 if policy == "never" else guard.next_draft
            T = 1 + d
            h, idx = bufs[T][:2]
            h.copy_(xs[T][t])
            e0.record()
            graphs[T].replay()
            e1.record()
            e1.synchronize()
            ms = e0.elapsed_time(e1)
            acc = 0
            while acc < d and rng.random() < rate:
                acc += 1
            if guard is not None:
                guard.step(d, acc, ms * 1e3)
            produced += 1 + acc
            total_ms += ms
            drafted_steps += 1 if d else 0
            ix = idx.cpu().numpy()
            reads += sum(len(set(ix[li][ix[li] >= 0].tolist())) + 1 for li in range(NL))
        out = {"tokens_per_s": round(produced / (total_ms / 1e3), 2),
               "tokens_per_step": round(produced / K, 3),
               "expert_reads_per_token": round(reads / produced, 2),
               "draft_fraction": round(drafted_steps / K, 3)}
        if tiered:
            miss = sum(c.stats()["misses"] for c in st.caches) - miss0
            out["host_link_gb_per_token"] = round(miss * expert_bytes(s)["total"] / produced / 1e9, 4)
        return out

    table = {}
    for rate in rates:
        table[str(rate)] = {p: run(p, rate) for p in ("never", "always", "guard")}
        log(f"[bench] guard, acceptance {rate}: {table[str(rate)]}")
    mid = table[str(rates[len(rates) // 2])]
    result = {
        "metric": ("MoE-stack tokens/s under the adaptive speculation guard "
                   f"({NL} int4 layers, Zipf popularity, expert top-p 0.7, {D} drafts per verify)"),
        "value": mid["guard"]["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": 0,
        "ms_per_step": round(1e3 * mid["guard"]["tokens_per_step"] / mid["guard"]["tokens_per_s"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4xint8->int32,fp32-scale",
        "data": "synthetic (acceptance simulated at the stated per-draft rates)",
        "config": {
            "workload": f"{NL} GLM-5.2-shaped routed-MoE layers ("
                        + (f"tiered: {args.slots} HBM slots per layer over pinned host memory, "
                           "caches emptied before each policy" if tiered else "resident")
                        + "); each step decodes one token or verifies it with "
                        f"{D} drafts as one {1 + D}-token batch union per layer; one HIP graph "
                        "per batch size; policies never / always / guard (per-step GPU time "
                        "as the cost, probe every 16 steps, weight 0.25)",
            "value_rate": rates[len(rates) // 2],
        },
        "policies": table,
    }
    print(json.dumps(result), flush=True)
    return 0


def fp8_main(args) -> int:
    """FP8 -> container requantisation of GLM-5.2 expert matrices: each step
    converts one expert's three matrices (three launches of the FP8 kernel),
    cycling over resident experts so that no step's codes are still cached."""
    import numpy as np
    import torch

    import oracle
    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs

    dev = "cuda"
    s = inputs.GLM if args.bits is None else inputs.GLM.with_(bits=args.bits)
    H, I, b = s.hidden, s.inter, s.bits
    K, W, NE = args.steps, args.warmup, 16
    shapes = [(I, H), (I, H), (H, I)]  # gate, up, down
    src = [[inputs.fp8_checkpoint(r, c, 100 + e * 3 + m, dev) for m, (r, c) in enumerate(shapes)]
           for e in range(NE)]
    outs = [(torch.empty(r, c * b // 8, dtype=torch.uint8, device=dev),
             torch.empty(r, device=dev)) for (r, c) in shapes]
    torch.cuda.synchronize()

    def convert(e):
        for m in range(3):
            codes, bs = src[e][m]
            B.coli_quant_pack_fp8(b, codes, bs, outs[m][0], outs[m][1])

    for t in range(W):
        convert(t % NE)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for t in range(K):
        convert(t % NE)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    # each launch's own duration, from events around it on the launch stream;
    # the launches queue behind a short spin on the GPU so that they run
    # back to back (no host launch gap inside an interval)
    KP = min(K, 64)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(KP * 3)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)
    for t in range(KP):
        for m in range(3):
            codes, bs = src[t % NE][m]
            evs[t * 3 + m][0].record()
            B.coli_quant_pack_fp8(b, codes, bs, outs[m][0], outs[m][1])
            evs[t * 3 + m][1].record()
    torch.cuda.synchronize()
    k_ms = float(np.mean([a.elapsed_time(z) for a, z in evs]))

    code_bytes = 3 * H * I
    bscale_bytes = sum(((r + 127) // 128) * ((c + 127) // 128) * 4 for r, c in shapes)
    out_bytes = 3 * H * I * b // 8 + (2 * I + H) * 4
    step_bytes = code_bytes + bscale_bytes + out_bytes
    launch_bytes = step_bytes / 3
    ms_per_step = total_ms / K
    experts_per_s = K / (total_ms / 1e3)
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    k_gbps = launch_bytes / (k_ms * 1e-3) / 1e9
    log(f"[bench] fp8convert: {ms_per_step * 1e3:.2f} us/expert, {experts_per_s:.0f} experts/s, "
        f"{step_bytes / 1e6:.2f} MB/expert -> {gbps:.0f} GB/s; kernel {k_ms * 1e3:.2f} us avg "
        f"-> {k_gbps:.0f} GB/s")

    result = {
        "metric": f"FP8 -> int{b} expert requantisation (GLM-5.2 expert, 128x128 block scales)",
        "value": round(experts_per_s, 1),
        "unit": "experts/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3->fp32->int%d" % b,
        "data": "synthetic",
        "config": {
            "workload": f"one GLM-5.2 expert per step (gate, up 2048 x 6144; down 6144 x 2048) "
                        f"of FP8 E4M3 codes with 128x128 fp32 block scales -> packed int{b} "
                        f"with per-row fp32 scales; {NE} experts resident",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"k_quant_pack_fp8<{b}> (one expert matrix)",
            "achieved": round(k_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(k_gbps / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "avg_launch_us": round(k_ms * 1e3, 3),
            "bytes_per_launch": int(launch_bytes),
        },
    }
    if args.cpu_seconds > 0:
        B.coli_quant_pack_fp8(b, src[0][0][0], src[0][0][1], outs[0][0], outs[0][1])
        torch.cuda.synchronize()
        codes, bs = (t.cpu().numpy() for t in src[0][0])
        t0 = time.perf_counter()
        q_ref, s_ref = oracle.requant_fp8_block(b, codes, bs)
        spent = time.perf_counter() - t0
        same = (np.array_equal(q_ref, outs[0][0].cpu().numpy())
                and np.array_equal(s_ref, outs[0][1].cpu().numpy()))
        result["cpu_baseline"] = {
            "value": round(1.0 / (3 * spent), 3),
            "unit": "experts/s",
            "cores": oracle.num_threads(),
            "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the oracle's dequantisation + requantisation of one 2048 x 6144 gate "
                      f"matrix ({spent:.2f} s), times three for the expert",
        }
        result["cpu_baseline"]["gpu_bytes_equal"] = bool(same)
    print(json.dumps(result), flush=True)
    return 0


def gemv_f32_main(args) -> int:
    """The f32-activation expert GEMV for one token: each step runs it on one
    gate-shaped and one down-shaped matrix of a GLM-5.2 expert, cycling over
    16 resident experts so no step's weights are still cached."""
    import numpy as np
    import torch

    import oracle
    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs

    dev = "cuda"
    s = inputs.GLM if args.bits is None else inputs.GLM.with_(bits=args.bits)
    H, I, b = s.hidden, s.inter, s.bits
    K, W, NE = args.steps, args.warmup, 16
    # stacked: the 16 experts' matrices as one tall matrix of each shape
    shapes = [(NE * I, H), (NE * H, I)] if args.stacked else [(I, H), (H, I)]
    if args.stacked:
        NE = 1
    mats = []
    for e in range(NE):
        row = []
        for m, (r, c) in enumerate(shapes):
            w = inputs.normal((r, c), 0.02, dev, 200 + e, m)
            q = torch.empty(r, c * b // 8, dtype=torch.uint8, device=dev)
            sc = torch.empty(r, device=dev)
            B.coli_quant_pack(b, w, q, sc)
            row.append((q, sc))
            del w
        mats.append(row)
    xs = [inputs.normal((c,), 1.0, dev, 300, m) for m, (r, c) in enumerate(shapes)]
    ys = [torch.empty(r, device=dev) for (r, c) in shapes]
    torch.cuda.synchronize()

    def step(e):
        for m in range(2):
            B.coli_gemv_f32act(b, mats[e][m][0], mats[e][m][1], xs[m], ys[m])

    for t in range(W):
        step(t % NE)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for t in range(K):
        step(t % NE)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    KP = min(K, 64)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(2)] for _ in range(KP)]
    torch.cuda.synchronize()
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(50_000_000)
    for t in range(KP):
        for m in range(2):
            evs[t][m][0].record()
            B.coli_gemv_f32act(b, mats[t % NE][m][0], mats[t % NE][m][1], xs[m], ys[m])
            evs[t][m][1].record()
    torch.cuda.synchronize()
    k_ms = [float(np.mean([evs[t][m][0].elapsed_time(evs[t][m][1]) for t in range(KP)]))
            for m in range(2)]
    mbytes = [r * c * b // 8 + r * 4 + c * 4 + r * 4 for (r, c) in shapes]  # codes, scales, x, y
    gbps = [mbytes[m] / (k_ms[m] * 1e-3) / 1e9 for m in range(2)]
    ms_per_step = total_ms / K
    step_gbps = sum(mbytes) / (ms_per_step * 1e-3) / 1e9
    log(f"[bench] gemvf32 int{b}: {ms_per_step * 1e3:.2f} us per gate + down pair "
        f"({step_gbps:.0f} GB/s); gate-shaped {k_ms[0] * 1e3:.2f} us ({gbps[0]:.0f} GB/s), "
        f"down-shaped {k_ms[1] * 1e3:.2f} us ({gbps[1]:.0f} GB/s)")
    result = {
        "metric": f"f32-activation int{b} expert GEMV, one token (GLM-5.2 gate + down matrices)",
        "value": round(K / (total_ms / 1e3), 1),
        "unit": "matrix pairs/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{b}xf32->f32",
        "data": "synthetic",
        "config": {"workload": (f"one token through 16 GLM-5.2 experts' rows stacked: a "
                                f"{shapes[0][0]} x {shapes[0][1]} and a {shapes[1][0]} x {shapes[1][1]} "
                                f"int{b} matrix with per-row fp32 scales, binary32 activations"
                                if args.stacked else
                                f"one token through a GLM-5.2 expert's gate-shaped (2048 x 6144) "
                                f"and down-shaped (6144 x 2048) int{b} matrices with per-row "
                                f"fp32 scales, binary32 activations; {NE} experts resident")},
        "roofline": {
            "bound": "hbm",
            "kernel": f"k_gemv_f32act<{b}> ({shapes[0][0]} x {shapes[0][1]} matrix)",
            "achieved": round(gbps[0], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps[0] / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "avg_launch_us": round(k_ms[0] * 1e3, 3),
            "bytes_per_launch": int(mbytes[0]),
            "down_shaped_us": round(k_ms[1] * 1e3, 3),
        },
    }
    if args.cpu_seconds > 0:
        q, sc = (t.cpu().numpy() for t in mats[0][0])
        x0 = xs[0].cpu().numpy()[None, :]
        step(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        y_ref = oracle.qdot_f32act(b, q, sc, H, x0)[0]
        spent = time.perf_counter() - t0
        err = float(np.abs(ys[0].cpu().numpy().astype(np.float64) - y_ref).max() / np.abs(y_ref).max())
        result["cpu_baseline"] = {
            "value": round(1.0 / (2 * spent), 2),
            "unit": "matrix pairs/s",
            "cores": oracle.num_threads(),
            "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the oracle's product on one gate-shaped matrix ({spent * 1e3:.1f} ms), "
                      f"twice for the pair; GPU output within {err:.1e} of max |y| of it",
        }
    print(json.dumps(result), flush=True)
    return 0


def stack_cpu_baseline(stk, xs, ws, budget_s):
    """The oracle's own chain for step 0: layer after layer on its own hidden
    state (its logits plus the layer's offsets, its routing, its experts
    packed from the same fp32 draws, untimed; the glue in numpy), until the
    budget is spent; the per-layer time is extrapolated to the whole stack.
    The GPU's hidden state after each of those layers is compared with it."""
    import numpy as np
    import torch

    import oracle
    from quantized_moe_coli_amd import binding as B
    from quantized_moe_coli_amd import inputs, stack

    s = stk.s
    ocfg = oracle.make_cfg(s.n_experts, s.top_k, s.n_group, s.topk_group, 1, s.rsf, s.top_p, 1)
    # the GPU chain for step 0, keeping h after every layer
    h = xs[0].clone()
    y = torch.empty_like(h)
    h_gpu = []
    for li, L in enumerate(stk.layers):
        B.coli_moe_forward(L, stack.rmsnorm(h), y, ws, c_layer=stk.c_layers[li])
        h.add_(y)
        h_gpu.append(h.cpu().numpy())
    hc = xs[0].cpu().numpy().astype(np.float32)
    spent, done, max_err = 0.0, 0, 0.0
    times, first = [], None
    n_all = oracle.num_threads()
    for li, L in enumerate(stk.layers):
        gate_w = L.gate_w.cpu().numpy()
        bias = L.gate_bias.cpu().numpy()
        off = stk.offsets[li].cpu().numpy()
        hd = hc.astype(np.float64)
        hn = (hd / np.sqrt((hd * hd).mean(axis=1, keepdims=True) + stack.RMS_EPS)).astype(np.float32)
        lg = (oracle.logits(hn, gate_w) + off[None, :]).astype(np.float32)
        idx, _ = oracle.route(ocfg, lg, bias)

        def ex(e):
            g, u, d = (t.cpu().numpy() for t in
                       inputs.expert_weights(s, stack.layer_seed(li), e, "cuda"))
            return oracle.Expert.from_float(s.bits, g, u, d)

        exps = [None] * s.n_experts
        for e in set(idx.ravel().tolist()):
            if e >= 0:
                exps[e] = ex(e)
        layer = oracle.Layer(s.hidden, s.inter, s.bits, ocfg, exps, ex(s.n_experts), gate_w, bias)
        if first is None:
            first = (layer, hn, lg)
        t0 = time.perf_counter()
        y_r, _, _, _ = oracle.moe_forward(layer, hn, lg)
        times.append(time.perf_counter() - t0)
        spent += times[-1]
        hc = (hc + y_r).astype(np.float32)
        done += 1
        d = np.abs(h_gpu[li].astype(np.float64) - hc).max() / np.abs(hc).max()
        max_err = max(max_err, float(d))
        if spent >= budget_s * 2 / 3 and done >= 3:
            break
    T = xs.shape[1]
    tok_s = T / (float(np.median(times)) * stk.n_layers)
    # the same first layer on one thread: three samples, median rate
    oracle.set_num_threads(1)
    layer, hn, lg = first
    oracle.moe_forward(layer, hn, lg)  # untimed warm call

    def run_one():
        t0 = time.perf_counter()
        oracle.moe_forward(layer, hn, lg)
        return time.perf_counter() - t0, 1

    one = sorted(c / t for c, t in timed_samples(run_one, budget_s / 3))
    oracle.set_num_threads(n_all)
    tok_s_1 = T * float(np.median(one)) / stk.n_layers
    log(f"[bench] oracle chain, step 0: {done} layers in {spent:.2f}s on {n_all} threads -> "
        f"{tok_s:.3f} tokens/s (median layer) extrapolated to {stk.n_layers} layers, "
        f"{tok_s_1:.4f} on 1 thread; GPU hidden state within {max_err:.2e} (rel. to max |h|) "
        f"of the oracle's over those layers")
    return {
        "value": round(tok_s, 5),
        "unit": "tokens/s",
        "cores": n_all,
        "kind": "oracle",
        "cpu": cpu_model(),
        "single_thread": {"threads": 1, "value": round(tok_s_1, 5),
                          "samples_layers_per_s": [round(r, 4) for r in one]},
        "all_threads": {"threads": n_all, "value": round(tok_s, 5),
                        "layer_seconds": [round(t, 4) for t in times]},
        "sample": f"step 0 ({T} token(s)) through layers 0..{done - 1} of the oracle's own "
                  f"chain on {n_all} threads ({spent:.1f} s of timed forward calls, the median "
                  f"layer time extrapolated to {stk.n_layers} layers); layer 0 again on one "
                  f"thread, three samples, median; the GPU's chained hidden state is within "
                  f"{max_err:.1e} of max |h| of the oracle's (each side chains its own "
                  f"outputs, so a near-tied routing decision can flip an expert and the "
                  f"chains drift; single layers are checked bit-exact in routing by the "
                  f"tests)",
    }


if __name__ == "__main__":
    sys.exit(main())
