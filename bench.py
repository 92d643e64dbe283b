#!/usr/bin/env python3
"""Benchmark: sparse FFN decode µs/layer and active-weight HBM GB/s on one MI355X.

Workload (default): the OPT-6.7B-shaped ReLU FFN stack with every layer at 10% target
activity (the metric's condition), 32 layers, d=4096, d_ffn=16384, fp16 weights,
predictor rank 256, batch 1, Zipf(1.1) neuron frequencies, hot 20% of neurons packed
first. `--config` selects another workload (C1 OPT-125m layer, C2 the same stack on its
5% -> 10% activity ramp, C3 Llama-7B-shaped gated stack, C4 its batch sweep with
`--batch`, C5 OPT-175B-shaped slice); every weight, token and profile token is seeded
synthetic data (no model checkpoint, no dataset).

A step is one decode token (or one batch of `--batch` tokens) through every layer of the
stack: for each layer, the predictor (both stages), threshold, compaction, gather-GEMV +
ReLU and down projection, all through the library's single-call decode entry point, in
the library's default mode (y bitwise reproducible: the down projection's row splits are
summed in a fixed order). Each
(token, layer) reads its own pre-drawn x, so the calibrated activity holds; y is not
chained into the next layer. Steps are replayed from HIP graphs with inputs resident in
HBM; exactly --steps steps are timed, bracketed by device synchronizations.

Also measured, beside the headline number:
  - the per-layer time of each graph replay in the timed region (p10 / p50 / p90);
  - cache-cold layer times: one-step graphs with a 512 MiB pass over a flush buffer before
    each replay (more than the 256 MB last-level cache), against the same graphs warm
    (`cache_cold`);
  - per-kernel durations from HIP events that each kernel dispatch stamps itself (start and
    end of execution, on the library's stream) over a second eager pass of --kernel-tokens
    steps (the first warms the launch path): the median dispatch, with the mean and the
    p10 / p90 beside it, and each kernel's algorithmic bytes (and,
    for the matrix-core kernels, flops) per launch; the roofline object also times a plain
    read of the dominant kernel's byte count;
  - a plain read stream over 4 GiB (the library's read probe) at 1, 2 and 8 workgroups a
    compute unit: the achievable read bandwidth (the best width), reported beside the
    nominal 8 TB/s peak;
  - the dense FFN two ways: the library itself with every neuron listed (threshold -inf),
    and torch's F.linear chain (hipBLASLt) on the same unpacked fp16 weights, both
    graph-captured and timed the same way, plus the dense bytes at the achievable read rate;
  - the fast mode (the down projection's row splits add into y with float atomics; y may
    vary in the last bits) timed the same way;
  - at one token, the look-ahead decode (each layer's set predicted from the previous
    layer's input, fused into the previous layer's two launches), reported beside the
    metric since its masks differ;
  - the predictor's recall and precision against the true ReLU signs (a diagnostic of the
    synthetic calibrated predictor, not graded);
  - for the default workload, the same stack on its 5% -> 10% ramp (`c2_ramp`);
  - the up projection of the gated Llama-7B shape, whose input is about half zeros, as
    the decode path's row gather against a column-major W_u that skips the zero inputs
    (`input_sparse_up`);
  - the sparse decode against the dense route (every neuron, no predictor) on the
    Llama-7B-shaped gated stack at 16-64 tokens, where the union of the tokens' sets grows,
    and the dense route as 512-token prefill against torch (`dense_crossover`);
  - the fp64 CPU oracle on a bounded sample of the same workload, single-threaded and with
    OpenMP on the host's cores, with the host's core count and CPU model, and the oracle's
    dense FFN (every neuron, one thread);
  - the device, its compute units and peak clocks, and the HIP / ROCm versions (`device`).
Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of the part
TILE_MIN_B = 2                 # from this batch on the decode step runs the matrix-core kernels
METRIC = "sparse FFN decode µs/layer + active-weight HBM GB/s vs peak, 10% activity"
PROBE_BYTES = 4 << 30


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class HipEvents:
    """A pool of hipEvent_t created through the HIP runtime (timing on any stream)."""

    def __init__(self, count):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

    def record(self, i, stream):
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.ev[a], self.ev[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def kernel_source_sha():
    """sha256 over the library's device and host sources (sorted by name)."""
    csrc = os.path.join(ROOT, "activation_sparse_decode_rank_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel_file, workload):
    """HBM bytes per dispatch of the dominant kernel from the committed counter summary
    profiles/<kernel>_<workload>_pmc.md (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of
    known size), or None when there is none or the kernel source has changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel_file}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel source sha256") != kernel_source_sha():
        return None
    try:
        return float(fields["traffic bytes per dispatch"])
    except (KeyError, ValueError):
        return None


def kernel_names(cfg, B):
    """The three kernels the decode step's timing events cover, by path."""
    if B >= TILE_MIN_B and cfg.w_dtype == "f16" and cfg.d % 256 == 0:
        return ("stage1", "up_tiles", "down_tiles"), {
            "stage1": "k_pred_stage1 (predictor stage 1, q = P1 x)",
            "up_tiles": "k_up_mfma (gathered-tile up projection on the matrix cores)",
            "down_tiles": "k_down_mfma (gathered-tile down projection on the matrix cores)"}
    return ("stage1", "mid", "down"), {
        "stage1": "k_pred_stage1 (predictor stage 1, q = P1 x)",
        "mid": ("k_mid_b1" if B == 1 else "k_mid_bt" if B <= 8 else "k_fused_mid")
        + " (predictor stage 2 + threshold + compaction + gather-GEMV/ReLU)",
        "down": ("k_down_b1" if B == 1 else "k_down") + " (down projection over the active rows)"}


def kernel_cost(cfg, B, n_union):
    """Algorithmic bytes and flops per launch of each timed decode kernel for one step
    (n_union: rows in the union list)."""
    sw, sp = cfg.w_bytes, cfg.p_bytes
    d, n, r = cfg.d, cfg.n, cfg.rank
    ma = 2 if cfg.gated else 1
    names, _ = kernel_names(cfg, B)
    stage1 = r * d * sp + 4 * B * d + 4 * B * r
    if names[1] == "mid":
        # P2, biases, q and x; the union's activation rows; activity words, bits and
        # activations out
        mid = n * r * sp + 8 * n + 4 * B * r + 4 * B * d + n_union * (ma * d * sw + 8 + 4 * B)
        # activation rows, activations, list and bits out, y written once
        down = n_union * (d * sw + 4 + 4 * B + 8) + 4 * B * d
        return {"stage1": (stage1, 0.0), "mid": (mid, 0.0), "down": (down, 0.0)}
    up = n_union * (ma * d * sw + 4 + 8 + 4 + 4 * B) + 4 * B * d
    down = n_union * (d * sw + 4 + 4 * B) + 4 * B * d
    # flops of the products as defined (every token against the union rows); the kernels
    # issue each product twice (hi and lo halves of the fp32 activations)
    up_fl = 2.0 * ma * d * n_union * B
    down_fl = 2.0 * d * n_union * B
    return {"stage1": (stage1, 0.0), "up_tiles": (up, up_fl), "down_tiles": (down, down_fl)}


def host_cpu():
    """(nproc, usable cores, CPU model) of this host."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return os.cpu_count() or 1, usable, model


class Timer:
    """Graph-replayed timing of `step_fn(t)` over exactly `steps` steps after `warmup`: graphs
    of G steps (the last one shorter when the count is not a multiple of G), an event
    before and after every replay (per-replay times for percentiles)."""

    def __init__(self, torch, T, G, steps, warmup, cap, use_graphs):
        self.torch, self.T, self.G = torch, T, G
        self.steps, self.warmup, self.cap, self.use_graphs = steps, warmup, cap, use_graphs

    def _plan(self, n):
        full, rem = divmod(n, self.G)
        return [self.G] * full + ([rem] if rem else [])

    def run(self, step_fn):
        torch = self.torch
        G, T = self.G, self.T
        groups = {}
        if self.use_graphs:
            for gi in range(T // G):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=self.cap):
                    for t in range(gi * G, (gi + 1) * G):
                        step_fn(t, self.cap)
                groups.setdefault(G, []).append(g)
            for rem in {len_ for len_ in self._plan(self.steps) + self._plan(self.warmup)
                        if len_ != G}:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=self.cap):
                    for t in range(rem):
                        step_fn(t, self.cap)
                groups[rem] = [g]
            torch.cuda.synchronize()
        cursor = {"i": 0}

        def replay(len_):
            if self.use_graphs:
                lst = groups[len_]
                lst[cursor["i"] % len(lst)].replay()
                cursor["i"] += 1
            else:
                for _ in range(len_):
                    step_fn(cursor["i"] % T, None)
                    cursor["i"] += 1

        for len_ in self._plan(self.warmup):
            replay(len_)
        torch.cuda.synchronize()
        plan = self._plan(self.steps)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan) + 1)]
        torch.cuda.synchronize()
        evs[0].record()
        for i, len_ in enumerate(plan):
            replay(len_)
            evs[i + 1].record()
        torch.cuda.synchronize()
        total = evs[0].elapsed_time(evs[-1])
        per = [evs[i].elapsed_time(evs[i + 1]) / len_ for i, len_ in enumerate(plan)]
        del groups
        return total / self.steps, per


def device_env(torch):
    """The device and software the run used: name, architecture, compute units, peak engine
    and memory clocks (HIP device attributes), HIP, ROCm and torch versions."""
    p = torch.cuda.get_device_properties(0)
    env = {"device": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
           "hbm_bytes": int(p.total_memory), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        env["rocm"] = open("/opt/rocm/.info/version", encoding="utf-8").read().strip()
    except OSError:
        pass
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipDeviceGetAttribute.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_int,
                                              ctypes.c_int]

        def attr(a):
            v = ctypes.c_int()
            return int(v.value) if hip.hipDeviceGetAttribute(ctypes.byref(v), a, 0) == 0 else None

        # hipDeviceAttribute_t values: ClockRate 5 and MemoryClockRate 60 (kHz),
        # MultiprocessorCount 63; the clocks are kept only when the count read the same way
        # agrees with torch's
        if attr(63) == p.multi_processor_count:
            sclk, mclk = attr(5), attr(60)
            if sclk:
                env["sclk_peak_mhz"] = sclk / 1000.0
            if mclk:
                env["mclk_peak_mhz"] = mclk / 1000.0
    except OSError:
        pass
    return env


def run_cold(torch, step_fn, L, T, reps=32, flush_mib=512):
    """Cache-cold layer times: before each replay of a one-step graph (all L layers of one
    step), a torch add over a flush_mib MiB buffer evicts the L2 caches and the 256 MB
    last-level cache; events around the replay alone time it. The same one-step graphs
    replayed back to back without the flush give the warm figure beside it."""
    cap = torch.cuda.Stream()
    K = min(8, T)
    graphs = []
    for t in range(K):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step_fn(t, cap)
        graphs.append(g)
    torch.cuda.synchronize()
    flush = torch.zeros(flush_mib << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for mode in ("warm", "cold"):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        for i in range(reps + K):  # the first K replays are warm-up
            if mode == "cold":
                flush.add_(1)
            j = i - K
            if j >= 0:
                ev[2 * j].record()
            graphs[i % K].replay()
            if j >= 0:
                ev[2 * j + 1].record()
        torch.cuda.synchronize()
        v = np.array([ev[2 * j].elapsed_time(ev[2 * j + 1]) for j in range(reps)]) * 1000.0 / L
        out[mode] = {"us_per_layer_p50": round(float(np.median(v)), 3),
                     "p10": round(float(np.percentile(v, 10)), 3),
                     "p90": round(float(np.percentile(v, 90)), 3)}
    del graphs, flush
    out["cold_over_warm"] = round(out["cold"]["us_per_layer_p50"] / out["warm"]["us_per_layer_p50"], 4)
    out["method"] = (f"one-step graphs ({L} layers, {K} tokens in turn), {reps} timed replays "
                     f"each way; cold: a {flush_mib} MiB read-modify-write pass before every "
                     f"replay, outside the events")
    return out


def percentiles_us(per_step_ms, L):
    v = np.asarray(per_step_ms) * 1000.0 / L
    return {"p10": round(float(np.percentile(v, 10)), 3), "p50": round(float(np.percentile(v, 50)), 3),
            "p90": round(float(np.percentile(v, 90)), 3), "replays": int(len(v))}


def read_probe(torch, NAT, reps=10):
    """Achievable read bandwidth (GB/s): the best of `reps` timed read streams over 4 GiB, for
    each of a few launch widths (1, 2 and 8 workgroups a compute unit); the best width's
    figure is the one reported."""
    buf = torch.empty(PROBE_BYTES, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    widths = [cus, 2 * cus, 8 * cus]
    sink = torch.zeros(max(widths), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    per_width = {}
    for wg in widths:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        NAT.sparse_ffn_read_probe(buf.data_ptr(), PROBE_BYTES, wg, sink.data_ptr(), s.cuda_stream)
        torch.cuda.synchronize()
        for i in range(reps):
            ev[2 * i].record()
            NAT.sparse_ffn_read_probe(buf.data_ptr(), PROBE_BYTES, wg, sink.data_ptr(), s.cuda_stream)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)]
        rates = [PROBE_BYTES / (m * 1e-3) / 1e9 for m in ms]
        per_width[wg] = (max(rates), float(np.median(rates)))
    del buf, sink
    best = max(per_width, key=lambda w: per_width[w][0])
    return {"gbps": round(per_width[best][0], 1), "median_gbps": round(per_width[best][1], 1),
            "bytes": PROBE_BYTES, "reps": reps, "workgroups": best,
            "by_workgroups": {str(w): round(v[0], 1) for w, v in per_width.items()},
            "impl": "sparse_ffn_read_probe: 16-byte non-temporal loads, 8 in flight per thread, "
                    "256-thread workgroups; best of 1, 2 and 8 workgroups a compute unit"}


def sized_read_us(torch, NAT, nbytes, reps=20):
    """The shortest time (us) a plain read of nbytes takes on this device: the read probe over
    a buffer of that size (rounded up to 16 bytes), best of `reps` at each of 1, 2 and 4
    workgroups a compute unit. At a few tens of MB the launch and the first round trip are
    a large part of it, so it bounds a kernel that moves that many bytes more tightly than
    the streaming peak does."""
    nb = (int(nbytes) + 15) // 16 * 16
    buf = torch.ones(nb, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(4 * cus, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream()
    best = float("inf")
    for wg in (cus, 2 * cus, 4 * cus):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
        NAT.sparse_ffn_read_probe(buf.data_ptr(), nb, wg, sink.data_ptr(), s.cuda_stream)
        for i in range(reps):
            ev[2 * i].record()
            NAT.sparse_ffn_read_probe(buf.data_ptr(), nb, wg, sink.data_ptr(), s.cuda_stream)
            ev[2 * i + 1].record()
        torch.cuda.synchronize()
        best = min(best, min(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(reps)) * 1000.0)
    del buf, sink
    return best


def build_stack(cfg, B, L, args, keep_originals, **kw):
    import torch

    from activation_sparse_decode_rank_amd import SparseFFN
    from synth import make_layer, make_tokens
    Xprof = make_tokens(cfg, args.profile_tokens, 100, "cuda")
    layers, originals = [], []
    for l in range(L):
        src_layer = 0 if cfg.rotate_copies > 1 else l
        Lt = make_layer(cfg, src_layer, "cuda")
        s = SparseFFN(w_act=Lt.w_a, w_up=Lt.w_u, w_down_t=Lt.w_o, p1=Lt.p1, p2=Lt.p2,
                      b_act=Lt.b_a, b_out=Lt.b_o, p_bias=Lt.c, max_batch=B, profile_x=Xprof,
                      hot_frac=cfg.hot_frac, **kw)
        layers.append(s)
        originals.append(Lt if keep_originals(l) else None)
        del Lt
        if l % 8 == 0 or l == L - 1:
            log(f"{cfg.name}: layer {l + 1}/{L} generated, profiled and packed")
    del Xprof
    torch.cuda.synchronize()
    return layers, originals


def decode_pass(torch, layers, X, t, y_buf, idx_buf, tok_buf, counts, stream=None):
    for l, s in enumerate(layers):
        s.decode(X[t, l], y=y_buf[l], idx=idx_buf[l], count=counts[t, l:l + 1],
                 tokmask=tok_buf[l], stream=stream)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode steps (each = all layers)")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="C2_10")
    ap.add_argument("--batch", type=int, default=1, help="tokens decoded together per step")
    ap.add_argument("--tokens", type=int, default=256, help="distinct pre-drawn steps")
    ap.add_argument("--group", type=int, default=8, help="steps per captured graph")
    ap.add_argument("--profile-tokens", type=int, default=4096)
    ap.add_argument("--kernel-tokens", type=int, default=32, help="steps in the per-kernel event pass")
    ap.add_argument("--layers", type=int, default=0, help="override the number of layers")
    ap.add_argument("--activity", type=float, default=0.0,
                    help="override every layer's target activity")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-probe", action="store_true", help="skip the 4 GiB read-stream probe")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the all-active, fast-mode, single-pass, recall, ramp and "
                         "crossover legs")
    ap.add_argument("--no-input-sparse", action="store_true",
                    help="skip the input-sparse up projection comparison (rows vs columns)")
    ap.add_argument("--no-crossover", action="store_true",
                    help="skip the sparse-vs-dense crossover on the gated batch stack")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU work per oracle leg (single-threaded, then OpenMP)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every decode eagerly instead of replaying captured graphs "
                         "(for per-dispatch counter collection; the timing is then not the metric)")
    ap.add_argument("--no-lookahead", action="store_true",
                    help="skip the look-ahead decode (next layer's mask predicted from the current "
                         "layer's input, fused into the current layer's two launches; one token), "
                         "which is otherwise timed and reported beside the metric")
    ap.add_argument("--lookahead-streams", action="store_true",
                    help="also time the look-ahead schedule on two streams (separate calls)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB 4 times (the known-size "
                         "kernel that scales HBM counter readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("--steps must be >= 1 and --warmup >= 0")

    import torch
    import torch.nn.functional as F

    from activation_sparse_decode_rank_amd import (LookaheadBuffers, decode_lookahead,
                                                   decode_lookahead_fused)
    from activation_sparse_decode_rank_amd import _native as NAT
    from synth import get_config, make_tokens

    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    if args.activity > 0:
        cfg = dataclasses.replace(cfg, activity=tuple([args.activity] * cfg.layers),
                                  name=f"{cfg.name}_act{args.activity:g}",
                                  description=f"{cfg.description}; every layer at "
                                              f"{100 * args.activity:g}% target activity")
    B = int(args.batch)
    if not 1 <= B <= NAT.SFFN_MAX_BATCH:
        raise SystemExit(f"--batch must be in 1..{NAT.SFFN_MAX_BATCH}")
    L = args.layers or (cfg.rotate_copies if cfg.rotate_copies > 1 else cfg.layers)
    d, n, r = cfg.d, cfg.n, cfg.rank
    G = max(1, args.group)
    T = max(G, (args.tokens // G) * G)
    steps, warmup = int(args.steps), int(args.warmup)
    names, knames = kernel_names(cfg, B)
    t_setup = time.time()
    if args.copy_mib > 0:
        src = torch.ones(args.copy_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 4 x {args.copy_mib} MiB read + {args.copy_mib} MiB written")
        del src, dst

    probe = None
    if not args.no_probe:
        probe = read_probe(torch, NAT)
        log(f"read probe: {probe['gbps']} GB/s best, {probe['median_gbps']} median over 4 GiB")

    # ------------------------------------------------------------------ offline: layers
    layers, originals = build_stack(cfg, B, L, args,
                                    lambda l: not args.no_dense or not args.no_extra
                                    or (not args.no_cpu and l < 2))
    X = make_tokens(cfg, T * L * B, 200, "cuda").view(T, L, B, d).contiguous()
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s; {T} steps x {L} layers x {B} token(s)")

    # ------------------------------------------------------------------ sparse decode graphs
    y_buf = torch.empty((L, B, d), dtype=torch.float32, device="cuda")
    idx_buf = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(L)]
    tok_buf = [torch.empty(n, dtype=torch.int64, device="cuda") for _ in range(L)]
    counts = torch.zeros((T, L), dtype=torch.int32, device="cuda")
    per_tok = np.zeros((T, L), np.int64)  # sum over tokens of each token's own actives

    # one eager pass over every step: union sizes and, for batches, each token's actives
    for t in range(T):
        decode_pass(torch, layers, X, t, y_buf, idx_buf, tok_buf, counts)
        if B > 1:
            torch.cuda.synchronize()
            for l in range(L):
                k = int(counts[t, l].item())
                bits = tok_buf[l][:k].cpu().numpy().view(np.uint64)
                per_tok[t, l] = int(sum(int(((bits >> np.uint64(b)) & np.uint64(1)).sum())
                                        for b in range(B)))
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    timer = Timer(torch, T, G, steps, warmup, cap, not args.no_graph)

    def step(stack):
        return lambda t, s: decode_pass(torch, stack, X, t, y_buf, idx_buf, tok_buf, counts, s)

    ms_per_step, per_replay = timer.run(step(layers))
    us_per_layer = ms_per_step * 1000.0 / L
    log(f"sparse decode: {ms_per_step:.4f} ms/step, {us_per_layer:.3f} us/layer")
    cold = None
    if not args.no_extra and not args.no_graph:
        cold = run_cold(torch, step(layers), L, T)
        log(f"cache-cold: {cold['cold']['us_per_layer_p50']} us/layer against "
            f"{cold['warm']['us_per_layer_p50']} warm (one-step graphs)")

    cnt = counts.cpu().numpy().astype(np.int64)  # union rows per (step, layer)
    if B == 1:
        per_tok = cnt
    n_union_mean = float(cnt.mean())
    n_tok_mean = float(per_tok.mean()) / B
    b_active = n_union_mean * cfg.m * d * cfg.w_bytes  # weight bytes the step must move
    b_pred = (r * d + n * r) * cfg.p_bytes + 4 * n
    active_gbps = b_active / (us_per_layer * 1e-6) / 1e9

    # ------------------------------------------------------------------ look-ahead schedule
    lookahead = None
    if args.lookahead_streams or (B == 1 and not args.no_lookahead):
        lookahead = {"mask": "layer l >= 1 from layer l-1's input (layer l's predictor); layer 0 "
                             "from its own input"}
        side = torch.cuda.Stream()
        la_bufs = LookaheadBuffers(layers, B)

        def la_step(t, stream=None):
            decode_lookahead(layers, [X[t, l] for l in range(L)], la_bufs,
                             stream=stream if stream is not None else torch.cuda.current_stream(),
                             side_stream=side)

        def la_fused_step(t, stream=None):
            decode_lookahead_fused(layers, [X[t, l] for l in range(L)], la_bufs, stream=stream)

        if args.lookahead_streams:
            la_step(0)
            torch.cuda.synchronize()
            la_ms, _ = timer.run(la_step)
            la_us = la_ms * 1000.0 / L
            lookahead.update({"streams_us_per_layer": round(la_us, 3),
                              "streams_speedup_vs_metric_path": round(us_per_layer / la_us, 3),
                              "streams": "separate predict + compact calls on a second stream "
                                         "beside the previous layer's forward"})
            log(f"look-ahead decode (two streams): {la_ms:.4f} ms/step, {la_us:.3f} us/layer")
        if B == 1 and not args.no_lookahead:
            try:
                la_fused_step(0)
                torch.cuda.synchronize()
                fu_ms, _ = timer.run(la_fused_step)
            except Exception as e:  # shapes the fused kernels do not cover
                log(f"fused look-ahead not run: {e}")
            else:
                fu_us = fu_ms * 1000.0 / L
                la_cnt = la_bufs.count.cpu().numpy().astype(np.int64)  # last step's lists
                fu_gbps = float(la_cnt.mean()) * cfg.m * d * cfg.w_bytes / (fu_us * 1e-6) / 1e9
                lookahead.update({
                    "us_per_layer": round(fu_us, 3), "ms_per_step": round(fu_ms, 5),
                    "speedup_vs_metric_path": round(us_per_layer / fu_us, 3),
                    "active_weight_gbps": round(fu_gbps, 1),
                    "active_weight_frac_of_peak": round(fu_gbps / HBM_PEAK_GBPS, 4),
                    "launches": "two a layer: gather + next layer's stage 1, then down "
                                "projection + next layer's scores"})
                log(f"look-ahead decode (fused): {fu_ms:.4f} ms/step, {fu_us:.3f} us/layer")
                # each launch timed by its own dispatch (events pairs 1 and 2 of a handle)
                KT = min(args.kernel_tokens, T)
                fev = HipEvents(6 * KT * L)
                for t in range(KT):
                    layers[0].lookahead_begin(X[t, 0])
                    for l in range(L):
                        base = 6 * (t * L + l)
                        NAT.sparse_ffn_set_timing_events(layers[l].handle, fev.ev[base:base + 6])
                        layers[l].decode_ahead(X[t, l], layers[l + 1] if l + 1 < L else None,
                                               y=la_bufs.y[l], idx=la_bufs.idx[l],
                                               count=la_bufs.count[l:l + 1],
                                               tokmask=la_bufs.tokmask[l])
                        NAT.sparse_ffn_set_timing_events(layers[l].handle, None)
                torch.cuda.synchronize()
                fa = [1000.0 * fev.elapsed_ms(6 * i + 2, 6 * i + 3) for i in range(KT * L)]
                fb = [1000.0 * fev.elapsed_ms(6 * i + 4, 6 * i + 5) for i in range(KT * L)]
                fev.close()
                lookahead["launch_us"] = {"gather_and_next_stage1": round(float(np.mean(fa)), 3),
                                          "down_and_next_scores": round(float(np.mean(fb)), 3)}
        del la_bufs

    # ------------------------------------------------------------------ per-kernel event pass
    KT = min(args.kernel_tokens, T)
    hev = HipEvents(6 * KT * L)
    for rep in range(2):  # the first pass warms the eager launch path; the second is kept
        for t in range(KT):
            for l in range(L):
                base = 6 * (t * L + l)
                NAT.sparse_ffn_set_timing_events(layers[l].handle, hev.ev[base:base + 6])
                layers[l].decode(X[t, l], y=y_buf[l], idx=idx_buf[l], count=counts[t, l:l + 1],
                                 tokmask=tok_buf[l])
        torch.cuda.synchronize()
    for l in range(L):
        NAT.sparse_ffn_set_timing_events(layers[l].handle, None)
    kus = {k: [] for k in names}
    kbytes = {k: [] for k in names}
    kflops = {k: [] for k in names}
    for t in range(KT):
        for l in range(L):
            base = 6 * (t * L + l)
            cost = kernel_cost(cfg, B, int(cnt[t, l]))
            for j, k in enumerate(names):
                kus[k].append(1000.0 * hev.elapsed_ms(base + 2 * j, base + 2 * j + 1))
                kbytes[k].append(cost[k][0])
                kflops[k].append(cost[k][1])
    hev.close()
    kernels = {}
    for k in names:
        # the median dispatch: the eager event pass has a tail of slow dispatches (its mean
        # moved by 10% between runs on one device) that the graph replays of the timed
        # region do not show; their kernel-trace mean agrees with this median within 1%
        v = np.sort(np.asarray(kus[k]))
        us = float(np.median(v))
        gb = float(np.mean(kbytes[k])) / (us * 1e-6) / 1e9
        kernels[k] = {"avg_us": round(us, 3), "algorithmic_bytes": int(np.mean(kbytes[k])),
                      "gbps": round(gb, 1), "estimator": "median of the event pass",
                      "mean_us": round(float(np.mean(v)), 3),
                      "p10_us": round(float(np.percentile(v, 10)), 3),
                      "p90_us": round(float(np.percentile(v, 90)), 3)}
        if np.mean(kflops[k]) > 0:
            tf = float(np.mean(kflops[k])) / (us * 1e-6) / 1e12
            kernels[k]["algorithmic_flops"] = int(np.mean(kflops[k]))
            kernels[k]["tflops"] = round(tf, 2)
            kernels[k]["mfma_util"] = round(tf / MFMA_F16_PEAK_TFLOPS, 5)
    dom = max(names[1:], key=lambda k: kernels[k]["avg_us"])
    log("kernels:", json.dumps(kernels))

    # ------------------------------------------------------------------ extra legs
    dense_bytes = (n * d * (3 if cfg.gated else 2)) * cfg.w_bytes
    all_active = fast_mode = quality = single_pass = None
    if not args.no_extra:
        # the library's own dense FFN: every neuron listed (threshold -inf), same weights
        dense_layers = [s.clone(threshold=float("-inf")) for s in layers]
        aa_ms, _ = timer.run(step(dense_layers))
        aa_us = aa_ms * 1000.0 / L
        all_active = {"us_per_layer": round(aa_us, 3),
                      "gbps": round(dense_bytes / (aa_us * 1e-6) / 1e9, 1),
                      "impl": "this library's decode with threshold -inf (every neuron listed): "
                              "predictor, compaction and the gather kernels over all rows"}
        assert int(counts[0, 0].item()) == n, "all-active leg did not list every neuron"
        log(f"library all-active: {aa_us:.3f} us/layer")
        del dense_layers
        # fast mode (float atomics join the down projection's splits), same masks
        fast_layers = [s.clone(deterministic=False) for s in layers]
        fa_ms, fa_per = timer.run(step(fast_layers))
        fa_us = fa_ms * 1000.0 / L
        fast_mode = {"us_per_layer": round(fa_us, 3),
                     "metric_path_cost_vs_fast": round(us_per_layer / fa_us, 4),
                     "layer_us_percentiles": percentiles_us(fa_per, L),
                     "mode": "deterministic=False: split sums added into y with float atomics"}
        log(f"fast mode (atomics): {fa_us:.3f} us/layer")
        del fast_layers
        # the single-pass decode (gather and down rows in one pass, fixed-order reduction)
        if B == 1:
            sp_layers = [s.clone(single_pass=True) for s in layers]
            sp_ms, sp_per = timer.run(step(sp_layers))
            sp_us = sp_ms * 1000.0 / L
            single_pass = {"split_layout_us_per_layer": round(sp_us, 3),
                           "speedup_vs_metric_path": round(us_per_layer / sp_us, 4)}
            log(f"single pass (split layout): {sp_us:.3f} us/layer")
            del sp_layers
        # predictor recall / precision against the true ReLU signs on sampled steps
        tp = fp = fn = 0
        ns = min(8, T)
        for t in range(ns):
            decode_pass(torch, layers, X, t, y_buf, idx_buf, tok_buf, counts)
            torch.cuda.synchronize()
            for l in range(L):
                o = originals[l]
                a = F.linear(X[t, l], o.w_a.float(), o.b_a)           # [B, n] true ReLU input
                k = int(counts[t, l].item())
                pidx = layers[l].perm_dev[idx_buf[l][:k].long()]       # original neuron ids
                bits = tok_buf[l][:k]
                for b in range(B):
                    pm = torch.zeros(n, dtype=torch.bool, device="cuda")
                    sel = ((bits >> b) & 1).bool() if B > 1 else torch.ones(k, dtype=torch.bool,
                                                                              device="cuda")
                    pm[pidx[sel]] = True
                    tm = a[b] > 0
                    tp += int((pm & tm).sum())
                    fp += int((pm & ~tm).sum())
                    fn += int((~pm & tm).sum())
        quality = {"recall": round(tp / max(tp + fn, 1), 4),
                   "precision": round(tp / max(tp + fp, 1), 4),
                   "sample": f"{ns} steps x {L} layers x {B} token(s); true mask = fp32 "
                             f"W_a x + b_a > 0 (torch), predicted = the decode's list",
                   "note": "synthetic calibrated random-subspace predictor (no trained "
                           "predictor exists here): a diagnostic, not graded"}
        log(f"predictor recall {quality['recall']}, precision {quality['precision']}")

    # the single-pass decode over neuron bundles: its own packed copy of the stack
    if single_pass is not None:
        bl, _ = build_stack(cfg, B, L, args, lambda l: False, bundle=True, single_pass=True)
        bu_ms, bu_per = timer.run(step(bl))
        bu_us = bu_ms * 1000.0 / L
        KT2 = min(args.kernel_tokens, T)
        bev = HipEvents(6 * KT2 * L)
        for t in range(KT2):
            for l in range(L):
                base = 6 * (t * L + l)
                NAT.sparse_ffn_set_timing_events(bl[l].handle, bev.ev[base:base + 6])
                bl[l].decode(X[t, l], y=y_buf[l], idx=idx_buf[l], count=counts[t, l:l + 1],
                             tokmask=tok_buf[l])
                NAT.sparse_ffn_set_timing_events(bl[l].handle, None)
        torch.cuda.synchronize()
        bk = {}
        for j, k in enumerate(("stage1", "bundle_pass", "reduce")):
            bk[k] = round(float(np.mean([1000.0 * bev.elapsed_ms(6 * i + 2 * j, 6 * i + 2 * j + 1)
                                         for i in range(KT2 * L)])), 3)
        bev.close()
        pass_bytes = [n * r * cfg.p_bytes + 8 * n + 4 * r + 4 * d
                      + int(cnt[t, l]) * (cfg.m * d * cfg.w_bytes + 8) for t in range(KT2)
                      for l in range(L)]
        pb_mean = float(np.mean(pass_bytes))
        single_pass.update({
            "bundle_layout_us_per_layer": round(bu_us, 3),
            "bundle_speedup_vs_metric_path": round(us_per_layer / bu_us, 4),
            "bundle_layer_us_percentiles": percentiles_us(bu_per, L),
            "kernel_us": bk,
            "bundle_pass_algorithmic_bytes": int(pb_mean),
            "bundle_pass_gbps": round(pb_mean / (bk["bundle_pass"] * 1e-6) / 1e9, 1),
            "impl": "stage 1, then k_bundle_b1 (scores, threshold, compaction, and each active "
                    "neuron's input and down rows in one batch of loads; partial outputs of four "
                    "ranges per workgroup), then k_bundle_reduce (fixed-order sum + list)"})
        log(f"single pass (bundle layout): {bu_us:.3f} us/layer; kernels {bk}")
        del bl

    # ------------------------------------------------------------------ dense baseline
    dense = None
    if not args.no_dense:
        wdt = originals[0].w_a.dtype  # the dense chain computes in the weights' dtype
        Xw = X.to(wdt)
        bw = [o.b_a.to(wdt) for o in originals]
        bow = [o.b_o.to(wdt) for o in originals]

        def dense_step(t, stream=None):
            for l in range(L):
                o = originals[l]
                x = Xw[t, l]
                a = F.linear(x, o.w_a, bw[l])
                h = F.relu(a)
                if o.w_u is not None:
                    h = h * F.linear(x, o.w_u)
                _ = torch.matmul(h, o.w_o) + bow[l]

        for t in range(2):
            dense_step(t)
        torch.cuda.synchronize()
        dms, _ = timer.run(dense_step)
        dense_us = dms * 1000.0 / L
        dense = {"us_per_layer": round(dense_us, 3),
                 "gbps": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                 "dense_weight_bytes_per_layer": int(dense_bytes),
                 "impl": f"torch F.linear/matmul (hipBLASLt/rocBLAS), {cfg.w_dtype}, {B} token(s), "
                         f"graph-captured"}
        if all_active:
            dense["library_all_active"] = all_active
        if probe:
            dense["ideal_us_at_achievable_peak"] = round(dense_bytes / (probe["gbps"] * 1e9) * 1e6, 3)
        log(f"dense: {dense_us:.3f} us/layer ({dense['gbps']} GB/s)")
        del Xw

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle
        oracle.load()
        n_cpu_layers = min(L, 2)
        host = [originals[l].numpy() for l in range(n_cpu_layers)]
        Xh = X[:, :n_cpu_layers].cpu().numpy()

        def time_oracle(seconds):
            times = []
            t_start = time.time()
            done = 0
            while time.time() - t_start < seconds and done < T * n_cpu_layers:
                t, l = done // n_cpu_layers, done % n_cpu_layers
                Lh = host[l]
                x = np.ascontiguousarray(Xh[t, l])
                c0 = time.perf_counter()
                S = oracle.predict(x, Lh["p1"], Lh["p2"], Lh["c"])
                idx, k, tok = oracle.compact(oracle.threshold(S, 0.0))
                _ = oracle.forward(x, Lh["w_a"], Lh["w_o"], idx, tok, Wu=Lh["w_u"], b_a=Lh["b_a"],
                                   b_o=Lh["b_o"])
                times.append((time.perf_counter() - c0) * 1e6)
                done += 1
            return times

        nproc, usable, model = host_cpu()
        t1 = time_oracle(args.cpu_seconds)
        single = {"value": round(float(np.median(t1)), 1), "unit": "us/layer", "cores": 1,
                  "samples": len(t1)}
        log(f"cpu oracle, 1 thread: {single['value']} us/layer over {len(t1)} samples")
        prev = oracle.set_library(oracle.open_library(oracle.OMP_LIB_PATH))
        try:
            threads = oracle.threads()
            tm = time_oracle(args.cpu_seconds)
        finally:
            oracle.set_library(prev)
        cpu = {"value": round(float(np.median(tm)), 1), "unit": "us/layer", "cores": threads,
               "kind": "oracle",
               "sample": f"{len(tm)} (step, layer) decodes of {B} token(s), layers "
                         f"0..{n_cpu_layers - 1}: predict + threshold + compact + forward in "
                         f"fp64 (OpenMP over neurons and output columns, {threads} threads), "
                         f"median; single_thread: the same, one thread",
               "nproc": nproc, "usable_cores": usable, "cpu_model": model,
               "single_thread": single}
        log(f"cpu oracle, OpenMP {threads} threads: {cpu['value']} us/layer over {len(tm)} samples "
            f"({model}, nproc {nproc})")
        if B == 1:
            # the dense FFN on the CPU: every neuron, no predictor, in the oracle's fp64
            # arithmetic (its dense routine is single-threaded)
            td, t_start = [], time.time()
            while (time.time() - t_start < args.cpu_seconds / 2 and len(td) < 64) or len(td) < 3:
                l = len(td) % n_cpu_layers
                Lh = host[l]
                x = np.ascontiguousarray(Xh[len(td) % T, l])
                c0 = time.perf_counter()
                _ = oracle.dense(x, Lh["w_a"], Lh["w_o"], Wu=Lh["w_u"], b_a=Lh["b_a"],
                                 b_o=Lh["b_o"])
                td.append((time.perf_counter() - c0) * 1e6)
            cpu["dense_ffn"] = {"value": round(float(np.median(td)), 1), "unit": "us/layer",
                                "cores": 1, "samples": len(td),
                                "what": "the FFN over every neuron (no predictor), fp64 oracle "
                                        "arithmetic, one thread"}
            log(f"cpu dense FFN, 1 thread: {cpu['dense_ffn']['value']} us/layer")
        del host, Xh

    # ------------------------------------------------------------------ the 5% -> 10% ramp
    ramp = None
    if not args.no_extra and cfg.name == "opt6.7b_stack_10pct" and B == 1 and not args.layers:
        layers = originals = None  # free the headline stack before building the ramp's
        ramp = run_ramp(torch, args, timer, dense)

    crossover = input_sparse = None
    if not args.no_extra and not args.no_crossover and B == 1:
        layers = originals = None
        crossover = run_crossover(torch, args, cap)
    if not args.no_extra and not args.no_input_sparse and B == 1:
        layers = originals = None
        input_sparse = run_input_sparse_up(torch, args, NAT)

    # ------------------------------------------------------------------ report
    kd = kernels[dom]
    kfile = knames[dom].split(" ")[0]
    traffic = measured_traffic(kfile, f"{cfg.name}_b{B}")
    roof = {"bound": "hbm", "kernel": knames[dom], "achieved": kd["gbps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(kd["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": (int(traffic) if traffic is not None else None),
            "algorithmic_bytes": kd["algorithmic_bytes"]}
    if probe:
        roof["achievable_peak"] = probe["gbps"]
        roof["frac_of_achievable"] = round(kd["gbps"] / probe["gbps"], 4)
        # a plain read of the same byte count, timed the same way: the kernel's time against
        # the shortest time that many bytes take on this device at all
        sr = sized_read_us(torch, NAT, kd["algorithmic_bytes"])
        roof["size_matched_read_us"] = round(sr, 3)
        roof["kernel_us"] = kd["avg_us"]
        roof["frac_of_size_matched_read"] = round(sr / kd["avg_us"], 4)
        log(f"a plain read of the dominant kernel's {kd['algorithmic_bytes']} bytes: {sr:.3f} us "
            f"(kernel {kd['avg_us']} us)")
    if "mfma_util" in kd:
        # the matrix-core kernels stay bound by HBM at these arithmetic intensities; their
        # flops rate against the fp16 matrix-core peak rides along
        roof["mfma"] = {"achieved_tflops": kd["tflops"], "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                        "util": kd["mfma_util"]}
    act_lo, act_hi = min(cfg.activity), max(cfg.activity)
    out = {
        "metric": METRIC,
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "layers": L, "d": d, "d_ffn": n, "rank": r, "batch": B,
            "weights": cfg.w_dtype, "predictor": cfg.p_dtype,
            "activity_target": (f"{act_lo:.3f}-{act_hi:.3f}" if act_lo != act_hi else f"{act_lo:.3f}"),
            "tokens": T, "graph_steps": G,
            "mode": "deterministic (y bitwise reproducible; the library's default)",
        },
        "layer_us_percentiles": percentiles_us(per_replay, L),
        "n_act_mean": round(n_tok_mean, 1),
        "n_union_mean": round(n_union_mean, 1),
        "activity_measured": round(n_tok_mean / n, 4),
        "union_fraction": round(n_union_mean / n, 4),
        "active_weight_bytes_per_layer": int(b_active),
        "predictor_bytes_per_layer": int(b_pred),
        "active_weight_gbps": round(active_gbps, 1),
        "active_weight_frac_of_peak": round(active_gbps / HBM_PEAK_GBPS, 4),
        "layer_gbps_all_bytes": round((b_active + b_pred) / (us_per_layer * 1e-6) / 1e9, 1),
        "kernels": kernels,
        "dense": dense,
        "speedup_vs_dense": (round(dense["us_per_layer"] / us_per_layer, 3) if dense else None),
        "speedup_vs_library_all_active": (round(all_active["us_per_layer"] / us_per_layer, 3)
                                          if all_active else None),
        "speedup_vs_ideal_dense": (round(dense["ideal_us_at_achievable_peak"] / us_per_layer, 3)
                                   if dense and "ideal_us_at_achievable_peak" in dense else None),
        "roofline": roof,
        "hbm_read_probe": probe,
        "fast_mode": fast_mode,
        "input_sparse_up": input_sparse,
        "single_pass": single_pass,
        "predictor_quality": quality,
        "cpu_baseline": cpu,
        "cache_cold": cold,
        "device": device_env(torch),
        "lookahead": lookahead,
        "c2_ramp": ramp,
        "dense_crossover": crossover,
        "kernel_source_sha256": kernel_source_sha(),
    }
    if lookahead and dense and "us_per_layer" in lookahead:
        lookahead["speedup_vs_dense"] = round(dense["us_per_layer"] / lookahead["us_per_layer"], 3)
    print(json.dumps(out), flush=True)


def run_crossover(torch, args, cap):
    """The sparse decode against the dense route (every neuron, no predictor) on the
    Llama-7B-shaped gated stack with independent per-token masks, at growing batches: the
    union of the tokens' sets grows with the batch until the sparse path stops paying. Also
    the dense route as prefill (512 tokens) against torch's F.linear chain on the same
    weights, on the first four layers."""
    import torch.nn.functional as F
    from synth import get_config, make_tokens
    cfg = get_config("C4")
    L, d, n = cfg.layers, cfg.d, cfg.n
    Bmax = 64
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    layers, originals = build_stack(cfg, Bmax, L, args, lambda l: l < 4)
    T, G = 16, 4
    X = make_tokens(cfg, T * L * Bmax, 200, "cuda").view(T, L, Bmax, d).contiguous()
    y_buf = torch.empty((L, Bmax, d), dtype=torch.float32, device="cuda")
    idx_buf = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(L)]
    tok_buf = [torch.empty(n, dtype=torch.int64, device="cuda") for _ in range(L)]
    counts = torch.zeros((T, L), dtype=torch.int32, device="cuda")
    timer = Timer(torch, T, G, 16, 4, cap, True)
    rows = []
    for B in (16, 32, 48, 64):
        Xb = X[:, :, :B].contiguous()
        for t in range(T):
            decode_pass(torch, layers, Xb, t, y_buf, idx_buf, tok_buf, counts)
        torch.cuda.synchronize()
        union = float(counts.float().mean()) / n
        sp_ms, _ = timer.run(lambda t, st: decode_pass(torch, layers, Xb, t, y_buf, idx_buf,
                                                       tok_buf, counts, st))
        de_ms, _ = timer.run(lambda t, st: [layers[l].dense(Xb[t, l], y=y_buf[l, :B], stream=st)
                                            for l in range(L)])
        rows.append({"batch": B, "union_fraction": round(union, 4),
                     "sparse_us_per_layer": round(sp_ms * 1000.0 / L, 3),
                     "dense_route_us_per_layer": round(de_ms * 1000.0 / L, 3)})
        log(f"crossover B={B}: union {union:.3f}, sparse {rows[-1]['sparse_us_per_layer']} us, "
            f"dense route {rows[-1]['dense_route_us_per_layer']} us")
    cross = next((r_["union_fraction"] for r_ in rows
                  if r_["dense_route_us_per_layer"] < r_["sparse_us_per_layer"]), None)
    # prefill: 512 tokens through the first four layers
    P, LP = 512, 4
    Xp = make_tokens(cfg, P * LP, 300, "cuda").view(LP, P, d).contiguous()
    yp = torch.empty((LP, P, d), dtype=torch.float32, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def time_fn(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    lib_ms = time_fn(lambda: [layers[l].dense(Xp[l], y=yp[l]) for l in range(LP)])
    pf_work = layers[0].prefill_work(P)
    pf_ms = time_fn(lambda: [layers[l].prefill(Xp[l], y=yp[l], work=pf_work) for l in range(LP)])
    pf16_ms = time_fn(lambda: [layers[l].prefill(Xp[l], y=yp[l], work=pf_work,
                                                 fp16_activations=True) for l in range(LP)])
    Xh = Xp.half()

    def torch_prefill():
        for l in range(LP):
            o = originals[l]
            a = F.linear(Xh[l], o.w_a, o.b_a.half())
            h = F.relu(a) * F.linear(Xh[l], o.w_u)
            _ = torch.matmul(h, o.w_o) + o.b_o.half()

    th_ms = time_fn(torch_prefill)
    # algorithmic flops of the dense FFN per layer (the products as defined, once)
    pf_flops = 2.0 * P * n * d * (3 if cfg.gated else 2)
    out_pf = {
        "prefill_ms_per_layer": round(pf_ms / LP, 4),
        "prefill_tokens_per_s": round(P / (pf_ms / LP * 1e-3), 1),
        "prefill_tflops": round(pf_flops / (pf_ms / LP * 1e-3) / 1e12, 2),
        "prefill_mfma_frac": round(pf_flops / (pf_ms / LP * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
        "prefill_fp16_act_ms_per_layer": round(pf16_ms / LP, 4),
        "prefill_fp16_act_tflops": round(pf_flops / (pf16_ms / LP * 1e-3) / 1e12, 2),
        "dense_route_ms_per_layer": round(lib_ms / LP, 4),
        "torch_ms_per_layer": round(th_ms / LP, 4),
        "torch_fp16_tokens_per_s": round(P / (th_ms / LP * 1e-3), 1),
        "note": "per layer. prefill: sparse_ffn_prefill (128 x 128 tiles on the matrix cores, each "
                "weight tile read once per 128 tokens; fp32 activations as hi + lo fp16 pairs, so "
                "the matrix cores run twice the algorithmic products); prefill_fp16_act: the same "
                "kernels with x and h rounded to fp16 once (SFFN_PREFILL_FP16_ACT), one product "
                "each, torch's activation precision. dense_route: "
                "sparse_ffn_dense over the decode kernels, 64 tokens per pass. torch: fp16 "
                "activations through hipBLASLt"}
    # a short prompt: 128 tokens (one token tile) of the same layers
    S_ = 128
    pf_ms_s = time_fn(lambda: [layers[l].prefill(Xp[l][:S_], y=yp[l][:S_], work=pf_work)
                               for l in range(LP)])
    pf16_ms_s = time_fn(lambda: [layers[l].prefill(Xp[l][:S_], y=yp[l][:S_], work=pf_work,
                                                   fp16_activations=True) for l in range(LP)])
    lib_ms_s = time_fn(lambda: [layers[l].dense(Xp[l][:S_], y=yp[l][:S_]) for l in range(LP)])

    def torch_prefill_short():
        for l in range(LP):
            o = originals[l]
            a = F.linear(Xh[l][:S_], o.w_a, o.b_a.half())
            h = F.relu(a) * F.linear(Xh[l][:S_], o.w_u)
            _ = torch.matmul(h, o.w_o) + o.b_o.half()

    th_ms_s = time_fn(torch_prefill_short)
    out_pf_short = {
        "prefill_ms_per_layer": round(pf_ms_s / LP, 4),
        "prefill_fp16_act_ms_per_layer": round(pf16_ms_s / LP, 4),
        "dense_route_ms_per_layer": round(lib_ms_s / LP, 4),
        "torch_ms_per_layer": round(th_ms_s / LP, 4)}
    out = {"workload": f"{cfg.name}: {cfg.description}", "rows": rows,
           "crossover_union_fraction": cross,
           "note": "dense route = every neuron through the forward kernels (tile path), no "
                   "predictor; the decode switches to it when sffn_desc.dense_union is set and "
                   "the expected union exceeds it",
           "prefill_512_tokens": out_pf, "prefill_128_tokens": out_pf_short}
    log(f"prefill 512 tokens: library prefill {pf_ms / LP:.3f} ms/layer "
        f"({out_pf['prefill_tflops']} TFLOP/s), fp16 activations {pf16_ms / LP:.3f}, "
        f"dense route {lib_ms / LP:.3f}, torch "
        f"{th_ms / LP:.3f} ms/layer")
    log(f"prefill 128 tokens: library prefill {pf_ms_s / LP:.3f} ms/layer, fp16 activations "
        f"{pf16_ms_s / LP:.3f}, dense route {lib_ms_s / LP:.3f}, torch {th_ms_s / LP:.3f}")
    del layers, originals
    return out


def run_input_sparse_up(torch, args, NAT):
    """The up projection of the ReLU-fied gated shape, whose input x = relu(rmsnorm(z)) is
    about half zeros (novita.ai activation-sparsity article, section 第二階段), two ways for
    the same listed neurons: gathering their rows of W_u (the decode path's layout) and a
    column-major copy of W_u that skips zero inputs and 16-byte pieces without a listed
    neuron (the library's sparse_ffn_up_probe). Eight layers, packed hot-first, each with
    the list its own decode step publishes for its token; each way captured as one graph of
    the eight calls and replayed."""
    from synth import get_config, make_tokens
    cfg = get_config("C3")
    L, d, n = 8, cfg.d, cfg.n
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    layers, originals = build_stack(cfg, 1, L, args, lambda l: True)
    X = make_tokens(cfg, L, 700, "cuda").view(L, 1, d).contiguous()
    rows_w, cols_w, idx_l, cnt_l, words_l = [], [], [], [], []
    row_bytes = col_bytes = col_lines = 0
    zeros = []
    for l in range(L):
        _, idx, count, _ = layers[l].decode(X[l])
        torch.cuda.synchronize()
        k = int(count.item())
        perm = torch.as_tensor(layers[l].perm, device="cuda").long()
        wr = originals[l].w_u.index_select(0, perm).contiguous()
        rows_w.append(wr)
        cols_w.append(wr.t().contiguous())
        idx_l.append(idx)
        cnt_l.append(count)
        ih = idx[:k].cpu().numpy().astype(np.int64)
        w = np.zeros((n + 63) // 64, np.uint64)
        np.bitwise_or.at(w, ih // 64, np.left_shift(np.uint64(1), (ih % 64).astype(np.uint64)))
        words_l.append(torch.from_numpy(w.view(np.int64)).cuda())
        nz = int((X[l] != 0).sum())
        zeros.append(1.0 - nz / d)
        live = np.zeros(n // 8, bool)
        live[ih // 8] = True
        lines = np.zeros((n + 63) // 64, bool)
        lines[ih // 64] = True
        row_bytes += k * d * 2
        col_bytes += nz * int(live.sum()) * 16
        col_lines += nz * int(lines.sum()) * 128
    del layers, originals
    u = torch.empty((L, n), dtype=torch.float32, device="cuda")
    wb = NAT.sparse_ffn_up_probe_work_bytes(n)
    work = torch.empty(wb // 4, dtype=torch.float32, device="cuda")

    def run(layout, st):
        for l in range(L):
            if layout == NAT.SFFN_UP_ROWS:
                NAT.sparse_ffn_up_probe(rows_w[l].data_ptr(), layout, d, n, X[l].data_ptr(),
                                        idx_l[l].data_ptr(), cnt_l[l].data_ptr(), None,
                                        u[l].data_ptr(), None, 0, st)
            else:
                NAT.sparse_ffn_up_probe(cols_w[l].data_ptr(), layout, d, n, X[l].data_ptr(),
                                        None, None, words_l[l].data_ptr(), u[l].data_ptr(),
                                        work.data_ptr(), wb, st)

    side = torch.cuda.Stream()
    out = {"workload": f"{cfg.name} shape, {L} layers, one token each",
           "zero_input_fraction": round(float(np.mean(zeros)), 4),
           "listed_rows_mean": round(row_bytes / (d * 2) / L, 1)}
    reps = 32
    for name, layout in (("rows", NAT.SFFN_UP_ROWS), ("columns", NAT.SFFN_UP_COLUMNS)):
        run(layout, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run(layout, side.cuda_stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        g.replay()
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            g.replay()
        ev[1].record()
        torch.cuda.synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1000.0 / (reps * L)
        out[name + "_us_per_layer"] = round(us, 3)
        del g
    out["rows_bytes_per_layer"] = int(row_bytes / L)
    out["columns_bytes_read_per_layer"] = int(col_bytes / L)
    out["columns_128B_lines_touched_per_layer"] = int(col_lines / L)
    out["columns_vs_rows_time"] = round(out["columns_us_per_layer"] / out["rows_us_per_layer"], 3)
    out["note"] = ("rows: the listed neurons' W_u rows, every input; columns: W_u transposed, "
                   "inputs with x_j = 0 and pieces of 8 neurons with none listed skipped, plus "
                   "a fixed-order sum of 16 input splits")
    log(f"input-sparse up probe: rows {out['rows_us_per_layer']} us, columns "
        f"{out['columns_us_per_layer']} us per layer")
    return out


def run_ramp(torch, args, timer, dense):
    """The OPT-6.7B stack on its 5% -> 10% per-layer activity ramp (same weights, biases
    set for the ramp): the headline path only, timed the same way."""
    from synth import get_config, make_tokens
    cfg = get_config("C2")
    L, d, n = cfg.layers, cfg.d, cfg.n
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    layers, _ = build_stack(cfg, 1, L, args, lambda l: False)
    X = make_tokens(cfg, timer.T * L, 200, "cuda").view(timer.T, L, 1, d).contiguous()
    y_buf = torch.empty((L, 1, d), dtype=torch.float32, device="cuda")
    idx_buf = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(L)]
    tok_buf = [torch.empty(n, dtype=torch.int64, device="cuda") for _ in range(L)]
    counts = torch.zeros((timer.T, L), dtype=torch.int32, device="cuda")
    for t in range(timer.T):
        decode_pass(torch, layers, X, t, y_buf, idx_buf, tok_buf, counts)
    torch.cuda.synchronize()
    ms, per = timer.run(lambda t, s: decode_pass(torch, layers, X, t, y_buf, idx_buf, tok_buf,
                                                 counts, s))
    us = ms * 1000.0 / L
    cnt = counts.cpu().numpy().astype(np.int64)
    b_active = float(cnt.mean()) * cfg.m * d * cfg.w_bytes
    gbps = b_active / (us * 1e-6) / 1e9
    log(f"C2 ramp: {us:.3f} us/layer")
    out = {"workload": f"{cfg.name}: {cfg.description}", "us_per_layer": round(us, 3),
           "layer_us_percentiles": percentiles_us(per, L),
           "activity_measured": round(float(cnt.mean()) / n, 4),
           "active_weight_gbps": round(gbps, 1),
           "active_weight_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
    if dense:  # the same weight shapes: the dense time does not depend on the activity
        out["speedup_vs_dense"] = round(dense["us_per_layer"] / us, 3)
    del layers
    return out


if __name__ == "__main__":
    main()
