#!/usr/bin/env python3
"""Benchmark: sparse FFN decode µs/layer and active-weight HBM GB/s on one MI355X.

Workload (default): the OPT-6.7B-shaped ReLU FFN stack, 32 layers, d=4096, d_ffn=16384,
fp16 weights, predictor rank 256, batch 1, per-layer activity 5% -> 10% (Zipf 1.1), hot
20% of neurons packed first. Every weight, token and profile token is seeded synthetic
data (no model checkpoint, no dataset).

A step is one decode token through every layer of the stack: for each layer, the predictor
(both stages), threshold, compaction, gather-GEMV + ReLU and down projection, all through
the library's single-call decode entry point. Each (token, layer) reads its own pre-drawn
x, so the calibrated activity holds; y is not chained into the next layer. Steps are
replayed from HIP graphs (one per group of tokens) with inputs resident in HBM; the timed
region is bracketed by device synchronizations.

Also measured, beside the headline number:
  - per-kernel durations from HIP events that each kernel dispatch stamps itself
    (start and end of execution, on the library's stream);
  - the dense FFN of the same shapes on the same (unpacked) fp16 weights, through torch
    (hipBLASLt), graph-captured and timed the same way;
  - the fp64 CPU oracle on a bounded sample of the same workload, on the host cores.
Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "sparse FFN decode µs/layer + active-weight HBM GB/s vs peak, 10% activity"


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
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(e.value)

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


def measured_traffic(kernel_file, workload):
    """HBM bytes per dispatch of the dominant kernel from the committed counter summary
    profiles/<kernel>_<workload>_pmc.md (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of
    known size), or None when there is none or the kernel source has changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_file}_{workload}_pmc.md")
    src = os.path.join(ROOT, "activation_sparse_decode_rank_amd", "csrc", "sffn_kernels.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("kernel source sha256") != digest:
        return None
    try:
        return float(fields["traffic bytes per dispatch"])
    except (KeyError, ValueError):
        return None


def kernel_bytes(cfg, n_act):
    """Algorithmic bytes per launch of each decode kernel for one token."""
    sw, sp = cfg.w_bytes, cfg.p_bytes
    d, n, r = cfg.d, cfg.n, cfg.rank
    ma = 2 if cfg.gated else 1
    stage1 = r * d * sp + 4 * d + 4 * r
    mid = n * r * sp + 4 * n + 4 * r + 4 * d + n_act * (ma * d * sw + 4 + 4 + 8 + 4)
    down = n_act * (d * sw + 4 + 4 + 8 + 4 + 8) + 4 * d + 4 * d
    return {"stage1": stage1, "mid": mid, "down": down}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode tokens (each = all layers)")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="C2")
    ap.add_argument("--tokens", type=int, default=256, help="distinct pre-drawn tokens")
    ap.add_argument("--group", type=int, default=8, help="tokens per captured graph")
    ap.add_argument("--profile-tokens", type=int, default=4096)
    ap.add_argument("--kernel-tokens", type=int, default=32, help="tokens in the per-kernel event pass")
    ap.add_argument("--layers", type=int, default=0, help="override the number of layers")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every decode eagerly instead of replaying captured graphs "
                         "(for per-dispatch counter collection; the timing is then not the metric)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB 4 times (the known-size "
                         "kernel that scales HBM counter readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    import torch.nn.functional as F

    from activation_sparse_decode_rank_amd import SparseFFN
    from activation_sparse_decode_rank_amd import _native as NAT
    from synth import get_config, make_layer, make_tokens

    torch.cuda.set_device(0)
    cfg = get_config(args.config)
    L = args.layers or (cfg.rotate_copies if cfg.rotate_copies > 1 else cfg.layers)
    d, n, r = cfg.d, cfg.n, cfg.rank
    G = max(1, args.group)
    T = max(G, (args.tokens // G) * G)
    steps = max(G, ((args.steps + G - 1) // G) * G)
    warmup = ((args.warmup + G - 1) // G) * G
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

    # ------------------------------------------------------------------ offline: layers
    Xprof = make_tokens(cfg, args.profile_tokens, 100, "cuda")
    layers, originals = [], []
    for l in range(L):
        src_layer = 0 if cfg.rotate_copies > 1 else l
        Lt = make_layer(cfg, src_layer, "cuda")
        s = SparseFFN(w_act=Lt.w_a, w_up=Lt.w_u, w_down_t=Lt.w_o, p1=Lt.p1, p2=Lt.p2,
                      b_act=Lt.b_a, b_out=Lt.b_o, p_bias=Lt.c, max_batch=1, profile_x=Xprof,
                      hot_frac=cfg.hot_frac)
        layers.append(s)
        originals.append(Lt)
        if l % 8 == 0 or l == L - 1:
            log(f"layer {l + 1}/{L} generated, profiled and packed")
    del Xprof
    X = make_tokens(cfg, T * L, 200, "cuda").view(T, L, d).contiguous()
    torch.cuda.synchronize()
    log(f"setup {time.time() - t_setup:.1f}s; {T} tokens x {L} layers")

    # ------------------------------------------------------------------ sparse decode graphs
    y_buf = torch.empty((L, 1, d), dtype=torch.float32, device="cuda")
    idx_buf = [torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(L)]
    tok_buf = [torch.empty(n, dtype=torch.int64, device="cuda") for _ in range(L)]
    counts = torch.zeros((T, L), dtype=torch.int32, device="cuda")

    def decode_token(t):
        for l in range(L):
            layers[l].decode(X[t, l:l + 1], y=y_buf[l], idx=idx_buf[l], count=counts[t, l:l + 1],
                             tokmask=tok_buf[l])

    for t in range(min(T, 2)):
        decode_token(t)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    graphs = []
    if not args.no_graph:
        for gi in range(T // G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for t in range(gi * G, (gi + 1) * G):
                    decode_token(t)
            graphs.append(g)
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} graphs of {G * L * 3} kernels")

    def replay(graph_list, ntok):
        if not graph_list:
            for i in range(ntok):
                decode_token(i % T)
            return
        for i in range(ntok // G):
            graph_list[i % len(graph_list)].replay()

    replay(graphs, warmup)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    replay(graphs, steps)
    e1.record()
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / steps
    us_per_layer = ms_per_step * 1000.0 / L
    log(f"sparse decode: {ms_per_step:.4f} ms/token, {us_per_layer:.3f} us/layer")

    cnt = counts.cpu().numpy().astype(np.int64)  # actual active neurons per (token, layer)
    used = [t % T for t in range(steps)]
    n_act_used = cnt[used].astype(np.float64)
    n_act_mean = float(n_act_used.mean())
    m = cfg.m
    b_active = n_act_mean * m * d * cfg.w_bytes
    b_pred = (r * d + n * r) * cfg.p_bytes + 4 * n
    active_gbps = b_active / (us_per_layer * 1e-6) / 1e9

    # ------------------------------------------------------------------ per-kernel event pass
    KT = min(args.kernel_tokens, T)
    hev = HipEvents(6 * KT * L)
    for t in range(KT):
        for l in range(L):
            base = 6 * (t * L + l)
            NAT.sparse_ffn_set_timing_events(layers[l].handle, hev.ev[base:base + 6])
            layers[l].decode(X[t, l:l + 1], y=y_buf[l], idx=idx_buf[l], count=counts[t, l:l + 1],
                             tokmask=tok_buf[l])
    torch.cuda.synchronize()
    for l in range(L):
        NAT.sparse_ffn_set_timing_events(layers[l].handle, None)
    kus = {"stage1": [], "mid": [], "down": []}
    kbytes = {"stage1": [], "mid": [], "down": []}
    for t in range(KT):
        for l in range(L):
            base = 6 * (t * L + l)
            for j, k in enumerate(("stage1", "mid", "down")):
                kus[k].append(1000.0 * hev.elapsed_ms(base + 2 * j, base + 2 * j + 1))
            kb = kernel_bytes(cfg, int(cnt[t, l]))
            for k in kb:
                kbytes[k].append(kb[k])
    hev.close()
    kernels = {}
    for k in kus:
        us = float(np.mean(kus[k]))
        gb = float(np.mean(kbytes[k])) / (us * 1e-6) / 1e9
        kernels[k] = {"avg_us": round(us, 3), "algorithmic_bytes": int(np.mean(kbytes[k])),
                      "gbps": round(gb, 1)}
    dom = max(("mid", "down"), key=lambda k: kernels[k]["avg_us"])
    kname = {"mid": "k_mid_b1 (predictor stage 2 + threshold + compaction + gather-GEMV/ReLU)",
             "down": "k_down (down projection, column-owned)"}[dom]
    log("kernels:", json.dumps(kernels))

    # ------------------------------------------------------------------ dense baseline
    dense = None
    if not args.no_dense:
        X16 = X.half()
        b16 = [o.b_a.half() for o in originals]
        bo16 = [o.b_o.half() for o in originals]

        def dense_token(t):
            for l in range(L):
                o = originals[l]
                x = X16[t, l:l + 1]
                a = F.linear(x, o.w_a, b16[l])
                h = F.relu(a)
                if o.w_u is not None:
                    h = h * F.linear(x, o.w_u)
                _ = torch.matmul(h, o.w_o) + bo16[l]

        for t in range(2):
            dense_token(t)
        torch.cuda.synchronize()
        dgraphs = []
        for gi in range(T // G):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for t in range(gi * G, (gi + 1) * G):
                    dense_token(t)
            dgraphs.append(g)
        replay(dgraphs, warmup)
        torch.cuda.synchronize()
        e0.record()
        replay(dgraphs, steps)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / steps
        dense_us = dms * 1000.0 / L
        dense_bytes = (n * d * (3 if cfg.gated else 2)) * cfg.w_bytes
        dense = {"us_per_layer": round(dense_us, 3),
                 "gbps": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
                 "impl": "torch F.linear/matmul (hipBLASLt), fp16, graph-captured"}
        log(f"dense: {dense_us:.3f} us/layer ({dense['gbps']} GB/s)")
        del dgraphs

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        import oracle
        oracle.load()
        n_cpu_layers = min(L, 2)
        host = [originals[l].numpy() for l in range(n_cpu_layers)]
        Xh = X[:, :n_cpu_layers].cpu().numpy()
        times = []
        t_start = time.time()
        done = 0
        while time.time() - t_start < args.cpu_seconds and done < T * n_cpu_layers:
            t, l = done // n_cpu_layers, done % n_cpu_layers
            Lh = host[l]
            x = np.ascontiguousarray(Xh[t, l:l + 1])
            c0 = time.perf_counter()
            S = oracle.predict(x, Lh["p1"], Lh["p2"], Lh["c"])
            idx, k, tok = oracle.compact(oracle.threshold(S, 0.0))
            _ = oracle.forward(x, Lh["w_a"], Lh["w_o"], idx, tok, Wu=Lh["w_u"], b_a=Lh["b_a"],
                               b_o=Lh["b_o"])
            times.append((time.perf_counter() - c0) * 1e6)
            done += 1
        cpu = {"value": round(float(np.median(times)), 1), "unit": "us/layer", "cores": 1,
               "kind": "oracle",
               "sample": f"{len(times)} (token, layer) decodes of layers 0..{n_cpu_layers - 1}, "
                         f"tokens 0..{(len(times) - 1) // n_cpu_layers}: predict + threshold + "
                         f"compact + forward in fp64, single thread, median"}
        log(f"cpu oracle: {cpu['value']} us/layer over {len(times)} samples")

    # ------------------------------------------------------------------ report
    kd = kernels[dom]
    traffic = measured_traffic({"mid": "k_mid_b1", "down": "k_down"}[dom], cfg.name)
    roof = {"bound": "hbm", "kernel": kname, "achieved": kd["gbps"], "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(kd["gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": (int(traffic) if traffic is not None else None),
            "algorithmic_bytes": kd["algorithmic_bytes"]}
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
            "layers": L, "d": d, "d_ffn": n, "rank": r, "batch": 1,
            "weights": cfg.w_dtype, "predictor": cfg.p_dtype,
            "activity_target": (f"{act_lo:.3f}-{act_hi:.3f}" if act_lo != act_hi else f"{act_lo:.3f}"),
            "tokens": T, "graph_tokens": G,
        },
        "n_act_mean": round(n_act_mean, 1),
        "activity_measured": round(n_act_mean / n, 4),
        "active_weight_bytes_per_layer": int(b_active),
        "predictor_bytes_per_layer": int(b_pred),
        "active_weight_gbps": round(active_gbps, 1),
        "active_weight_frac_of_peak": round(active_gbps / HBM_PEAK_GBPS, 4),
        "layer_gbps_all_bytes": round((b_active + b_pred) / (us_per_layer * 1e-6) / 1e9, 1),
        "kernels": kernels,
        "dense": dense,
        "speedup_vs_dense": (round(dense["us_per_layer"] / us_per_layer, 3) if dense else None),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
