#!/usr/bin/env python3
"""Benchmark: RACE attention forward + backward on one MI355X.

One step = race_attn_forward + race_attn_backward (the whole hot path) over
the workload's synthetic, seeded inputs, already resident in HBM.  Prints one
JSON line with tokens/s, the roofline position of the dominant kernel
(timed live with HIP events recorded by the library around each kernel) and
the fp64 oracle timed on the host cores on a bounded prefix of the same
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "RACE attn fwd+bwd tokens/s at N=4M causal d=64; % of MFMA/HBM roofline"


def metric_name(w) -> str:
    """The headline workload keeps the library's headline metric string; the
    others name their own shape and passes."""
    if w.name == "causal_n4m_bf16":
        return METRIC
    passes = "fwd+bwd" if w.backward else "fwd"
    mode = "causal" if w.causal else "non-causal"
    n = f"{w.N / 1e6:g}M" if w.N >= 1_000_000 else (f"{w.N // 1024}K" if w.N % 1024 == 0 else str(w.N))
    heads = f" B*H={w.B * w.H}" if w.B * w.H > 1 else ""
    tail = ("; latency-bound, see latency_us" if not w.backward and w.tokens <= 4096
            else "; % of MFMA/HBM roofline")
    return (f"RACE attn {passes} tokens/s at N={n}{heads} {mode} d={w.d} L={w.L} {w.dtype}"
            f"{tail}")

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}


def algorithmic_per_token(w, dw: bool = False, saved: bool = True):
    """Algorithmic work of the method per token (one (b, h) row).

    flops: projections 2 d L P per hashed row (Q and K in the forward, and
    the dx_hat = du W product of Q and of K in the backward), sketch and
    readout 2 F (d+1) each, the query-side gradient 2 F (d+1), the gradient
    sketch 2 F (d+1), dV and dphi(k) 2 F d each.  saved = False: the
    backward also recomputes the hash of Q and K (2 d L P each); with the
    forward's saved state (how the step is timed) it reads them instead.
    bytes: one read of every input and one write of every output per pass.
    dw: the backward also forms the projection gradient, 2 d L P per row of Q
    (in dq) and of K (in dk).
    """
    d, L, P = w.d, w.L, w.P
    F, d1 = L * (1 << P), d + 1
    e = 2 if w.dtype == "bf16" else 4
    proj = 2 * d * L * P
    # kernels that hash their own rows carry those projections
    rehash = 0 if saved else proj
    per_kernel = {
        # fused kernels (bf16, L <= 32)
        "sum_kv": proj + 2 * F * d1,            # hash K, sketch of the keys
        "fwd_o": proj + 2 * F * d1,             # hash Q, readout
        "sum_qd": rehash + 2 * F * d1,          # (recomputed hash Q), gradient sketch
        "dq": 2 * F * d1 + proj,                # query-side gradient, dx_hat = du W
        "dk": rehash + 2 * F * d + proj,        # (recomputed hash K), dphi(k), dx_hat = du W
        "dv": 2 * F * d,                        # dV readout
        # unfused kernels (fp32, L > 32)
        "hash_q": proj, "hash_k": proj,
        "seg_sum_kv": 2 * F * d1, "readout_o": 2 * F * d1,
        "hash_q_chain": proj, "hash_k_chain": proj,
        "seg_sum_qd_t": 2 * F * d1,
        "dpsi_q": 2 * F * d1 + proj, "dpsi_k": 2 * F * d + proj,
        "readout_dv": 2 * F * d,
    }
    if dw:
        per_kernel["dq"] += proj
        per_kernel["dk"] += proj
    fwd_flops = 4 * d * L * P + 4 * F * d1
    bwd_flops = (4 * d * L * P + 2 * rehash + 4 * F * d1 + 4 * F * d
                 + (4 * d * L * P if dw else 0))
    if not w.backward:
        return fwd_flops, 4 * d * e + 4, per_kernel
    return fwd_flops + bwd_flops, 12 * d * e + 8, per_kernel


# The sources the fused 16-bit kernels (sum_kv ... dv) are built, launched and
# planned from; the other files of csrc/ hold other kernels (the fp32 path,
# d = 128 rows, hard hashing, the streaming state) that leave these unchanged.
FUSED_SOURCES = ("csrc/race_walk.h", "csrc/race_common.h", "csrc/race_fwd.h", "csrc/race_squash.h",
                 "csrc/race_host.h", "csrc/race_attn.hip", "csrc/race_inst_bf16_fwd.hip",
                 "csrc/race_inst_bf16_bwd.hip")


def kernel_sources_digest() -> str:
    """sha256 over the fused kernels' sources and the C header (each file's
    name, then its bytes, sorted by name)."""
    import hashlib
    files = [os.path.join(HERE, "sketch_attention_soft_amd", f) for f in FUSED_SOURCES]
    files.append(os.path.join(HERE, "include", "race_attn.h"))
    h = hashlib.sha256()
    for f in sorted(files, key=os.path.basename):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str) -> dict:
    """HBM bytes per launch from the committed counter summary of this workload,
    or {} when it is missing or was taken on other kernel sources."""
    path = os.path.join(HERE, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return {}
    out, digest = {}, None
    with open(path) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) >= 3 and parts[0] == "traffic":
                out[parts[1]] = float(parts[2])
            elif len(parts) == 2 and parts[0] == "source_sha256":
                digest = parts[1]
    return out if digest == kernel_sources_digest() else {}


def graph_latency_us(step, outs, steps: int, torch):
    """Microseconds per replay of one step captured as a HIP graph (the
    library enqueues only kernels on the caller's stream: no allocation, copy
    or memset), and whether a replay writes the same bits as the eager step."""
    ref = tuple(t.clone() for t in outs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # settle allocations outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for t in outs:
        t.zero_()
    g.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(outs, ref))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return round(a.elapsed_time(b) / steps * 1e3, 2), same


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="causal_n4m_bf16")
    ap.add_argument("--cpu-tokens", type=int, default=524288,
                    help="tokens of the workload's first head timed on the oracle (0: skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters), then exit")
    ap.add_argument("--dw", action="store_true",
                    help="the backward also returns the projection gradient dW "
                         "(race_attn_backward_dw, learned hyperplanes)")
    ap.add_argument("--hard", action="store_true",
                    help="time the hard-hash forward (race_attn_forward_hard) on the workload")
    ap.add_argument("--generality", action="store_true",
                    help="time fwd+bwd of the 4M-token head with fp16 rows, d = 32, P = 2 and a "
                         "right-padded batch beside the bf16 d = 64 P = 4 step")
    ap.add_argument("--stream", action="store_true",
                    help="time the streaming state entry points instead (decode of one token "
                         "per head over 64 heads, bulk state_add of the 4M-token head)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "path is a design note, not part of this library", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}), flush=True)
        return 0

    from sketch_attention_soft_amd import binding
    from sketch_attention_soft_amd import inputs as I

    if args.stream:
        return stream_bench(args, binding, I, np, torch)
    if args.generality:
        return generality_bench(args, binding, I, np, torch)
    if args.hard:
        return hard_bench(args, binding, I, np, torch)

    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.time()
    x = I.workload_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def put(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = put(x["q"]), put(x["k"]), put(x["v"])
    do = put(x["do"]) if w.backward else None
    W = torch.from_numpy(x["W"]).to(dev)
    del x
    print(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    B, H, N, d = q.shape
    o = torch.empty_like(q)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    grads = tuple(torch.empty_like(q) for _ in range(3)) if w.backward else None
    wsf = torch.empty(binding.workspace_bytes(B, H, N, d, w.L, w.P, w.causal, w.chunk, tdt, False),
                      dtype=torch.uint8, device=dev)
    wsb = (torch.empty(binding.workspace_bytes(B, H, N, d, w.L, w.P, w.causal, w.chunk, tdt,
                                               2 if args.dw else 1),
                       dtype=torch.uint8, device=dev) if w.backward else None)
    # the forward's key state, kept for the backward (as autograd would)
    saved = binding.new_saved(q, W, w.causal, w.chunk) if w.backward else None

    def step(trf=None, trb=None):
        binding.forward(q, k, v, W, w.tau, w.causal, w.chunk, workspace=wsf, out=(o, den),
                        trace=trf, saved=saved)
        if w.backward:
            binding.backward(q, k, v, W, o, den, do, w.tau, w.causal, w.chunk, workspace=wsb,
                             out=grads, trace=trb, saved=saved, dw=args.dw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    traces = [(binding.Trace(), binding.Trace() if w.backward else None) for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # a latency-bound step (a short forward) is timed without the per-kernel
    # events, which would add their own gaps between its few short kernels;
    # the events are then taken over a second loop of the same steps
    latency_bound = not w.backward and w.tokens <= 4096
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        if latency_bound:
            step()
        else:
            step(*traces[i])
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    graph_us = None
    if latency_bound:
        for i in range(args.steps):
            step(*traces[i])
        torch.cuda.synchronize()
        graph_us = graph_latency_us(step, (o, den), args.steps, torch)
    tokens = w.tokens
    value = tokens / (ms * 1e-3)
    print(f"[bench] {ms:.3f} ms/step", file=sys.stderr, flush=True)

    # per-kernel averages over the timed steps
    kern: dict[str, float] = {}
    for tf, tb in traces:
        for tr in (tf, tb):
            if tr is None:
                continue
            for name, t in tr.results():
                kern[name] = kern.get(name, 0.0) + t / args.steps
    flops_tok, bytes_tok, per_kernel = algorithmic_per_token(w, args.dw)
    dom = max(kern, key=kern.get)
    dom_ms = kern[dom]
    peak = PEAK_TFLOPS[w.dtype]
    achieved = per_kernel.get(dom, 0) * tokens / (dom_ms * 1e-3) / 1e12
    t_mfma = flops_tok * tokens / (peak * 1e12) * 1e3
    t_hbm = bytes_tok * tokens / (PEAK_HBM_GBS * 1e9) * 1e3
    # the counters were taken on the plain backward
    traffic = None if args.dw else measured_traffic(w.name).get(dom)
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 5),
                "traffic": round(traffic) if traffic is not None else None, "kernel": dom,
                "kernel_ms": round(dom_ms, 4)}

    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        n_cpu = min(args.cpu_tokens, w.N)
        xs = I.workload_inputs(w, n_rows=n_cpu)
        hq, hk, hv = (I.to_f64(xs[n], w.dtype)[:1, :1] for n in ("q", "k", "v"))
        cores = oracle.threads()
        tc = time.time()
        if w.backward:
            hg = I.to_f64(xs["do"], w.dtype)[:1, :1]
            oracle.forward_backward(hq, hk, hv, hg, xs["W"], w.tau, w.causal)
        else:
            oracle.forward(hq, hk, hv, xs["W"], w.tau, w.causal)
        dt = time.time() - tc
        cpu = {"value": round(n_cpu / dt, 1), "unit": "tokens/s", "cores": cores,
               "kind": "oracle",
               "sample": f"first {n_cpu} tokens of head 0 of {w.name}, "
                         f"{'fwd+bwd' if w.backward else 'fwd'} in fp64 ({dt:.1f} s)"}

    line = {
        "metric": metric_name(w), "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "latency_us": round(ms * 1e3, 2),
        **({"latency_us_hip_graph": graph_us[0], "hip_graph_matches_eager": graph_us[1]}
           if graph_us else {}),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Philox N(0,1); Q, K rows L2-normalised)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "L": w.L,
                   "P": w.P, "tau": w.tau, "causal": w.causal,
                   "passes": ("fwd+bwd+dW" if args.dw else "fwd+bwd") if w.backward else "fwd",
                   "chunk": w.chunk},
        "roofline": roofline,
        "step_roofline": {"t_mfma_ms": round(t_mfma, 4), "t_hbm_ms": round(t_hbm, 4),
                          "frac": round(max(t_mfma, t_hbm) / ms, 5)},
        "kernels_ms": {k2: round(v2, 4) for k2, v2 in kern.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def generality_bench(args, binding, I, np, torch) -> int:
    """One JSON line: the fwd+bwd step (saved state, as the main bench times
    it) of causal_n4m_bf16's shape in the variants the library supports
    beyond it -- fp16 rows, head dimension 32 and 128, P = 2, 5 and 6
    hyperplanes per table, and a right-padded batch of four sequences of 4M, 3M, 2M and 1M tokens
    padded to 4M (tokens/s counts real tokens only; the binding's padded_chunk
    segments) -- beside the bf16 d = 64
    P = 4 step itself, in one process.  Inputs are drawn on the device (torch
    N(0, 1), Q and K rows normalised): these are timing runs, parity is
    tested elsewhere.  Each variant reports its algorithmic flops and bytes
    against the MFMA and HBM peaks (step_frac = max(t_mfma, t_hbm) / t)."""
    import dataclasses
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    base = I.WORKLOADS["causal_n4m_bf16"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(4243)
    variants = [("bf16_d64_P4", torch.bfloat16, 64, 4, None),
                ("f16_d64_P4", torch.float16, 64, 4, None),
                ("bf16_d32_P4", torch.bfloat16, 32, 4, None),
                ("bf16_d64_P2", torch.bfloat16, 64, 2, None),
                ("bf16_d64_P5", torch.bfloat16, 64, 5, None),
                ("bf16_d64_P6", torch.bfloat16, 64, 6, None),
                ("bf16_d128_P4", torch.bfloat16, 128, 4, None),
                ("bf16_padded_4x4M", torch.bfloat16, 64, 4, (4 << 20, 3 << 20, 2 << 20, 1 << 20))]
    out = {}
    for name, tdt, d, P, lens in variants:
        B = len(lens) if lens else 1
        N, L = base.N, base.L

        def rows(normalise):
            x = torch.randn((B, 1, N, d), generator=gen, device=dev, dtype=torch.float32)
            if normalise:
                x = x / x.norm(dim=-1, keepdim=True)
            return x.to(tdt)

        q, k, v, do = rows(True), rows(True), rows(False), rows(False)
        W = torch.randn((L, P, d), generator=gen, device=dev, dtype=torch.float32)
        tokens = sum(lens) if lens else N
        o = torch.zeros_like(q)
        den = torch.zeros((B, 1, N), dtype=torch.float32, device=dev)
        grads = tuple(torch.zeros_like(q) for _ in range(3))
        ch = binding.padded_chunk(B, 1, N) if lens else 0
        wsf = torch.empty(binding.workspace_bytes(B, 1, N, d, L, P, True, ch, tdt, False),
                          dtype=torch.uint8, device=dev)
        wsb = torch.empty(binding.workspace_bytes(B, 1, N, d, L, P, True, ch, tdt, True),
                          dtype=torch.uint8, device=dev)
        if lens:
            sl = torch.tensor(lens, dtype=torch.int32, device=dev)

            def step():
                binding.forward_padded(q, k, v, W, sl, base.tau, True, ch, workspace=wsf,
                                       out=(o, den))
                binding.backward_padded(q, k, v, W, o, den, do, sl, base.tau, True, ch,
                                        workspace=wsb, out=grads)
        else:
            saved = binding.new_saved(q, W, True, 0)

            def step():
                binding.forward(q, k, v, W, base.tau, True, 0, workspace=wsf, out=(o, den),
                                saved=saved)
                binding.backward(q, k, v, W, o, den, do, base.tau, True, 0, workspace=wsb,
                                 out=grads, saved=saved)

        for _ in range(args.warmup):
            step()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        wv = dataclasses.replace(base, d=d, P=P, dtype="bf16")
        flops_tok, bytes_tok, _ = algorithmic_per_token(wv)
        t_mfma = flops_tok * tokens / (PEAK_TFLOPS["bf16"] * 1e12) * 1e3
        t_hbm = bytes_tok * tokens / (PEAK_HBM_GBS * 1e9) * 1e3
        out[name] = {"ms_per_step": round(ms, 4), "tokens": tokens,
                     "tokens_per_s": round(tokens / (ms * 1e-3), 1),
                     "flops_per_token": flops_tok, "bytes_per_token": bytes_tok,
                     "step_frac": round(max(t_mfma, t_hbm) / ms, 5)}
        print(f"[bench] {name}: {ms:.3f} ms/step", file=sys.stderr, flush=True)
        del q, k, v, do, o, den, grads, wsf, wsb
        torch.cuda.empty_cache()
    ref = out["bf16_d64_P4"]["tokens_per_s"]
    for r in out.values():
        r["vs_bf16_d64_P4"] = round(r["tokens_per_s"] / ref, 4)
    line = {
        "metric": "RACE attn fwd+bwd tokens/s, library variants at the 4M-token causal shape",
        "value": out["bf16_d64_P4"]["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": out["bf16_d64_P4"]["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (torch N(0,1) on the device; Q, K rows L2-normalised)",
        "config": {"workload": "causal_n4m_variants", "N": base.N, "L": base.L, "tau": base.tau,
                   "causal": True, "passes": "fwd+bwd"},
        "variants": out,
    }
    print(json.dumps(line), flush=True)
    return 0


def hard_bench(args, binding, I, np, torch) -> int:
    """One JSON line for the hard-hash forward on the workload (forward only:
    the hash has no gradient).  Its algorithmic bytes are one read of Q, K, V
    and one write of O and den (4 d e + 4 per token); on 16-bit rows with
    L <= 32 it runs on integer bucket ids (hash ids of Q and K, count and
    value sums per segment, scans, the walk), so it is reported against HBM,
    with the projections' matrix-core rate beside it."""
    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    x = I.workload_inputs(w, with_grad=False)

    def put(a):
        if w.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    q, k, v = put(x["q"]), put(x["k"]), put(x["v"])
    W = torch.from_numpy(x["W"]).to(dev)
    del x
    B, H, N, d = q.shape
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    o = torch.empty_like(q)
    den = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(binding.workspace_bytes(B, H, N, d, w.L, w.P, w.causal, w.chunk, tdt, 4),
                     dtype=torch.uint8, device=dev)

    def step():
        binding.forward_hard(q, k, v, W, w.causal, w.chunk, workspace=ws, out=(o, den))

    for _ in range(args.warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    e = 2 if w.dtype == "bf16" else 4
    bytes_tok = 4 * d * e + 4
    # the projections u = W x of the query and the key rows; the rest of the
    # hard path is integer counting and value gathers
    fwd_flops_tok = 2 * 2 * d * w.L * w.P
    gbs = bytes_tok * w.tokens / (ms * 1e-3) / 1e9
    tfl = fwd_flops_tok * w.tokens / (ms * 1e-3) / 1e12
    line = {
        "metric": "RACE hard-hash attention forward tokens/s (true bucket counts)",
        "value": round(w.tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Philox N(0,1); Q, K rows L2-normalised)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "L": w.L,
                   "P": w.P, "causal": w.causal, "passes": "fwd (hard hash)", "chunk": w.chunk},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": None,
                     "kernel": "whole forward (ids of Q and K, sums, scans, walk)",
                     "bytes_per_token": bytes_tok},
        "mfma": {"achieved": round(tfl, 3), "peak": PEAK_TFLOPS["bf16" if w.dtype == "bf16" else "f32"],
                 "unit": "TFLOP/s", "flops_per_token": fwd_flops_tok},
    }
    print(json.dumps(line), flush=True)
    return 0


def stream_bench(args, binding, I, np, torch) -> int:
    """One JSON line for the streaming state API (race_attn_decode,
    race_attn_state_add).  Decode: 4 x 16 heads, one token each per call, the
    state of a 2048-token prefix; bound by reading and writing the fp32 state
    (F x 65 floats per head), so its roofline is HBM bytes per call / time.
    Bulk add: the 4,194,304-token head of causal_n4m_bf16; fp32 vector
    arithmetic, 2 F (d + 1) + 2 d L P flops per token (update and
    projection), against the fp32 vector peak."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    L, P, d, tau = 32, 4, 64, 1.0
    F = L << P

    def put(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def timed(fn, iters, warm):
        for _ in range(warm):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    # decode: 64 heads, one token per head per call
    B, H, N0 = 4, 16, 2048
    x = I.make_inputs(B, H, N0 + 1, d, L, P, "bf16", 4242, with_grad=False)
    q, k, v = (put(x[n]) for n in ("q", "k", "v"))
    W = torch.from_numpy(x["W"]).to(dev)
    st = binding.new_state(B, H, d, L, P, dev)
    binding.state_add(st, k[:, :, :N0].contiguous(), v[:, :, :N0].contiguous(), W, tau)
    q1, k1, v1 = (t[:, :, N0:].contiguous() for t in (q, k, v))
    o1 = torch.empty_like(q1)
    den1 = torch.empty((B, H, 1), dtype=torch.float32, device=dev)
    ms_dec = timed(lambda: binding.decode(st, q1, k1, v1, W, tau, out=(o1, den1)),
                   max(args.steps, 10) * 10, args.warmup + 5)
    bytes_dec = 2 * B * H * F * (d + 1) * 4 + 4 * B * H * d * 2 + B * H * 4
    gbs = bytes_dec / (ms_dec * 1e-3) / 1e9

    # bulk add of the headline head
    w = I.WORKLOADS["causal_n4m_bf16"]
    xa = I.workload_inputs(w, with_grad=False)
    ka, va = put(xa["k"]), put(xa["v"])
    Wa = torch.from_numpy(xa["W"]).to(dev)
    del xa
    sa = binding.new_state(1, 1, d, L, P, dev)
    ws = torch.empty(binding.state_add_workspace_bytes(1, 1, w.N, d, L, P), dtype=torch.uint8,
                     device=dev)
    ms_add = timed(lambda: binding.state_add(sa, ka, va, Wa, tau, workspace=ws), max(args.steps, 3),
                   1)
    flops_tok = 2 * F * (d + 1) + 2 * d * L * P
    tflops = flops_tok * w.N / (ms_add * 1e-3) / 1e12
    # the same add through the fused segment sum (bf16 operands, fp32 sums)
    wsf = torch.empty(binding.workspace_bytes(1, 1, w.N, d, L, P, True, 0, torch.bfloat16, 3),
                      dtype=torch.uint8, device=dev)
    ms_fast = timed(lambda: binding.state_add(sa, ka, va, Wa, tau, workspace=wsf, fast=True),
                    max(args.steps, 3), 1)
    tf_fast = flops_tok * w.N / (ms_fast * 1e-3) / 1e12

    line = {
        "metric": "RACE streaming decode tokens/s (64 heads x 1 token, L=32, d=64, bf16 rows, "
                  "fp32 state); % of HBM roofline",
        "value": round(B * H / (ms_dec * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": max(args.steps, 10) * 10, "warmup": args.warmup + 5,
        "ms_per_step": round(ms_dec, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded Philox N(0,1); Q, K rows L2-normalised)",
        "config": {"workload": "decode_64h_1tok_L32", "B": B, "H": H, "prefix": N0, "L": L,
                   "P": P, "d": d, "tau": tau},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": None,
                     "kernel": "stream_kernel (decode)", "bytes_per_call": bytes_dec},
        "state_add": {"workload": w.name, "tokens": w.N, "ms": round(ms_add, 4),
                      "tokens_per_s": round(w.N / (ms_add * 1e-3), 1),
                      "roofline": {"bound": "alu", "achieved": round(tflops, 3),
                                   "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                                   "frac": round(tflops / PEAK_TFLOPS["f32"], 5),
                                   "flops_per_token": flops_tok}},
        "state_add_fast": {"workload": w.name, "tokens": w.N, "ms": round(ms_fast, 4),
                           "tokens_per_s": round(w.N / (ms_fast * 1e-3), 1),
                           "roofline": {"bound": "mfma", "achieved": round(tf_fast, 3),
                                        "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s",
                                        "frac": round(tf_fast / PEAK_TFLOPS["bf16"], 5),
                                        "flops_per_token": flops_tok}},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
