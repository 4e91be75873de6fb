#!/usr/bin/env python3
"""Benchmark: zero-start tail replay on one MI355X.

Workload (the 5% tail-replay case): 16 requests x 32 heads, d_k = d_v = 128,
bf16 q/k/v/alpha/beta, float32 state, matched prefix m = 32768, so each request
replays k = ceil(0.05 m) = 1639 positions from the zero state, writing the
per-token outputs o_t and the final state.  One step = one gdn_tail_replay call
over the whole batch (all heads of one layer); inputs are resident in HBM
before timing starts.

Reported: replayed tokens/s per layer (all heads), the roofline fraction of
the dominant kernel (algorithmic bytes or flops per launch / its measured
duration), and the fp64 CPU oracle timed on a bounded sample of the same
workload on the host cores.  Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector, published
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix, published


def measured_traffic(kernel_src: str, profile: str):
    """HBM bytes per launch from the committed counter summary (rocprofv3
    FETCH_SIZE and WRITE_SIZE runs of this same command, scaled by a copy of
    known size), with a label naming that source; (None, reason) when the
    kernel source changed since the counters were taken."""
    import hashlib
    try:
        txt = open(profile).read()
        sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None, "no counter summary"
    vals = dict(l.split(":", 1) for l in txt.splitlines() if l.startswith(("traffic_bytes_per_launch:",
                                                                            "kernel_source_sha256_prefix:")))
    rel = os.path.relpath(profile, ROOT)
    if vals.get("kernel_source_sha256_prefix", "").strip() != sha:
        return None, f"{rel} was taken on another kernel source (sha256 prefix differs from {sha})"
    return int(vals["traffic_bytes_per_launch"]), (f"{rel}: rocprofv3 FETCH_SIZE / WRITE_SIZE of this command, "
                                                   f"committed for kernel source sha256 prefix {sha}; "
                                                   "not measured in this run")


def host_cpu():
    """Logical CPUs of the host, those this process may use, and the CPU model."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"nproc": usable, "logical_cpus": os.cpu_count(), "model": model}


def algorithmic_bytes(token_heads: int, pairs: int, dk: int, dv: int, elem: int,
                      with_o: bool = True) -> int:
    """Bytes a replay must move: q, k, v, alpha, beta in; o out; final state out."""
    per_tok = elem * (2 * dk + dv) + 2 * elem + (elem * dv if with_o else 0)
    return token_heads * per_tok + pairs * dv * dk * 4


def algorithmic_flops(token_heads: int, dk: int, dv: int) -> int:
    """S k (2 d_k d_v), rank-1 update (3 d_k d_v: scale, multiply-add), S q (2 d_k d_v)."""
    return token_heads * 7 * dk * dv


def cpu_baseline(w, spans, budget_s: float = 15.0):
    """Time the fp64 C oracle, as written, on a bounded sample of (request, head) pairs."""
    import numpy as np
    import torch
    import oracle
    if not oracle.c_oracle_available():
        from oracle.build import build_c_oracle
        build_c_oracle()
    threads = oracle.c_oracle_threads()
    H = w.H
    allp = [(b, h) for b in range(w.B) for h in range(w.H)]

    def run(pairs):
        S0s, qs, ks, vs, al, bt = [], [], [], [], [], []
        for (b, h) in pairs:
            p0, n = spans[b]
            r0 = w.tok_offset[b] + (p0 - w.first_pos[b])
            sl = slice(r0, r0 + n)
            f = lambda t: t[sl, h].to(torch.float64).cpu().numpy()
            S0s.append(np.zeros((w.dv, w.dk)))
            qs.append(f(w.q)); ks.append(f(w.k)); vs.append(f(w.v))
            al.append(f(w.alpha)); bt.append(f(w.beta))
        t0 = time.perf_counter()
        oracle.scan_rank1_c_batch(S0s, qs, ks, vs, al, bt, normalize_k=True, normalize_q=True)
        return time.perf_counter() - t0, sum(spans[b][1] for (b, _) in pairs)

    # calibrate on one pair per thread, then size the sample to ~budget_s of wall time
    n0 = min(len(allp), max(1, threads))
    dt, toks = run(allp[:n0])
    per_pair = dt / n0 * threads  # CPU-seconds per pair
    n = int(min(len(allp), max(n0, budget_s * threads / max(per_pair, 1e-9))))
    n = max(threads, (n // threads) * threads) if n >= threads else n
    n = min(n, len(allp))
    dt, toks = run(allp[:n])
    rate = toks / H / dt  # token-heads / H = tokens with all heads
    cpu = host_cpu()
    return {"value": rate, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "nproc": cpu["nproc"], "logical_cpus": cpu["logical_cpus"], "cpu_model": cpu["model"],
            "sample": f"{n} of {len(allp)} (request, head) pairs, {spans[0][1]} tokens each, "
                      f"fp64 C rank-1 oracle with OpenMP; {dt:.1f} s wall"}


def planner_bench(gdn):
    """Host planner: wall time of the O(N M) placement and the expected
    recomputation it reaches against the balanced placement and no checkpoint."""
    import numpy as np

    def dists(N):
        x = np.arange(N + 1) / N
        u = np.r_[0.0, np.full(N, 1.0 / N)]
        bimodal = np.exp(-((x - 0.35) / 0.04) ** 2) + np.exp(-((x - 0.75) / 0.08) ** 2) + 0.02
        bimodal[0] = 0.05
        head = 0.9995 ** np.arange(N + 1)
        return {"uniform": u, "bimodal": bimodal / bimodal.sum(), "geometric": head / head.sum()}

    for N, M in [(8192, 8), (32768, 16), (65536, 16), (262144, 64)]:
        for name, p in dists(N).items():
            reps = 3
            t0 = time.perf_counter()
            for _ in range(reps):
                pos, cost = gdn.plan_checkpoints(p, M)
            ms = (time.perf_counter() - t0) / reps * 1e3
            bal = gdn.expected_recompute(p, gdn.balanced_checkpoints(N, M))
            none = gdn.expected_recompute(p, [])
            print(json.dumps({"metric": "checkpoint placement (host planner)", "distribution": name,
                              "N": N, "M": M, "ms": round(ms, 3), "ns_per_NM": round(ms * 1e6 / (N * M), 3),
                              "expected_recompute": {"planned": cost, "balanced": bal, "none": none},
                              "planned_vs_balanced": cost / bal if bal > 0 else None}), flush=True)


def overlap_bench(torch, gdn, w, dev):
    """Replay of the 5% tail workload while a pinned host buffer standing in for
    the attention layers' KV cache is copied to the device on another stream:
    medians of T_KV, T_replay, the serial sum and the overlapped call, against
    the latency model max(T_KV, T_replay) of the Tail-Replay page (§2.5)."""
    import numpy as np
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = torch.empty_like(w.v)
    cs = torch.cuda.Stream(device=dev)
    ev = torch.cuda.Event()
    cur = torch.cuda.current_stream(dev)

    def replay():
        gdn.tail_replay(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.m, w.r_num, w.r_den,
                        first_pos=w.first_pos, flags=w.flags, state_out=st, o=o)

    def timed(fn, reps=11):
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(cur)
            fn()
            b.record(cur)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))

    for _ in range(200):
        replay()
    torch.cuda.synchronize()
    t_rep = timed(replay)
    for mib in (4, 16, 64, 256):
        n = mib << 20
        src = torch.empty(n, dtype=torch.uint8).pin_memory()
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        t_kv = timed(lambda: dst.copy_(src, non_blocking=True))
        t_ser = timed(lambda: (dst.copy_(src, non_blocking=True), replay()))
        t_ov = timed(lambda: gdn.tail_replay_with_h2d(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.m,
                                                      w.r_num, w.r_den, src, dst, cs, ev,
                                                      first_pos=w.first_pos, flags=w.flags,
                                                      state_out=st, o=o))
        print(json.dumps({"metric": "tail replay overlapped with KV transfer", "kv_mib": mib,
                          "h2d_GBps": n / (t_kv * 1e-3) / 1e9, "T_KV_ms": t_kv, "T_replay_ms": t_rep,
                          "T_serial_ms": t_ser, "T_overlap_ms": t_ov,
                          "model_max_ms": max(t_kv, t_rep), "overlap_vs_model": t_ov / max(t_kv, t_rep),
                          "saved_vs_serial_ms": t_ser - t_ov}), flush=True)
        del src, dst


def prefill_bench(torch, gdn, w, dev, args):
    """Prefill with emission, one pass against the sequence-split path: HIP-event
    time per call (after warm-up), tokens/s and the fraction of the HBM peak."""
    M = len(w.ckpt_pos[0])
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    ck = torch.empty(w.B, M, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = torch.empty_like(w.v)
    ws = torch.empty(gdn.prefill_split_workspace_bytes(w.B, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    tokens = sum(w.n_tokens)
    nbytes = algorithmic_bytes(tokens * w.H, w.B * w.H, w.dk, w.dv, 2) + w.B * M * w.H * w.dv * w.dk * 4
    paths = {
        "one_pass": lambda: gdn.prefill_emit_checkpoints(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                                                         flags=w.flags, ckpt_states=ck, state_out=st, o=o),
        "split3": lambda: gdn.prefill_emit_checkpoints_split(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset,
                                                             w.ckpt_pos, flags=w.flags, ckpt_states=ck,
                                                             state_out=st, o=o, workspace=ws),
    }
    stream = torch.cuda.current_stream(dev)
    for name, fn in paths.items():
        for _ in range(max(args.warmup, 2)):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(3, min(args.steps, 10))
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        print(json.dumps({"metric": "prefill with checkpoint emission", "path": name, "ms": ms,
                          "tokens_per_s": tokens / (ms * 1e-3), "algorithmic_bytes": nbytes,
                          "hbm_frac": nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9),
                          "config": {"requests": w.B, "heads": w.H, "N": w.n_tokens[0], "checkpoints": M,
                                     "d": w.dk, "inputs": "bf16"}}), flush=True)


def workloads_bench(torch, gdn, W, dev, args):
    """Every headline workload at full size through the library, timed with HIP
    events on the launch stream (median of 5 timed batches after warm-up)."""
    import numpy as np
    stream = torch.cuda.current_stream(dev)

    def timed(fn, reps=10):
        # warm-up for a fixed wall time, until the GPU clocks have settled
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < max(args.device_warmup_s, 0.3):
            fn()
            torch.cuda.synchronize()
        out = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) / reps)
        return float(np.median(out))

    def line(name, ms, tokens, nbytes, extra=None):
        d = {"metric": "workload time", "workload": name, "ms": ms, "replayed_tokens": tokens,
             "tokens_per_s": tokens / (ms * 1e-3), "algorithmic_bytes": nbytes,
             "hbm_frac": nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9)}
        d.update(extra or {})
        print(json.dumps(d), flush=True)

    # resume: 8 x 16 pairs, prefix 8192, 8 balanced checkpoints, depths ~ U{1..N}
    w = W.named("resume_B8_H16_N8192", device=dev)
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = torch.empty_like(w.v)
    js = [0] * w.B
    spans = []
    for b in range(w.B):
        j = gdn.select_checkpoint(w.ckpt_pos[b], w.depth[b])
        c = 0 if j == 0 else w.ckpt_pos[b][j - 1]
        spans.append(w.depth[b] - c)
        js[b] = j
    toks = sum(spans)
    nb = algorithmic_bytes(toks * w.H, w.B * w.H, w.dk, w.dv, 2) + sum(1 for j in js if j > 0) * w.H * w.dv * w.dk * 4
    ms = timed(lambda: gdn.resume(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos, w.ckpt_states,
                                  w.depth, first_pos=w.first_pos, flags=w.flags, state_out=st, o=o))
    line(w.name, ms, toks, nb, {"mean_span": toks / w.B})
    # tail 5%
    w = W.named("tail5_B16_H32_m32768", device=dev)
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = torch.empty_like(w.v)
    ks = [gdn.tail_len(m, w.r_num, w.r_den) for m in w.m]
    ms = timed(lambda: gdn.tail_replay(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.m, w.r_num, w.r_den,
                                       first_pos=w.first_pos, flags=w.flags, state_out=st, o=o))
    line(w.name, ms, sum(ks), algorithmic_bytes(sum(ks) * w.H, w.B * w.H, w.dk, w.dv, 2))
    # grouped tail 10%, three layers: layer l+1 reads layer l's outputs as q = k = v
    w = W.named("tail10_grouped_B16_H32_m32768_L3", device=dev)
    ks = [gdn.tail_len(m, w.r_num, w.r_den) for m in w.m]
    alphas = [w.alpha] + list(w.layer_alpha)
    betas = [w.beta] + list(w.layer_beta)
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    outs = [torch.empty_like(w.v) for _ in range(3)]

    def group():
        q, k, v = w.q, w.k, w.v
        for layer in range(3):
            gdn.tail_replay(q, k, v, alphas[layer], betas[layer], w.tok_offset, w.m, w.r_num, w.r_den,
                            first_pos=w.first_pos, flags=w.flags, state_out=st, o=outs[layer])
            q = k = v = outs[layer]
    th = sum(ks) * w.H
    # layer 1 reads q, k, v; layers 2 and 3 read one tensor; each layer writes o and its states
    nb = (algorithmic_bytes(th, w.B * w.H, w.dk, w.dv, 2)
          + 2 * (th * (2 * w.dk + 2 * 2 + 2 * w.dv) + w.B * w.H * w.dv * w.dk * 4))
    ms = timed(group, reps=5)
    line(w.name, ms, sum(ks), nb, {"layers": 3, "tokens_are_per_layer": True, "path": "three calls"})
    # the same group in one call (one launch: each workgroup takes its pair through the layers)
    st3 = torch.empty(3, w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o3 = torch.empty((3,) + tuple(w.v.shape), dtype=w.v.dtype, device=dev)
    ms = timed(lambda: gdn.tail_replay_group(w.q, w.k, w.v, alphas, betas, w.tok_offset, w.m, w.r_num, w.r_den,
                                             first_pos=w.first_pos, flags=w.flags, state_out=st3, o=o3), reps=5)
    line(w.name, ms, sum(ks), nb, {"layers": 3, "tokens_are_per_layer": True, "path": "group call"})
    # prefill with emission, one pass and split
    w = W.named("prefill_emit_B4_H32_N65536", device=dev)
    M = len(w.ckpt_pos[0])
    st = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    ck = torch.empty(w.B, M, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = torch.empty_like(w.v)
    ws = torch.empty(gdn.prefill_split_workspace_bytes(w.B, w.H, w.dk, w.dv), dtype=torch.uint8, device=dev)
    toks = sum(w.n_tokens)
    nb = algorithmic_bytes(toks * w.H, w.B * w.H, w.dk, w.dv, 2) + w.B * M * w.H * w.dv * w.dk * 4
    ms = timed(lambda: gdn.prefill_emit_checkpoints(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.ckpt_pos,
                                                    flags=w.flags, ckpt_states=ck, state_out=st, o=o), reps=3)
    line(w.name, ms, toks, nb, {"path": "one pass"})
    ms = timed(lambda: gdn.prefill_emit_checkpoints_split(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset,
                                                          w.ckpt_pos, flags=w.flags, ckpt_states=ck, state_out=st,
                                                          o=o, workspace=ws), reps=3)
    line(w.name, ms, toks, nb, {"path": "three segments"})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--kernel", choices=["auto", "recurrent", "chunked"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-output", action="store_true", help="skip o (state only)")
    ap.add_argument("--device-warmup-s", type=float, default=0.3,
                    help="untimed repetitions of the step before the warm-up steps, until the "
                         "GPU clocks have settled (seconds of wall time)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the replay, time a plain device copy of this many MiB "
                         "(calibrates the FETCH_SIZE / WRITE_SIZE counters against known bytes)")
    ap.add_argument("--planner", action="store_true",
                    help="instead of the replay, time the host checkpoint-placement planner and "
                         "print one JSON line per (distribution, N, M)")
    ap.add_argument("--overlap", action="store_true",
                    help="instead of the headline line, time the tail replay overlapped with a "
                         "host-to-device KV transfer on a second stream, one JSON line per KV size")
    ap.add_argument("--prefill", action="store_true",
                    help="instead of the headline line, time the prefill with emission (4 x 32 and "
                         "1 x 32 pairs, N = 65536, 16 checkpoints) in one pass and split in three segments")
    ap.add_argument("--workloads", action="store_true",
                    help="instead of the headline line, print one line per headline workload (resume, "
                         "tail 5%%, grouped tail 10%% over three layers, prefill with emission): "
                         "HIP-event time per call, algorithmic bytes and the fraction of the HBM peak")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the replay shards over (request, head) pairs "
              "with no exchange, so a multi-GPU figure is not part of this benchmark.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_scan_amd as gdn
    import workloads as W

    gdn.load()
    if args.planner:
        planner_bench(gdn)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe_mib:
        copy_probe(torch, dev, args)
        return
    if args.workloads:
        workloads_bench(torch, gdn, W, dev, args)
        return
    if args.prefill:
        prefill_bench(torch, gdn, W.named("prefill_emit_B4_H32_N65536", device=dev), dev, args)
        # one request (32 pairs): the split's three segments have the idle CUs to run on
        prefill_bench(torch, gdn, W.prefill(device=dev, B=1, name="prefill_emit_B1_H32_N65536"), dev, args)
        return
    w = W.named("tail5_B16_H32_m32768", device=dev)
    if args.overlap:
        overlap_bench(torch, gdn, w, dev)
        return
    flags = w.flags | {"auto": 0, "recurrent": gdn.KERNEL_RECURRENT,
                       "chunked": gdn.KERNEL_CHUNKED}[args.kernel]
    ks = [gdn.tail_len(m, w.r_num, w.r_den) for m in w.m]
    spans = [(m - k + 1, k) for m, k in zip(w.m, ks)]
    tokens = sum(ks)
    token_heads = tokens * w.H
    pairs = w.B * w.H
    state = torch.empty(w.B, w.H, w.dv, w.dk, dtype=torch.float32, device=dev)
    o = None if args.no_output else torch.empty_like(w.v)

    def step():
        gdn.tail_replay(w.q, w.k, w.v, w.alpha, w.beta, w.tok_offset, w.m, w.r_num, w.r_den,
                        first_pos=w.first_pos, flags=flags, state_out=state, o=o,
                        want_o=o is not None)

    # Device warm-up (untimed): the first ~100 launches run while the GPU clocks
    # ramp up; repeat the step for a fixed wall-clock interval so that the timed
    # region measures the steady state, then the W warm-up steps proper.
    t_dev0 = time.perf_counter()
    n_dev = 0
    while time.perf_counter() - t_dev0 < args.device_warmup_s:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n_dev += 20
    device_warmup_s = time.perf_counter() - t_dev0
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    region0.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    ms_region = region0.elapsed_time(region1)
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = ms_region / args.steps
    kern_ms = sum(per_launch_ms) / len(per_launch_ms)

    elem = 2 if w.dtype == "bf16" else 4
    nbytes = algorithmic_bytes(token_heads, pairs, w.dk, w.dv, elem, with_o=o is not None)
    nflops = algorithmic_flops(token_heads, w.dk, w.dv)
    chunked = gdn.kernel_for(w.B, w.H, w.dk, w.dv, w.torch_dtype, flags) == "chunked"
    if chunked:
        roof = {"bound": "hbm", "achieved": nbytes / (kern_ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "alu", "achieved": nflops / (kern_ms * 1e-3) / 1e12,
                "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if chunked and o is not None:
        roof["traffic"], roof["traffic_source"] = measured_traffic(
            os.path.join(ROOT, "gated_delta_rule_scan_amd", "csrc", "gdn_chunked.hip"),
            os.path.join(ROOT, "profiles", "chunked_kernel_tail5pct_traffic.md"))
    else:
        roof["traffic"], roof["traffic_source"] = None, "no counter summary for this kernel configuration"
    roof["algorithmic_bytes_per_launch"] = nbytes
    roof["algorithmic_flops_per_launch"] = nflops
    roof["kernel_ms"] = kern_ms
    roof["hbm_frac"] = nbytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS

    out = {
        "metric": "replayed tokens/s per layer (all heads)",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if chunked else "f32",
        "data": "synthetic",
        "config": {"workload": "tail_replay_5pct", "requests": w.B, "heads": w.H, "d_k": w.dk,
                   "d_v": w.dv, "matched_prefix": w.m[0], "replay_ratio": "5/100",
                   "replay_tokens": ks[0], "inputs": w.dtype, "state": "f32",
                   "outputs": o is not None, "kernel": "chunked" if chunked else "recurrent"},
        "roofline": roof,
        "wall_s_timed_region": t_wall,
        "device_warmup": {"seconds": device_warmup_s, "steps": n_dev},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, spans)
    print(json.dumps(out), flush=True)


def copy_probe(torch, dev, args):
    """A plain copy of known size: one read and one write of n bytes per launch."""
    n = args.copy_probe_mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "ms": ms,
                      "GB/s_read+write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


if __name__ == "__main__":
    main()
