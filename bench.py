#!/usr/bin/env python3
"""Benchmark of one device's share of a blockwise ring-attention forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A bench "step" is one whole ring_attn_forward: every ring step of the
device's share (the causal-tiled step kernels, each also receiving the next
K/V block into the free slot, unless --receive memcpy) and the fused
finalize, over seeded synthetic Q/K/V already resident in HBM. Prints ONE
JSON line.

value     effective causal attention TFLOP/s of the whole forward:
          sum over steps of 4 * head_dim * heads_q * batch * (visible pairs),
          divided by the forward's wall time (HIP events around K forwards).
roofline  for the dominant kernel (the bf16 step kernel): the same algorithmic
          FLOPs per launch divided by its average launch duration, measured
          with HIP events recorded around every step launch inside the timed
          forwards, against the MI355X dense bf16 MFMA peak.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3         # MI355X fp32 vector
REALTIME_GHZ = 0.1              # s_memrealtime counts a constant 100 MHz reference clock
SMALL_SHARE_PAIRS = 1 << 27     # rows x heads x keys up to which the oracle times the whole share
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E
DEFAULT_WORKLOAD = "zigzag128k_8dev_gqa"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def effective_flops(wl, pairs):
    return [4.0 * wl.head_dim * wl.heads_q * wl.batch * p for p in pairs]


def host_info():
    """The host CPU the oracle runs on: model name, logical CPUs and the BLAS
    thread count its matrix products use."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas_threads": blas}


def cpu_baseline(wl, rank, share_flops, budget_s=12.0):
    """Time the float64 CPU oracle on a bounded sample of the same share, and
    extrapolate its rate to the whole share (labelled as extrapolated)."""
    import oracle
    import ring_inputs
    positions = oracle.device_positions(wl.partition, wl.world, rank, wl.local_len)
    G = wl.heads_q // wl.heads_kv
    kh = ring_inputs.head(wl, "k", 0, 0)
    vh = ring_inputs.head(wl, "v", 0, 0)
    k_pos = np.arange(wl.total_len)
    rng = np.random.default_rng(0)
    n_rows = 8
    spent = 0.0
    flops = 0.0
    rows_done = 0
    heads_done = 0
    while spent < budget_s and n_rows <= wl.local_len:
        rows = np.sort(rng.choice(wl.local_len, size=n_rows, replace=False))
        pos = positions[rows]
        qs = [ring_inputs.rows(wl, "q", 0, h, pos) for h in range(G)]
        t0 = time.perf_counter()
        for q in qs:
            oracle.attention_rows(q, pos, kh, vh, k_pos, wl.causal)
        dt = time.perf_counter() - t0
        spent += dt
        vis = oracle.visible_pair_count(pos, k_pos, wl.causal)
        flops += 4.0 * wl.head_dim * vis * G
        rows_done += n_rows
        heads_done = G
        n_rows *= 2
    host = host_info()
    rate = flops / spent
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": int(host["blas_threads"] or os.cpu_count() or 1),
        "kind": "oracle",
        "sample": f"{rows_done} query rows of device {rank} x {heads_done} query heads (one KV group), "
                  f"float64 full softmax over all {wl.total_len} global keys, {spent:.1f} s of CPU time; "
                  f"effective FLOPs counted as for the GPU; 'cores' is the BLAS thread count (the "
                  f"elementwise passes run on one thread)",
        **host,
        "full_share_s_extrapolated": round(share_flops / rate, 1),
        "extrapolation": "whole share's effective FLOPs / the sample's rate (not measured)",
    }


def cpu_baseline_full(wl, rank):
    """Time the float64 CPU oracle on the whole share (every local row of every
    query head), with all BLAS threads and with one; for shares small enough
    to finish in seconds."""
    import oracle
    import ring_inputs
    from threadpoolctl import threadpool_info, threadpool_limits
    positions = oracle.device_positions(wl.partition, wl.world, rank, wl.local_len)
    k_pos = np.arange(wl.total_len)
    G = wl.heads_q // wl.heads_kv
    vis = oracle.visible_pair_count(positions, k_pos, wl.causal)
    flops = 4.0 * wl.head_dim * vis * wl.heads_q * wl.batch

    def run():
        t0 = time.perf_counter()
        for b in range(wl.batch):
            for g in range(wl.heads_kv):
                kh = ring_inputs.head(wl, "k", b, g)
                vh = ring_inputs.head(wl, "v", b, g)
                for h in range(g * G, (g + 1) * G):
                    q = ring_inputs.rows(wl, "q", b, h, positions)
                    oracle.attention_rows(q, positions, kh, vh, k_pos, wl.causal)
        return time.perf_counter() - t0

    host = host_info()
    threads = host["blas_threads"] or 1
    t_all = run()
    with threadpool_limits(limits=1, user_api="blas"):
        t_one = run()
    what = (f"the full share: {wl.local_len} rows of device {rank} x {wl.heads_q} query heads x batch {wl.batch}, "
            f"float64 full softmax over all {wl.total_len} global keys (input generation included)")
    return {
        "value": flops / t_all / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{what}, {t_all:.2f} s",
        **host,
        "full_share_s": round(t_all, 3),
        "single_thread": {"value": flops / t_one / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": round(t_one, 3)},
    }


def load_balance(wl):
    """Visible (query, key) pairs of every device over the whole ring, per
    (batch, head): the work each device does for its rows."""
    from ring_attention_blockwise_amd import harness
    per_dev = [sum(harness.step_pairs(wl, r)) for r in range(wl.world)]
    mean = sum(per_dev) / len(per_dev)
    return {"partition": wl.partition, "max_over_mean": round(max(per_dev) / mean, 4),
            "min_over_mean": round(min(per_dev) / mean, 4),
            "pairs_max": int(max(per_dev)), "pairs_min": int(min(per_dev))}


def mfma_probe(blocks=256 * 8, iters=2048, reps=3):
    """Dense bf16 MFMA rate and shader clock from the library's matrix-core
    probe (the step kernel's instruction on register operands, every CU)."""
    import torch
    import ring_attention_blockwise_amd as ra
    dev = torch.device("cuda:0")
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stamps = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    ra.mfma_probe(blocks, iters, sink, stamps)  # warm-up
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ra.mfma_probe(blocks, iters, sink, stamps)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    st = stamps.view(blocks, 4).cpu().numpy().astype(np.float64)
    ratio = (st[:, 1] - st[:, 0]) / np.maximum(st[:, 3] - st[:, 2], 1.0)
    flops = blocks * 4 * iters * 4 * 32768.0
    tflops = flops / (best * 1e-3) / 1e12
    return {"instruction": "v_mfma_f32_32x32x16_bf16", "tflops": round(tflops, 1), "ms": round(best, 4),
            "frac_of_spec": round(tflops / PEAK_BF16_TFLOPS, 4),
            "shader_clock_ghz": round(float(np.median(ratio)) * REALTIME_GHZ, 3)}


# Sources the bf16 step kernel is built from; a counter summary is only used
# while their digest matches the one recorded with it.
KERNEL_SOURCES = ("step_bf16.hip", "bf16_tiles.h", "common.h")


BACKWARD_SOURCES = ("backward_bf16.hip", "backward.h", "bf16_tiles.h", "common.h")


def traffic_from_profile(kernel_name, workload_name, sources=KERNEL_SOURCES):
    """HBM bytes per launch (per step for the backward pair) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source;
    else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload_name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    digest = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "ring_attention_blockwise_amd", "csrc", name), "rb") as f:
            digest.update(f.read())
    if rec.get("source_sha256") != digest.hexdigest():
        return None
    return rec.get("bytes_per_launch")


def receive_modes(share, ws, out, lse, K, copy_stream, timed_ms, timed_mode, rounds=5):
    """The forward with each receive copy, and the same step kernels with no
    receive at all (ring_attn_step over the blocks in place, no finalize:
    the fused finalize of the last step writes less than a plain step, so
    this baseline is, if anything, slightly slow). The forwards run without
    a key split, as the baseline's steps do. The modes are timed in
    turn, `rounds` times over, and each reports its median (ms per forward),
    so that clock drift over the run does not favour one of them; overhead
    = forward / no-receive - 1."""
    import torch
    from ring_attention_blockwise_amd import harness
    cur = torch.cuda.current_stream()
    wl = share.workload
    n = max(2, K // 2)

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(n):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    state = harness.new_state(share)

    # without a key split, like the step calls of the baseline
    def fwd(mode, cs):
        return lambda: harness.run_forward(share, copy_stream=cs, workspace=ws, out=out, lse=lse, receive=mode,
                                           key_split=1)

    modes = {"no_receive": lambda: harness.run_steps(share, range(wl.world), state=state),
             "fused": fwd("fused", None), "memcpy_side_stream": fwd("memcpy", copy_stream),
             "memcpy_compute_stream": fwd("memcpy", None)}
    for fn in modes.values():
        fn()
    torch.cuda.synchronize()
    runs = {k: [] for k in modes}
    for _ in range(rounds):
        for k, fn in modes.items():
            runs[k].append(timed(fn))
    ms = {k: float(np.median(v)) for k, v in runs.items()}
    base = ms["no_receive"]
    return {"timed_forwards": timed_mode, "rounds": rounds, "forwards_per_round": n,
            "ms": {k: round(v, 4) for k, v in ms.items()},
            "overhead_vs_no_receive": {k: round(v / base - 1.0, 4) for k, v in ms.items() if k != "no_receive"},
            "timed_forward_overhead": round(timed_ms / base - 1.0, 4)}


def hbm_kernels(share, reps=20):
    """GB/s of the HBM-bound pieces of the path at the share's shapes: the
    state merge, the finalize pass and the D2D receive copy of one K block
    (the copy ring_attn_forward issues). Bytes are the algorithmic ones: every
    operand read once and every result written once."""
    import torch
    import ring_attention_blockwise_amd as ra
    from ring_attention_blockwise_amd import harness

    wl = share.workload
    rd = share.ring_desc()
    sd, _ = ra.ring_step_desc(rd, 0)
    state_a = harness.run_steps(share, [0])
    state_b = harness.run_steps(share, [1] if wl.world > 1 else [0])
    out, lse = harness.alloc_outputs(share)
    k0 = share.k_blocks[0]
    recv = torch.empty_like(k0)
    cur = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(reps):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    o_bytes = state_a[0].numel() * 4
    ml_bytes = 2 * state_a[1].numel() * 4
    out_bytes = out.numel() * out.element_size() + lse.numel() * 4
    res = {}
    for name, fn, nbytes in (
        ("merge", lambda: ra.merge(sd, *state_a, *state_b), 3 * (o_bytes + ml_bytes)),
        ("finalize", lambda: ra.finalize(sd, *state_a, out, lse), o_bytes + ml_bytes + out_bytes),
        ("receive_copy", lambda: recv.copy_(k0), 2 * k0.numel() * k0.element_size()),
    ):
        ms = timed(fn)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"ms": round(ms, 4), "bytes": int(nbytes), "GB/s": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def bench_ulysses(wl, rank, K, Wm):
    """One device's Ulysses share: the whole call (gather, attention, scatter)
    and, separately, its local attention on already head-sharded tensors;
    the difference is the time of the two simulated all-to-alls."""
    import torch
    import ring_attention_blockwise_amd as ra
    from ring_attention_blockwise_amd import harness

    dev = torch.device("cuda:0")
    P = wl.world
    hr, hkr = wl.heads_q // P, wl.heads_kv // P
    heads_q = list(range(rank * hr, (rank + 1) * hr))
    heads_kv = list(range(rank * hkr, (rank + 1) * hkr))
    q, k, v = harness.build_ulysses_shards(wl, dev, heads_q=heads_q, heads_kv=heads_kv)
    dt = harness.torch_dtype(wl)
    dtype = ra.BF16 if wl.dtype == "bf16" else ra.F32
    L, B, d = wl.total_len, wl.batch, wl.head_dim
    outs = [torch.empty((B, wl.heads_q, wl.local_len, d), dtype=dt, device=dev) for _ in range(P)]
    lses = [torch.empty((B, wl.heads_q, wl.local_len), dtype=torch.float32, device=dev) for _ in range(P)]
    ud = ra.ulysses_desc(B, wl.heads_q, wl.heads_kv, d, L, P, rank, dtype=dtype, causal=wl.causal)
    ws = torch.empty(ra.ulysses_workspace_size(ud), dtype=torch.uint8, device=dev)
    # the same attention on already head-sharded tensors: a one-device ring is
    # exactly the single fused init+finalize launch the Ulysses call makes
    qf = torch.cat([x[:, heads_q] for x in q], dim=2).contiguous()
    kf = torch.cat([x[:, heads_kv] for x in k], dim=2).contiguous()
    vf = torch.cat([x[:, heads_kv] for x in v], dim=2).contiguous()
    rd = ra.ring_desc(B, hr, hkr, d, L, 1, 0, partition="contiguous", dtype=dtype, causal=wl.causal)
    ws_r = torch.empty(ra.forward_workspace_size(rd), dtype=torch.uint8, device=dev)
    out_f = torch.empty((B, hr, L, d), dtype=dt, device=dev)
    lse_f = torch.empty((B, hr, L), dtype=torch.float32, device=dev)
    cur = torch.cuda.current_stream()

    def whole():
        ra.ulysses_forward(ud, q, k, v, outs, lses, ws)

    def attention():
        ra.forward(rd, qf, [kf], [vf], out_f, lse_f, ws_r)

    def timed(fn):
        for _ in range(Wm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cur)
        for _ in range(K):
            fn()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    ms_whole = timed(whole)
    ms_attn = timed(attention)
    pairs = L * (L + 1) // 2 if wl.causal else L * L
    flops = 4.0 * d * hr * B * pairs
    es = 2 if wl.dtype == "bf16" else 4
    a2a_bytes = 2 * (B * (hr + 2 * hkr) * L * d * es) + 2 * (B * hr * L * (d * es + 4))  # read + write
    a2a_ms = max(ms_whole - ms_attn, 1e-6)
    value = flops / (ms_whole * 1e-3) / 1e12
    rec = {
        "metric": "effective causal attention TFLOP/s of one device's Ulysses share at 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_whole, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded, bf16-rounded; this device's heads only)",
        "config": {"workload": wl.name, "description": wl.description, "batch": B, "heads_q": wl.heads_q,
                   "heads_kv": wl.heads_kv, "head_dim": d, "global_seq_len": L, "world": P, "rank": rank,
                   "parallelism": "one device's share of simulated DeepSpeed-Ulysses (all-to-alls as D2D copies)"},
        "attention": {"ms": round(ms_attn, 4), "tflops": round(flops / (ms_attn * 1e-3) / 1e12, 2),
                      "frac_of_bf16_peak": round(flops / (ms_attn * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "all_to_all": {"ms": round(a2a_ms, 4), "bytes": int(a2a_bytes),
                       "GB/s": round(a2a_bytes / (a2a_ms * 1e-3) / 1e9, 1)},
    }
    print(json.dumps(rec), flush=True)


def bench_backward(wl, rank, K, Wm):
    """One device's backward pass over the whole ring (ring_attn_backward):
    row terms, one dQ and one dK/dV launch per step, dQ conversion. The
    forward output and LSE it reads are computed once, outside the timing.
    Effective FLOPs are the usual backward count, 10 * d * H_q * B per
    visible pair (five products of the forward's size); the kernels execute
    14 (S and dP are formed by both kernels)."""
    import torch
    import ring_attention_blockwise_amd as ra
    from ring_attention_blockwise_amd import harness

    dev = torch.device("cuda:0")
    share = harness.build_share(wl, rank, dev)
    copy_stream = torch.cuda.Stream()
    out, lse = harness.run_forward(share, copy_stream=copy_stream)
    d_out = harness.build_upstream(share)
    dk, dv = harness.new_kv_grads(share)
    ws = torch.empty(ra.backward_workspace_size(share.ring_desc()), dtype=torch.uint8, device=dev)
    pairs = harness.step_pairs(wl, rank)
    launched = [s for s in range(wl.world) if pairs[s] > 0]
    per_pair = 10.0 * wl.head_dim * wl.heads_q * wl.batch
    total_flops = per_pair * sum(pairs)
    events = [ra.StepEvents(2 * wl.world) for _ in range(K)]
    cur = torch.cuda.current_stream()
    for _ in range(Wm):
        harness.run_backward(share, out, lse, d_out, dk, dv, copy_stream=copy_stream, workspace=ws)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(cur)
    for i in range(K):
        harness.run_backward(share, out, lse, d_out, dk, dv, copy_stream=copy_stream, workspace=ws,
                             step_events=events[i])
    stop.record(cur)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / K
    step_ms = sum(ev.elapsed_ms(2 * s, 2 * s + 1) for ev in events for s in launched) / (K * len(launched))
    flops_per_step = per_pair * sum(pairs[s] for s in launched) / len(launched)
    achieved = flops_per_step / (step_ms * 1e-3) / 1e12
    value = total_flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": "effective causal attention-backward TFLOP/s of one device's ring share at 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic (seeded Q/K/V as the workload states, dO N(0,1); bf16-rounded)",
        "config": {"workload": wl.name, "pass": "backward", "description": wl.description, "batch": wl.batch,
                   "heads_q": wl.heads_q, "heads_kv": wl.heads_kv, "head_dim": wl.head_dim,
                   "local_len": wl.local_len, "world": wl.world, "rank": rank, "partition": wl.partition},
        "effective_tflop_per_backward": round(total_flops / 1e12, 4),
        "step_kernels": {"launch_pairs_per_backward": len(launched), "avg_step_ms": round(step_ms, 4),
                         "tflops": round(achieved, 2),
                         "executed_mfma_tflops": round(achieved * 1.4, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_from_profile("backward_bf16", wl.name, BACKWARD_SOURCES)},
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--receive", default="auto", choices=["auto", "memcpy", "fused"],
                    help="receive copy of the timed forwards (memcpy: hipMemcpyAsync on a side stream)")
    ap.add_argument("--key-split", type=int, default=0,
                    help="key split of the bf16 forward: 0 automatic (small shares), 1 never, 2..16 forced")
    ap.add_argument("--forwards-only", action="store_true",
                    help="time the forwards and skip every other measurement (for kernel traces)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass of the workload's share instead of the forward")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU: the ring is simulated on a single device "
                                   "(one device's share at its real shape); run with --gpus 1"}))
        sys.exit(2)

    import torch
    import ring_inputs
    import ring_attention_blockwise_amd as ra
    from ring_attention_blockwise_amd import harness

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    ra.lib()  # fail loudly if the HIP library is not built

    if args.workload in ring_inputs.ULYSSES_WORKLOADS:
        wl = ring_inputs.ULYSSES_WORKLOADS[args.workload]
        bench_ulysses(wl, wl.ranks[0] if args.rank is None else args.rank, args.steps, args.warmup)
        return
    wl = ring_inputs.WORKLOADS[args.workload]
    rank = wl.ranks[0] if args.rank is None else args.rank
    if args.backward:
        bench_backward(wl, rank, args.steps, args.warmup)
        return
    dev = torch.device("cuda:0")
    t0 = time.time()
    share = harness.build_share(wl, rank, dev)
    torch.cuda.synchronize()
    log(f"built {wl.name} share of device {rank} in {time.time() - t0:.1f} s")

    pairs = harness.step_pairs(wl, rank)
    flops = effective_flops(wl, pairs)
    total_flops = sum(flops)
    launched = [s for s in range(wl.world) if pairs[s] > 0]

    out, lse = harness.alloc_outputs(share)
    ksplit = args.key_split
    args.key_split_effective = harness.effective_key_split(share, ksplit)
    ws = harness.alloc_workspace(share, key_split=ksplit)
    copy_stream = torch.cuda.Stream()
    cur = torch.cuda.current_stream()
    K, Wm = args.steps, args.warmup
    events = [ra.StepEvents(2 * wl.world) for _ in range(K)]

    recv = args.receive
    for _ in range(Wm):
        harness.run_forward(share, copy_stream=copy_stream, workspace=ws, out=out, lse=lse, receive=recv,
                            key_split=ksplit)
    torch.cuda.synchronize()
    log(f"warmup done ({Wm} forwards)")

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(cur)
    wall0 = time.perf_counter()
    for i in range(K):
        harness.run_forward(share, copy_stream=copy_stream, workspace=ws, out=out, lse=lse,
                            step_events=events[i], receive=recv, key_split=ksplit)
    stop.record(cur)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K
    log(f"timed {K} forwards: {ms_per_step:.3f} ms each (host wall {1e3 * wall / K:.3f} ms)")

    kernel_ms = 0.0
    per_step_ms = np.zeros(wl.world)
    for ev in events:
        for s in launched:
            t = ev.elapsed_ms(2 * s, 2 * s + 1)
            per_step_ms[s] += t / K
            kernel_ms += t
    n_launch = K * len(launched)
    avg_launch_ms = kernel_ms / max(1, n_launch)
    flops_per_launch = sum(flops[s] for s in launched) / max(1, len(launched))
    achieved = flops_per_launch / (avg_launch_ms * 1e-3) / 1e12 if n_launch else 0.0
    bf16 = wl.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    kernel_name = "step_bf16" if bf16 else "step_f32"
    traffic = traffic_from_profile(kernel_name, wl.name)
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    if args.forwards_only:
        graph_ms = receive = hbm = probe = balance = cpu = None
        args.no_cpu_baseline = True
    else:
        graph_ms, receive, hbm, probe, balance = extras(share, ws, out, lse, K, copy_stream, ms_per_step, recv, wl,
                                                        ksplit)
    cpu = None
    if not args.no_cpu_baseline:
        if wl.local_len * wl.heads_q * wl.batch * wl.total_len <= SMALL_SHARE_PAIRS:
            log("timing the CPU oracle on the whole share (all threads, then one)")
            cpu = cpu_baseline_full(wl, rank)
        else:
            log("timing the CPU oracle on a bounded sample")
            cpu = cpu_baseline(wl, rank, total_flops)
    rec = record(args, wl, rank, K, Wm, value, ms_per_step, bf16, total_flops, launched, avg_launch_ms, per_step_ms,
                 achieved, peak, traffic, receive, graph_ms, hbm, probe, balance, cpu)
    print(json.dumps(rec), flush=True)
    for ev in events:
        ev.close()


def extras(share, ws, out, lse, K, copy_stream, ms_per_step, recv, wl, ksplit):
    """Graph replay, receive modes, HBM-bound kernels, matrix-core probe, load balance."""
    import torch
    from ring_attention_blockwise_amd import harness
    cur = torch.cuda.current_stream()
    # The same forward captured once into a HIP graph and replayed: identical
    # work (every step kernel and receive copy), without per-launch host cost.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        harness.run_forward(share, copy_stream=copy_stream, workspace=ws, out=out, lse=lse, receive=recv,
                            key_split=ksplit)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(cur)
    for _ in range(K):
        graph.replay()
    g1.record(cur)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / K
    del graph
    log(f"graph replay: {graph_ms:.3f} ms per forward")

    receive = receive_modes(share, ws, out, lse, K, copy_stream, ms_per_step, recv)
    log(f"receive: {receive}")

    hbm = hbm_kernels(share)
    log(f"HBM-bound pieces: {hbm}")

    probe = mfma_probe()
    log(f"matrix-core probe: {probe}")
    balance = load_balance(wl)
    return graph_ms, receive, hbm, probe, balance


def record(args, wl, rank, K, Wm, value, ms_per_step, bf16, total_flops, launched, avg_launch_ms, per_step_ms,
           achieved, peak, traffic, receive, graph_ms, hbm, probe, balance, cpu):
    rec = {
        "metric": "effective causal attention TFLOP/s per ring step at 1 GPU; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16-rounded)",
        "config": {
            "workload": wl.name, "description": wl.description, "batch": wl.batch, "heads_q": wl.heads_q,
            "heads_kv": wl.heads_kv, "head_dim": wl.head_dim, "local_len": wl.local_len,
            "global_seq_len": wl.total_len, "world": wl.world, "rank": rank, "partition": wl.partition,
            "ring_steps": wl.world, "parallelism": "one device's share of a simulated ring",
            "receive": args.receive,
            "key_split": args.key_split_effective,
        },
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "effective_tflop_per_forward": round(total_flops / 1e12, 4),
        "step_kernel": {
            "launches_per_forward": len(launched),
            "avg_launch_ms": round(avg_launch_ms, 4),
            "per_step_ms": [round(x, 4) for x in per_step_ms.tolist()],
            "tflops": round(achieved, 2),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
        },
        "receive": receive,
        "graph_forward": None if graph_ms is None else {
            "ms_per_forward": round(graph_ms, 4), "value": round(total_flops / (graph_ms * 1e-3) / 1e12, 3)},
        "hbm_kernels": hbm,
        "mfma_probe": None if probe is None else dict(
            probe, step_kernel_frac_of_probe=round(achieved / probe["tflops"], 4) if bf16 else None),
        "load_balance": balance,
        "cpu_baseline": cpu,
    }
    return rec


if __name__ == "__main__":
    main()
