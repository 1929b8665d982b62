"""Benchmark: NVFP4 W4A16 matmul on one MI355X.

Default workload (one JSON line on stdout): the square projection, K = N =
5120, M = 1, with 64 byte-identical NVFP4 weight copies (943.7 MB, past the
256 MB Infinity Cache) cycled call after call.  One step = one pass over the
64 copies (64 calls), captured once in a HIP graph and replayed.  Metric:
effective weight GB/s = (N*K/2 codes + N*K/16 scales + 4 B g) per call / time
per call, with % of the 8 TB/s HBM peak.  Exactly --steps replays are timed
(HIP events on the replay stream, split into 5 windows whose median and
minimum are also reported), after --warmup untimed replays.

The same line carries the metric's two operating points (M = 1 decode and
M = 7, a verify block of 6 drafts + 1) on the configurations that define
them: the square projection at M = 7, the fused gate/up + SwiGLU (K = 5120,
2 x N = 17408, 32 layer copies) and the down projection (K = 17408,
N = 5120, 32 copies), each at M = 1, 7 and 32 with median and minimum over 5
timed windows; the oracle timed on the host (one thread and all cores); an
achievable-read calibration; and the full-tower decode sweep (64 layers of
gate/up, down and q/k/v/o plus the 5120 -> 248320 head, M = 1 and 7; skip it
with --no-tower).  `--extra` adds the down projection at M = 2, 4, 8, 16
and the MLP block.

Inputs are resident in HBM before any timed region starts.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_square_m1.json")
WINDOWS = 5


def kernel_source_hash():
    """Hash of the matmul library's HIP sources: a stored traffic measurement is
    used only if it was taken on exactly these kernels (the calibration kernel's
    source, calib.hip, is not part of them)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_w4a16_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")) and not name.startswith("calib"):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """Calibrated HBM bytes per launch of the square GEMV from the committed
    rocprofv3 PMC runs, or None when absent or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def weight_bytes(N, K):
    return N * K // 2 + N * K // 16 + 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev_u8(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_dev_bf16(bits, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def replicate(t, copies):
    """`copies` byte-identical replicas in distinct allocations."""
    return [t.clone() for _ in range(copies)]


def gpu_weights(seed, N, K, dev):
    """W ~ N(0, 0.02) fp32 drawn on the device from a seeded generator and
    NVFP4-encoded by the library's quantiser (w4a16_quantize, bit-exact to the
    oracle's recipe): (wq, ws, g) device tensors.  Used for the large
    configurations, whose host-side encoding would take tens of seconds;
    the bytes differ from synth's, the distribution and recipe do not."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    w = torch.randn((N, K), generator=gen, device=dev, dtype=torch.float32).mul_(0.02)
    wq, ws, g = w4.quantize(w)
    del w
    torch.cuda.synchronize()
    return wq, ws, g


def capture(fns, stream):
    """A HIP graph holding one call of each fn(stream) (after one eager warm
    call of each on the capture stream)."""
    import torch
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        for f in fns:
            f(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        for f in fns:
            f(cap)
    torch.cuda.synchronize()
    return graph


def timed_replays(graph, stream, steps, windows=WINDOWS):
    """Replay `graph` exactly `steps` times on `stream`, bracketed by device
    synchronisation; HIP events split the replays into `windows` windows.
    Returns (total seconds, [seconds per replay of each window])."""
    import torch
    windows = max(1, min(windows, steps))
    bounds = [round(i * steps / windows) for i in range(windows + 1)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(windows + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for w in range(windows):
            for _ in range(bounds[w + 1] - bounds[w]):
                graph.replay()
            ev[w + 1].record(stream)
    ev[-1].synchronize()
    torch.cuda.synchronize()
    total = ev[0].elapsed_time(ev[-1]) * 1e-3
    per = [ev[w].elapsed_time(ev[w + 1]) * 1e-3 / (bounds[w + 1] - bounds[w]) for w in range(windows)]
    return total, per


def warm(graph, stream, seconds=0.05):
    """Untimed replays for at least `seconds`, so that the configuration timed
    next runs at steady clocks."""
    import torch
    t0 = time.perf_counter()
    while True:
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break


def config_line(calls_per_replay, bytes_per_call, per_window, replays_per_window):
    """µs per call, GB/s and fraction of peak from the median window, and the
    fastest window."""
    us = [p / calls_per_replay * 1e6 for p in per_window]
    med, mn = statistics.median(us), min(us)
    gbs = bytes_per_call / (med * 1e-6) / 1e9
    return {"us_per_call": round(med, 3), "us_per_call_min": round(mn, 3), "gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "windows": len(us),
            "calls_timed": calls_per_replay * replays_per_window * len(us)}


def time_config(fns, stream, bytes_per_call, replays_per_window=2):
    graph = capture(fns, stream)
    warm(graph, stream)
    _, per = timed_replays(graph, stream, replays_per_window * WINDOWS)
    del graph
    return config_line(len(fns), bytes_per_call, per, replays_per_window)


# ---- the default workload: square projection, M = 1 ------------------------------

def square_setup(dev):
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    c = synth.CONFIGS["square"]
    N, K, copies = c["N"], c["K"], c["copies"]
    log(f"[bench] generating square K={K} N={N} x{copies} copies")
    wq, ws, g = synth.nvfp4_weights(c["seed_w"], N, K)
    x = to_dev_bf16(synth.activations(c["seed_x"], 1, K), dev)
    wqs = replicate(to_dev_u8(wq, dev), copies)
    wss = replicate(to_dev_u8(ws, dev), copies)
    gs = replicate(torch.tensor([g], dtype=torch.float32, device=dev), copies)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    work = w4.new_workspace(1, N, K, dev)   # zeroed once; every call leaves it zeroed
    return dict(N=N, K=K, copies=copies, wqs=wqs, wss=wss, gs=gs, x=x, y=y, work=work, seed_x=c["seed_x"])


def square_fns(sq, x, y, work):
    import block_scaled_fp4_w4a16_amd as w4
    return [lambda s, i=i: w4.gemm(sq["wqs"][i], sq["wss"][i], sq["gs"][i], x, y=y, workspace=work, stream=s)
            for i in range(sq["copies"])]


def bench_square(args, dev, stream, sq):
    """One step = the 64 calls, captured once in a HIP graph; `warmup`
    untimed replays, then exactly `steps` timed replays."""
    import torch
    graph = capture(square_fns(sq, sq["x"], sq["y"], sq["work"]), stream)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    t0 = time.perf_counter()
    total, per = timed_replays(graph, stream, args.steps)
    wall = time.perf_counter() - t0
    del graph
    calls = args.steps * sq["copies"]
    return dict(total=total, wall=wall, per_window=per, calls=calls, per_call=total / calls)


def profile_square(args, dev, stream):
    """Only the default workload's graph replays (for a rocprofv3 kernel
    trace whose dispatches are exactly the timed calls and their warm-up)."""
    sq = square_setup(dev)
    r = bench_square(args, dev, stream, sq)
    bpc = weight_bytes(sq["N"], sq["K"])
    print(json.dumps({"mode": "profile-square", "steps": args.steps, "warmup": args.warmup,
                      "calls_timed": r["calls"], "us_per_call": round(r["per_call"] * 1e6, 4),
                      "gbs": round(bpc / r["per_call"] / 1e9, 1)}), flush=True)


PROFILE_CONFIGS = ("square_M1", "square_M7", "gate_up_M1", "gate_up_M7", "down_M1", "down_M7")


def profile_config(args, dev, stream):
    """Only one configuration's graph replays (for rocprofv3 passes that must
    see that configuration's dispatches alone): `--steps` replays of its 32-64
    calls after `--warmup`."""
    name = args.config
    kind, m = name.rsplit("_M", 1)
    M = int(m)
    if kind == "square":
        fns, b = square_m_fns(square_setup(dev), M, dev)
    elif kind == "gate_up":
        Gs, Us = gate_up_weights(dev)
        fns, b = gate_up_fns(Gs, Us, M, dev)
    else:
        fns, b = down_fns(down_weights(dev), M, dev)
    graph = capture(fns, stream)
    with torch_stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    total, per = timed_replays(graph, stream, args.steps)
    calls = args.steps * len(fns)
    print(json.dumps({"mode": "profile-config", "config": name, "calls_timed": calls,
                      "bytes_per_call": b, "us_per_call": round(total / calls * 1e6, 4)}), flush=True)


def torch_stream(stream):
    import torch
    return torch.cuda.stream(stream)


# ---- the metric's configurations ------------------------------------------------

def gate_up_weights(dev):
    """The gate/up configuration's weights: (gate, up) lists of 32 copies of
    (wq, ws, g) device tensors each, as [wq copies], [ws copies], [g copies]."""
    import synth
    c = synth.CONFIGS["gate_up"]
    N, K, copies = c["N"], c["K"], c["copies"]
    log(f"[bench] generating gate/up K={K} 2 x N={N} x{copies} (device quantiser)")
    G = gpu_weights(c["seed_gate"], N, K, dev)
    U = gpu_weights(c["seed_up"], N, K, dev)
    return [replicate(t, copies) for t in G], [replicate(t, copies) for t in U]


def down_weights(dev):
    """The down configuration's weights: [wq copies], [ws copies], [g copies]."""
    import synth
    c = synth.CONFIGS["down"]
    N, K, copies = c["N"], c["K"], c["copies"]
    log(f"[bench] generating down K={K} N={N} x{copies} (device quantiser)")
    return [replicate(t, copies) for t in gpu_weights(c["seed_w"], N, K, dev)]


def gate_up_fns(Gs, Us, M, dev):
    """One call per weight copy of gate/up + SwiGLU at M rows, and its bytes."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    c = synth.CONFIGS["gate_up"]
    N, K, copies = c["N"], c["K"], c["copies"]
    x = to_dev_bf16(synth.activations(c["seed_x"], M, K), dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    work = w4.new_workspace(M, N, K, dev, fused=True)
    fns = [lambda s, i=i: w4.gemm_gate_up_swiglu(Gs[0][i], Gs[1][i], Gs[2][i], Us[0][i], Us[1][i], Us[2][i],
                                                 x, y=y, workspace=work, stream=s) for i in range(copies)]
    return fns, 2 * weight_bytes(N, K)


def down_fns(Ds, M, dev):
    """One call per weight copy of the down projection at M rows, and its bytes."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    c = synth.CONFIGS["down"]
    N, K, copies = c["N"], c["K"], c["copies"]
    x = to_dev_bf16(synth.swiglu_activations(c["seed_a"], c["seed_b"], M, K), dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    work = w4.new_workspace(M, N, K, dev)
    fns = [lambda s, i=i: w4.gemm(Ds[0][i], Ds[1][i], Ds[2][i], x, y=y, workspace=work, stream=s)
           for i in range(copies)]
    return fns, weight_bytes(N, K)


def square_m_fns(sq, M, dev):
    """One call per weight copy of the square projection at M rows, and its bytes."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    x = to_dev_bf16(synth.activations(sq["seed_x"], M, sq["K"]), dev)
    y = torch.empty((M, sq["N"]), dtype=torch.bfloat16, device=dev)
    return square_fns(sq, x, y, w4.new_workspace(M, sq["N"], sq["K"], dev)), weight_bytes(sq["N"], sq["K"])


def bench_configs(dev, stream, sq, extra=False):
    """Square M = 7; gate/up + SwiGLU M = 1, 7, 32; down M = 1, 7, 32 (with
    --extra also down M = 2, 4, 8, 16 and the MLP block).  M = 32, a wide
    verify or prefill block, runs the 32 x 32 x 16 MFMA kernel."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    out = {}
    fns, b = square_m_fns(sq, 7, dev)
    out["square_M7"] = time_config(fns, stream, b, replays_per_window=2)
    log(f"[bench] square M=7: {out['square_M7']['us_per_call']} us/call, {out['square_M7']['gbs']} GB/s")

    Gs, Us = gate_up_weights(dev)
    for M in (1, 7, 32):
        fns, b = gate_up_fns(Gs, Us, M, dev)
        out[f"gate_up_M{M}"] = time_config(fns, stream, b)
        log(f"[bench] gate/up M={M}: {out[f'gate_up_M{M}']['us_per_call']} us/call, {out[f'gate_up_M{M}']['gbs']} GB/s")

    Ds = down_weights(dev)
    for M in ((1, 2, 4, 7, 8, 16, 32) if extra else (1, 7, 32)):
        fns, b = down_fns(Ds, M, dev)
        out[f"down_M{M}"] = time_config(fns, stream, b)
        log(f"[bench] down M={M}: {out[f'down_M{M}']['us_per_call']} us/call, {out[f'down_M{M}']['gbs']} GB/s")
    N, K, copies = synth.CONFIGS["down"]["N"], synth.CONFIGS["down"]["K"], synth.CONFIGS["down"]["copies"]

    if extra:
        # the whole MLP block per call: two launches (graph replay), and eager
        # calls with one (cooperative) launch and with two
        H, F = N, K
        b = 2 * weight_bytes(F, H) + weight_bytes(H, F)
        for M in (1, 7):
            x = to_dev_bf16(synth.activations(synth.CONFIGS["gate_up"]["seed_x"], M, H), dev)
            y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
            work = w4.new_workspace_mlp(M, H, F, dev)

            def call(s, i, one):
                w4.mlp_swiglu((Gs[0][i], Gs[1][i], Gs[2][i]), (Us[0][i], Us[1][i], Us[2][i]),
                              (Ds[0][i], Ds[1][i], Ds[2][i]), x, y=y, workspace=work, stream=s, one_launch=one,
                              check_barrier=False)
            res = {"one_launch_possible": w4.mlp_one_launch(M, H, F)}
            res["two_launches_graph"] = time_config([lambda s, i=i: call(s, i, False) for i in range(copies)],
                                                    stream, b)
            for one, name in ((True, "one_launch_eager"), (False, "two_launches_eager")):
                if one and res["one_launch_possible"] != 1:
                    continue  # the call would run as two launches
                for i in range(copies):
                    call(stream, i, one)
                torch.cuda.synchronize()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                for _ in range(4):
                    for i in range(copies):
                        call(stream, i, one)
                ev1.record(stream)
                ev1.synchronize()
                t = ev0.elapsed_time(ev1) * 1e-3 / (4 * copies)
                if one and w4.mlp_timed_out(work):
                    raise RuntimeError("one-launch MLP barrier timed out during the timed calls")
                res[name] = {"us_per_call": round(t * 1e6, 3), "gbs": round(b / t / 1e9, 1)}
            out[f"mlp_M{M}"] = res
            log(f"[bench] mlp block M={M}: {json.dumps(res)}")
    del Gs, Us, Ds
    torch.cuda.empty_cache()
    return out


def bench_tower(dev, stream, Ms=(1, 7), layers=64, replays=5):
    """Full-tower decode sweep, one token = one HIP graph replay of
    `layers` x (the MLP block: gate/up + SwiGLU 5120 -> 2 x 17408 and down
    17408 -> 5120, two launches; q, k, v, o 5120 -> 5120) followed by the
    5120 -> 248320 head GEMV with fused greedy argmax (the head alone is also
    timed with and without it): 385 launches and 14.1 GB of distinct weight
    allocations per token.  The MLP chain is wired (SwiGLU output feeds down,
    down's output feeds the next layer's gate/up); q/k/v/o and the head read
    fixed synthetic activations (there is no attention).  Weights per layer
    are byte-identical replicas of one encoded matrix per kind; the head
    matrix tiles the rows of the square matrix, since HBM traffic depends on
    the addresses read, not on the values."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    H, F, V = 5120, 17408, 248320
    cg, cd, cs = synth.CONFIGS["gate_up"], synth.CONFIGS["down"], synth.CONFIGS["square"]
    log(f"[bench] tower: encoding gate/up/down/square, {layers} layers + head")
    enc = {"gate": gpu_weights(cg["seed_gate"], F, H, dev), "up": gpu_weights(cg["seed_up"], F, H, dev),
           "down": gpu_weights(cd["seed_w"], H, F, dev)}
    sq = synth.nvfp4_weights(cs["seed_w"], H, H)
    enc["sq"] = (to_dev_u8(sq[0], dev), to_dev_u8(sq[1], dev),
                 torch.tensor([sq[2]], dtype=torch.float32, device=dev))

    def copies(kind, n):
        return [tuple(t.clone() for t in enc[kind]) for _ in range(n)]
    L = {"gate": copies("gate", layers), "up": copies("up", layers), "down": copies("down", layers),
         "q": copies("sq", layers), "k": copies("sq", layers), "v": copies("sq", layers),
         "o": copies("sq", layers)}
    reps = (V + H - 1) // H
    head = (torch.cat([enc["sq"][0]] * reps)[:V].contiguous(),
            torch.cat([enc["sq"][1]] * reps)[:V].contiguous(), enc["sq"][2].clone())
    del enc
    b_layer = 2 * weight_bytes(F, H) + weight_bytes(H, F) + 4 * weight_bytes(H, H)
    b_token = layers * b_layer + weight_bytes(V, H)
    out = {}
    for M in Ms:
        x0 = to_dev_bf16(synth.activations(cg["seed_x"], M, H), dev)
        xa = to_dev_bf16(synth.activations(cs["seed_x"], M, H), dev)
        xs = [torch.empty((M, H), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        ya = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        logits = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
        wk_mlp = w4.new_workspace_mlp(M, H, F, dev)
        wk_sq = w4.new_workspace(M, H, H, dev)
        wk_hd0 = w4.new_workspace(M, V, H, dev)
        wk_hd = torch.zeros(w4.workspace_size_argmax(M, V, H), dtype=torch.uint8, device=dev)
        tok_idx = torch.empty((M,), dtype=torch.int32, device=dev)
        tok_val = torch.empty((M,), dtype=torch.float32, device=dev)

        def token(s):
            x = x0
            for i in range(layers):
                nx = xs[i % 2]
                w4.mlp_swiglu(L["gate"][i], L["up"][i], L["down"][i], x, y=nx, workspace=wk_mlp, stream=s)
                for kind in ("q", "k", "v", "o"):
                    q = L[kind][i]
                    w4.gemm(q[0], q[1], q[2], xa, y=ya, workspace=wk_sq, stream=s)
                x = nx
            w4.gemm_argmax(head[0], head[1], head[2], x, idx=tok_idx, val=tok_val, workspace=wk_hd, stream=s)

        g = capture([token], stream)
        warm(g, stream)
        _, per = timed_replays(g, stream, replays)
        t = statistics.median(per)
        del g
        gh = capture([lambda s: w4.gemm(head[0], head[1], head[2], x0, y=logits, workspace=wk_hd0, stream=s)] * 8,
                     stream)
        warm(gh, stream)
        _, ph = timed_replays(gh, stream, replays)
        t_head = statistics.median(ph) / 8
        del gh
        ga = capture([lambda s: w4.gemm_argmax(head[0], head[1], head[2], x0, idx=tok_idx, val=tok_val,
                                               workspace=wk_hd, stream=s)] * 8, stream)
        warm(ga, stream)
        _, pa = timed_replays(ga, stream, replays)
        t_am = statistics.median(pa) / 8
        del ga
        bh = weight_bytes(V, H)
        out[f"head_M{M}"] = dict(us_per_call=round(t_head * 1e6, 2), gbs=round(bh / t_head / 1e9, 1),
                                 argmax_us_per_call=round(t_am * 1e6, 2), argmax_gbs=round(bh / t_am / 1e9, 1))
        out[f"tower_M{M}"] = dict(ms_per_token=round(t * 1e3, 4), tokens_per_s=round(1.0 / t, 2),
                                  launches_per_token=6 * layers + 1, head="fused greedy argmax",
                                  bytes_per_token=b_token, gbs=round(b_token / t / 1e9, 1),
                                  frac=round(b_token / t / 1e9 / HBM_PEAK_GBS, 4))
        log(f"[bench] tower M={M}: {t*1e3:.3f} ms/token, {b_token/t/1e9:.0f} GB/s; head {t_head*1e6:.1f} us, "
            f"with argmax {t_am*1e6:.1f} us")
    return out


# call sizes of the configurations, for the call-sized read calibration:
# (bytes of codes and scales per call, weight copies cycled)
CALL_SIZES = {"square": (5120 * 5120 // 2 + 5120 * 5120 // 16, 64),
              "gate_up": (2 * (17408 * 5120 // 2 + 17408 * 5120 // 16), 32),
              "down": (5120 * 17408 // 2 + 5120 * 17408 // 16, 32)}


def calibration(dev, stream, sizes=CALL_SIZES):
    """Achievable HBM read rates, from a plain 128-bit non-temporal streaming
    read (libw4a16_calib.so, not the matmul library, 8 loads in flight per
    thread): once on a 4 GiB buffer (32 workgroups of 1024 threads per CU: the
    fastest launch shape of a sweep on MI355X), and for each configuration's
    call size over as many buffers of that size as the configuration cycles
    weight copies, one workgroup per CU (the best of 256, 512 and 1024
    threads), in a HIP graph like the benchmark.  The call-sized rates include
    the same per-call fixed costs (launch, first-load latency, tail) as the
    matmul calls, so they are the floor a call of that size can reach."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_scaled_fp4_w4a16_amd", "libw4a16_calib.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m block_scaled_fp4_w4a16_amd.build`")
    lib = ctypes.CDLL(path)
    lib.w4a16_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.w4a16_calib_stream_read.restype = ctypes.c_int
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count

    def read(buf, nbytes, grid, block, s):
        st = lib.w4a16_calib_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                         grid, block, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"calibration read failed ({st})")

    big_bytes = 4 << 30
    big = torch.ones(big_bytes, dtype=torch.uint8, device=dev)
    g = capture([lambda s: read(big, big_bytes, 32 * cus, 1024, s)], stream)
    warm(g, stream)
    _, per = timed_replays(g, stream, 10)
    t_big = statistics.median(per)
    del g, big
    out = {"kind": "plain 128-bit non-temporal streaming read (libw4a16_calib.so)",
           "stream_4gib_gbs": round(big_bytes / t_big / 1e9, 1), "call_sized": {}}
    for name, (nbytes, copies) in sizes.items():
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        best = None
        for block in (256, 512, 1024):
            g = capture([lambda s, i=i: read(bufs[i], nbytes, cus, block, s) for i in range(copies)], stream)
            warm(g, stream)
            _, per = timed_replays(g, stream, 10)
            t = statistics.median(per) / copies
            del g
            if best is None or t < best[0]:
                best = (t, block)
        del bufs
        torch.cuda.empty_cache()
        out["call_sized"][name] = {"bytes": nbytes, "copies": copies, "block": best[1],
                                   "us_per_call": round(best[0] * 1e6, 3),
                                   "gbs": round(nbytes / best[0] / 1e9, 1)}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(window_s=3.0):
    """The CPU oracle (fp64 C, OpenMP over output rows) timed on a bounded
    sample of the default workload: repeated square GEMV calls (M = 1,
    K = N = 5120, the same seeded inputs), median of 3 windows of about
    `window_s` seconds each, at all host threads and at one thread."""
    import oracle
    import synth
    c = synth.CONFIGS["square"]
    N, K = c["N"], c["K"]
    wq, ws, g = synth.nvfp4_weights(c["seed_w"], N, K)
    x = synth.activations(c["seed_x"], 1, K)
    bpc = weight_bytes(N, K)

    def measure(threads):
        oracle.gemm(wq, ws, g, x, 1, N, K, nthreads=threads)   # warm
        t0 = time.perf_counter()
        oracle.gemm(wq, ws, g, x, 1, N, K, nthreads=threads)
        one = time.perf_counter() - t0
        reps = max(1, int(window_s / max(one, 1e-4)))
        per = []
        for _ in range(3):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.gemm(wq, ws, g, x, 1, N, K, nthreads=threads)
            per.append((time.perf_counter() - t0) / reps)
        return statistics.median(per), reps

    all_threads = oracle.max_threads()
    dt_all, reps_all = measure(all_threads)
    dt_one, reps_one = measure(1)
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return dict(value=round(bpc / dt_all / 1e9, 4), unit="GB/s", cores=all_threads, kind="oracle",
                sample=f"square GEMV (M=1, K=N=5120) by the fp64 C oracle, median of 3 windows of "
                       f"{reps_all} calls at {all_threads} threads ({dt_all*1e3:.2f} ms/call) and of "
                       f"{reps_one} calls at 1 thread ({dt_one*1e3:.1f} ms/call)",
                ms_per_call=round(dt_all * 1e3, 3),
                single_thread={"value": round(bpc / dt_one / 1e9, 5), "unit": "GB/s",
                               "ms_per_call": round(dt_one * 1e3, 2), "cores": 1},
                cpu_model=cpu_model(), nproc=os.cpu_count(), affinity_cpus=affinity)


def cpu_baseline_tower(Ms=(1, 7), layers=64):
    """The CPU oracle's time per decode token of the full tower, extrapolated
    from one timed oracle call per matrix shape (all host threads): per token
    `layers` x (gate/up + SwiGLU, down, 4 square projections) + the head.  A
    token of the tower takes the oracle tens of seconds (minutes at M = 7),
    so it is not run whole.  The inputs are seeded random codes and scales of
    the real shapes (the oracle's time does not depend on the values)."""
    import oracle
    import synth
    H, F, V = 5120, 17408, 248320
    threads = oracle.max_threads()
    out = {}
    for M in Ms:
        t = {}
        x_h = synth.integer_activations(91, M, H)
        x_f = synth.integer_activations(92, M, F)
        wq, ws = synth.exact_weights(93, H, H)
        t0 = time.perf_counter()
        oracle.gemm(wq, ws, np.float32(32.0), x_h, M, H, H, nthreads=threads)
        t["square"] = time.perf_counter() - t0
        wg, sg = synth.exact_weights(94, F, H)
        wu, su = synth.exact_weights(95, F, H)
        t0 = time.perf_counter()
        oracle.gate_up_swiglu(wg, sg, np.float32(32.0), wu, su, np.float32(32.0), x_h, M, F, H, nthreads=threads)
        t["gate_up"] = time.perf_counter() - t0
        del wg, sg, wu, su
        wd, sd = synth.exact_weights(96, H, F)
        t0 = time.perf_counter()
        oracle.gemm(wd, sd, np.float32(32.0), x_f, M, H, F, nthreads=threads)
        t["down"] = time.perf_counter() - t0
        del wd, sd
        wh, sh = synth.exact_weights(97, V, H)
        t0 = time.perf_counter()
        oracle.gemm(wh, sh, np.float32(32.0), x_h, M, V, H, nthreads=threads)
        t["head"] = time.perf_counter() - t0
        del wh, sh
        per_token = layers * (t["gate_up"] + t["down"] + 4 * t["square"]) + t["head"]
        bytes_token = layers * (2 * weight_bytes(F, H) + weight_bytes(H, F) + 4 * weight_bytes(H, H)) + \
            weight_bytes(V, H)
        out[f"M{M}"] = {"s_per_token": round(per_token, 3),
                        "tokens_per_s": round(1.0 / per_token, 5),
                        "gbs": round(bytes_token / per_token / 1e9, 4),
                        "s_per_call": {k: round(v, 4) for k, v in t.items()}}
        log(f"[bench] tower oracle M={M}: {per_token:.2f} s/token (extrapolated), calls {out[f'M{M}']['s_per_call']}")
    return dict(kind="oracle", cores=threads, cpu_model=cpu_model(), nproc=os.cpu_count(),
                method=f"{layers} x (gate/up + SwiGLU + down + 4 square projections) + head, from one "
                       f"timed oracle call per shape at {threads} threads", **out)


def copy_calibration(dev, mib=256, reps=4):
    """A plain device-to-device copy of known size, run under the same PMC
    passes as the GEMV to calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n * 4, "reps": reps}), flush=True)


def _csv_rows(d, pattern):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {pattern} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def ingest_pmc(d):
    """Calibrated HBM traffic of the square GEMV from four rocprofv3 --pmc runs
    under `d`: pmc_bench_FETCH_SIZE, pmc_bench_WRITE_SIZE (--mode
    profile-square) and pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE (--mode copy,
    a 256 MiB device copy).  Each counter (KiB per dispatch) is scaled by
    (known copy bytes) / (what the counter reads for the copy)."""
    def values(sub, pred):
        rows = _csv_rows(os.path.join(d, sub), "*counter_collection.csv")
        return [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]

    copy_kib = 256 * 1024
    out = {"kernel_source_hash": kernel_source_hash(), "unit": "bytes per launch"}
    total = 0.0
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        gemm = statistics.median(values(f"pmc_bench_{ctr}", lambda n: "k_gemm" in n))
        cal = statistics.median(values(f"pmc_copy_{ctr}", lambda n: "copyBuffer" in n))
        factor = copy_kib / cal
        out[ctr] = {"gemm_kib_per_dispatch": gemm, "copy_kib_per_dispatch": cal, "factor": round(factor, 4),
                    "calibrated_bytes": round(gemm * factor * 1024)}
        total += gemm * factor * 1024
    out["bytes_per_launch"] = round(total)
    out["algorithmic_bytes_per_launch"] = weight_bytes(5120, 5120)
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


TRAFFIC_CONFIGS_FILE = os.path.join(PROFILES, "traffic_configs.json")


def ingest_pmc_configs(d):
    """Calibrated HBM traffic per call of each configuration from rocprofv3
    --pmc runs under `d`: pmc_<config>_FETCH_SIZE and pmc_<config>_WRITE_SIZE
    (--mode profile-config --config <config>) and the copy calibration
    pmc_copy_FETCH_SIZE / pmc_copy_WRITE_SIZE (--mode copy).  Writes
    traffic_configs.json: per configuration the calibrated bytes per call, the
    algorithmic bytes and their ratio."""
    def values(sub, pred):
        rows = _csv_rows(os.path.join(d, sub), "*counter_collection.csv")
        return [float(r["Counter_Value"]) for r in rows if pred(r["Kernel_Name"])]

    copy_kib = 256 * 1024
    factor = {ctr: copy_kib / statistics.median(values(f"pmc_copy_{ctr}", lambda n: "copyBuffer" in n))
              for ctr in ("FETCH_SIZE", "WRITE_SIZE")}
    algo = {"square": weight_bytes(5120, 5120), "gate_up": 2 * weight_bytes(17408, 5120),
            "down": weight_bytes(5120, 17408)}
    out = {"kernel_source_hash": kernel_source_hash(), "unit": "bytes per call",
           "copy_factor": {k: round(v, 4) for k, v in factor.items()}, "configs": {}}
    for name in PROFILE_CONFIGS:
        if not os.path.isdir(os.path.join(d, f"pmc_{name}_FETCH_SIZE")):
            continue
        rec = {}
        total = 0.0
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            kib = statistics.median(values(f"pmc_{name}_{ctr}", lambda n: "k_gemm" in n))
            rec[ctr + "_kib_per_dispatch"] = kib
            total += kib * factor[ctr] * 1024
        a = algo[name.rsplit("_M", 1)[0]]
        rec.update(bytes_per_call=round(total), algorithmic_bytes_per_call=a, ratio=round(total / a, 4))
        out["configs"][name] = rec
    os.makedirs(PROFILES, exist_ok=True)
    with open(TRAFFIC_CONFIGS_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def ingest_trace(d):
    """Per-dispatch durations of the matmul kernels from a rocprofv3
    --kernel-trace run of --mode profile-square (there every dispatch of the
    square GEMV's kernel is a graph-replayed call: warm-up and timed replays)."""
    rows = _csv_rows(d, "*kernel_trace.csv")
    dur = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "k_gemm" in name:
            dur.setdefault(name, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = {}
    for name, v in dur.items():
        v = np.array(v, dtype=np.float64)
        out[name] = {"dispatches": int(v.size), "mean_ns": round(float(v.mean()), 1),
                     "median_ns": round(float(np.median(v)), 1), "p10_ns": round(float(np.percentile(v, 10)), 1),
                     "p90_ns": round(float(np.percentile(v, 90)), 1),
                     "gbs_at_mean": round(weight_bytes(5120, 5120) / (v.mean() * 1e-9) / 1e9, 1)}
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--extra", action="store_true",
                    help="also time the down projection at M = 2, 4, 8, 16, 32 and the MLP block")
    ap.add_argument("--tower", action="store_true",
                    help="(the default) time the full-tower decode sweep (64 layers + head, 14.1 GB, "
                         "M = 1 and 7)")
    ap.add_argument("--no-tower", action="store_true", help="skip the full-tower decode sweep")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the achievable-read-bandwidth calibration")
    ap.add_argument("--no-configs", action="store_true",
                    help="only the default workload (no square M=7, gate/up, down)")
    ap.add_argument("--mode", choices=["bench", "profile-square", "profile-config", "copy", "ingest-pmc",
                                       "ingest-pmc-configs", "ingest-trace"],
                    default="bench",
                    help="profile-square: only the default workload's graph replays (for rocprofv3); "
                         "profile-config: only --config's graph replays; copy: the PMC calibration copy; "
                         "ingest-*: summarise rocprofv3 outputs under --prof-dir")
    ap.add_argument("--config", choices=PROFILE_CONFIGS, default="square_M1")
    ap.add_argument("--prof-dir", default=None)
    args = ap.parse_args()
    if args.mode == "ingest-pmc":
        ingest_pmc(args.prof_dir)
        return
    if args.mode == "ingest-pmc-configs":
        ingest_pmc_configs(args.prof_dir)
        return
    if args.mode == "ingest-trace":
        ingest_trace(args.prof_dir)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(sharding is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    w4.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.mode == "copy":
        copy_calibration(dev)
        return
    if args.mode == "profile-config":
        profile_config(args, dev, stream)
        return
    if args.mode == "profile-square":
        profile_square(args, dev, stream)
        return
    sq = square_setup(dev)
    r = bench_square(args, dev, stream, sq)
    bpc = weight_bytes(sq["N"], sq["K"])
    gbs = bpc / r["per_call"] / 1e9
    win_us = [p / sq["copies"] * 1e6 for p in r["per_window"]]
    log(f"[bench] square M=1 (graph replay): {r['per_call']*1e6:.3f} us/call, {gbs:.1f} GB/s; "
        f"windows {[round(u, 3) for u in win_us]}")
    configs = None if args.no_configs else bench_configs(dev, stream, sq, extra=args.extra)
    cal = None if args.no_calibration else calibration(dev, stream)
    if cal is not None:
        cal["value_frac_of_stream"] = round(gbs / cal["stream_4gib_gbs"], 4)
        cal["value_frac_of_call_sized"] = round(cal["call_sized"]["square"]["us_per_call"] / (r["per_call"] * 1e6), 4)
        log(f"[bench] calibration: {cal}")
        # each configuration against a plain read of its call size: time of
        # that read / time of the call
        for name, rec in (configs or {}).items():
            kind = next((k for k in cal["call_sized"] if name.startswith(k + "_M")), None)
            if kind is not None and "us_per_call" in rec:
                rec["frac_of_call_sized_read"] = round(cal["call_sized"][kind]["us_per_call"] / rec["us_per_call"], 4)
    tower = None if args.no_tower else bench_tower(dev, stream)
    del sq
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    if tower is not None and not args.no_cpu_baseline:
        tower["cpu_baseline"] = cpu_baseline_tower()
    line = {
        "metric": "effective weight GB/s (NVFP4 codes + E4M3 scales + g per call / time per call), W4A16 GEMV",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["total"] * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4(e2m1+e4m3) x bf16 -> fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights NVFP4-encoded, N(0,1) bf16 activations)",
        "config": {"workload": "square projection GEMV, K=5120 N=5120 M=1, 64 byte-identical "
                               "weight copies (943.7 MB) cycled per call; one step = the 64 calls "
                               "captured in one HIP graph and replayed",
                   "K": 5120, "N": 5120, "M": 1, "copies": 64, "calls_timed": r["calls"],
                   "us_per_call": round(r["per_call"] * 1e6, 3),
                   "us_per_call_windows_median": round(statistics.median(win_us), 3),
                   "us_per_call_windows_min": round(min(win_us), 3), "windows": len(win_us)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic()},
        "cpu_baseline": cpu,
        # the metric's operating points on the configurations that define them
        # (M = 1 decode, M = 7 verify block): µs per call, GB/s and fraction of
        # the HBM peak, median and minimum of 5 timed windows
        "configs": configs,
        # achievable read rates on this box: `value` against them is "% of achievable"
        "calibration": cal,
    }
    if tower is not None:
        line["tower"] = tower
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
