"""Benchmark: NVFP4 W4A16 matmul on one MI355X.

Default workload (one JSON line on stdout): the square projection, K = N =
5120, M = 1, with 64 byte-identical NVFP4 weight copies (943.7 MB, past the
256 MB Infinity Cache) cycled call after call.  One step = one pass over the
64 copies (64 calls).  Metric: effective weight GB/s = (N*K/2 codes + N*K/16
scales + 4 B g) per call / time per call, plus % of the 8 TB/s HBM peak.
The same line also reports the same workload at M = 7 (a speculative-verify
block) under "square_M7"; `value` is the M = 1 figure.

`--extra` also times the fused gate/up (M = 1, 7) and down (M = 1, 2, 4, 7,
8) configurations and the whole MLP block (gate/up + SwiGLU + down, one
persistent launch vs two launches, M = 1, 7), and `--tower` the full-tower
decode sweep (64 layers of the MLP block and q/k/v/o plus the 248320-wide
head, one HIP graph replay per token, M = 1 and 7); both report under "extra"
in the same line.

The timed region brackets the calls with HIP events recorded on the stream
the kernels run on; inputs are resident in HBM before timing starts.
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

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_square_m1.json")


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


def time_calls(fns, cycles, warmup_cycles, stream):
    """Run every fn in `fns` once per cycle; return seconds per call (events)."""
    import torch
    for _ in range(warmup_cycles):
        for f in fns:
            f()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(cycles):
        for f in fns:
            f()
    end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / (cycles * len(fns))


def bench_square(args, dev, stream):
    """Square GEMV: one step = one call per weight copy (64 calls), captured
    once in a HIP graph and replayed; also times the same calls launched
    eagerly from Python for reference."""
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
    bpc = weight_bytes(N, K)

    def step(strm):
        for i in range(copies):
            w4.gemm(wqs[i], wss[i], gs[i], x, y=y, workspace=work, stream=strm)

    # eager reference (Python launches each call)
    step(stream)
    torch.cuda.synchronize()
    t_eager = time_calls([lambda: step(stream)], 3, 1, stream) / copies

    # capture one step, replay `warmup` untimed and exactly `steps` timed
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        step(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=cap):
        step(cap)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(args.steps):
            graph.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    calls = args.steps * copies
    per_call = ms * 1e-3 / calls
    # the same calls for a speculative-verify block (M = 7: K_spec = 6 drafts
    # + 1), each weight read once for all rows; timed like the extra configs
    M7 = 7
    x7 = to_dev_bf16(synth.activations(c["seed_x"], M7, K), dev)
    y7 = torch.empty((M7, N), dtype=torch.bfloat16, device=dev)
    work7 = w4.new_workspace(M7, N, K, dev)
    t7 = graph_time([lambda s, i=i: w4.gemm(wqs[i], wss[i], gs[i], x7, y=y7, workspace=work7, stream=s)
                     for i in range(copies)], 10, stream)
    return dict(N=N, K=K, copies=copies, calls=calls, ms=ms, wall=wall, per_call=per_call,
                bytes_per_call=bpc, gbs=bpc / per_call / 1e9, eager_per_call=t_eager,
                eager_gbs=bpc / t_eager / 1e9, m7_per_call=t7, m7_gbs=bpc / t7 / 1e9)


def graph_time(fns, cycles, stream):
    """Seconds per call of fns, captured once in a HIP graph (one call each)
    and replayed `cycles` times after at least 50 ms of untimed replays."""
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
    # untimed replays for at least 50 ms, so that the first configuration timed
    # after the host-side weight generation runs at steady clocks
    t_warm = time.perf_counter()
    while True:
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t_warm >= 0.05:
            break
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        start.record(stream)
        for _ in range(cycles):
            graph.replay()
        end.record(stream)
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e-3 / (cycles * len(fns))


def bench_extra(dev, stream, cycles=10):
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    out = {}
    c = synth.CONFIGS["gate_up"]
    N, K, copies = c["N"], c["K"], c["copies"]
    log(f"[bench] generating gate_up K={K} N={N} x{copies}")
    wg = synth.nvfp4_weights(c["seed_gate"], N, K)
    wu = synth.nvfp4_weights(c["seed_up"], N, K)
    G = [replicate(to_dev_u8(wg[0], dev), copies), replicate(to_dev_u8(wg[1], dev), copies),
         replicate(torch.tensor([wg[2]], device=dev), copies)]
    U = [replicate(to_dev_u8(wu[0], dev), copies), replicate(to_dev_u8(wu[1], dev), copies),
         replicate(torch.tensor([wu[2]], device=dev), copies)]
    for M in c["Ms"]:
        x = to_dev_bf16(synth.activations(c["seed_x"], M, K), dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        work = w4.new_workspace(M, N, K, dev, fused=True)
        fns = [lambda s, i=i: w4.gemm_gate_up_swiglu(G[0][i], G[1][i], G[2][i], U[0][i], U[1][i],
                                                     U[2][i], x, y=y, workspace=work, stream=s)
               for i in range(copies)]
        t = graph_time(fns, cycles, stream)
        b = 2 * weight_bytes(N, K)
        out[f"gate_up_M{M}"] = dict(us_per_call=t * 1e6, gbs=b / t / 1e9, pct_peak=100 * b / t / 1e9 / HBM_PEAK_GBS)
        log(f"[bench] gate_up M={M}: {t*1e6:.2f} us/call, {b/t/1e9:.0f} GB/s")
    c = synth.CONFIGS["down"]
    N, K, copies = c["N"], c["K"], c["copies"]
    log(f"[bench] generating down K={K} N={N} x{copies}")
    wd = synth.nvfp4_weights(c["seed_w"], N, K)
    D = [replicate(to_dev_u8(wd[0], dev), copies), replicate(to_dev_u8(wd[1], dev), copies),
         replicate(torch.tensor([wd[2]], device=dev), copies)]
    for M in c["Ms"]:
        x = to_dev_bf16(synth.swiglu_activations(c["seed_a"], c["seed_b"], M, K), dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        work = w4.new_workspace(M, N, K, dev)
        fns = [lambda s, i=i: w4.gemm(D[0][i], D[1][i], D[2][i], x, y=y, workspace=work, stream=s)
               for i in range(copies)]
        t = graph_time(fns, cycles, stream)
        b = weight_bytes(N, K)
        out[f"down_M{M}"] = dict(us_per_call=t * 1e6, gbs=b / t / 1e9, pct_peak=100 * b / t / 1e9 / HBM_PEAK_GBS)
        log(f"[bench] down M={M}: {t*1e6:.2f} us/call, {b/t/1e9:.0f} GB/s")
    # the whole MLP block (gate/up + SwiGLU + down) per call: one persistent
    # launch (forced under capture), and the same calls in two launches (what
    # a captured call takes by default)
    H, F = N, K          # the down projection's output and input widths
    nb = min(len(G[0]), len(D[0]))
    for M in (1, 7):
        x = to_dev_bf16(synth.activations(synth.CONFIGS["gate_up"]["seed_x"], M, H), dev)
        y = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        work = w4.new_workspace_mlp(M, H, F, dev)
        fns = [lambda s, i=i: w4.mlp_swiglu((G[0][i], G[1][i], G[2][i]), (U[0][i], U[1][i], U[2][i]),
                                            (D[0][i], D[1][i], D[2][i]), x, y=y, workspace=work, stream=s)
               for i in range(nb)]
        b = 2 * weight_bytes(F, H) + weight_bytes(H, F)
        # captured calls take two launches; the one-launch (cooperative) path
        # runs only for eager calls, so both are also timed eagerly
        res = {"one_launch_possible": w4.mlp_one_launch(M, H, F)}
        t = graph_time(fns, cycles, stream)
        res["two_launches_graph"] = dict(us_per_call=t * 1e6, gbs=b / t / 1e9,
                                         pct_peak=100 * b / t / 1e9 / HBM_PEAK_GBS)
        log(f"[bench] mlp block M={M} (two launches, graph): {t*1e6:.2f} us/call, {b/t/1e9:.0f} GB/s")
        for one, name in ((True, "one_launch_eager"), (False, "two_launches_eager")):
            efns = [lambda i=i: w4.mlp_swiglu((G[0][i], G[1][i], G[2][i]), (U[0][i], U[1][i], U[2][i]),
                                              (D[0][i], D[1][i], D[2][i]), x, y=y, workspace=work,
                                              stream=stream, one_launch=one)
                    for i in range(nb)]
            t = time_calls(efns, cycles, 2, stream)
            res[name] = dict(us_per_call=t * 1e6, gbs=b / t / 1e9, pct_peak=100 * b / t / 1e9 / HBM_PEAK_GBS)
            log(f"[bench] mlp block M={M} ({name}): {t*1e6:.2f} us/call, {b/t/1e9:.0f} GB/s")
        out[f"mlp_M{M}"] = res
    del G, U, D
    return out


def bench_tower(dev, stream, Ms=(1, 7), layers=64, replays=5):
    """Full-tower decode sweep, one token = one HIP graph replay of
    `layers` x (the MLP block: gate/up + SwiGLU 5120 -> 2 x 17408 and down
    17408 -> 5120 through w4a16_mlp_swiglu, which takes two launches under
    capture; q, k, v, o 5120 -> 5120) followed by the 5120 -> 248320 head GEMV
    with fused greedy argmax (the head alone is also timed with and without
    it): 385 launches and 14.1 GB of distinct weight allocations per token.
    The MLP
    chain is wired (SwiGLU output feeds down, down's output feeds the next
    layer's gate/up); q/k/v/o and the head read fixed synthetic activations
    (there is no attention).  Weights per layer are byte-identical replicas of
    one encoded matrix per kind; the head matrix tiles the rows of the square
    matrix (48.5 copies of its 5120 rows), since HBM traffic depends on the
    addresses read, not on the values."""
    import torch
    import block_scaled_fp4_w4a16_amd as w4
    import synth
    H, F, V = 5120, 17408, 248320
    cg, cd, cs = synth.CONFIGS["gate_up"], synth.CONFIGS["down"], synth.CONFIGS["square"]
    log(f"[bench] tower: encoding gate/up/down/square, {layers} layers + head")
    enc = {
        "gate": synth.nvfp4_weights(cg["seed_gate"], F, H),
        "up": synth.nvfp4_weights(cg["seed_up"], F, H),
        "down": synth.nvfp4_weights(cd["seed_w"], H, F),
        "sq": synth.nvfp4_weights(cs["seed_w"], H, H),
    }
    dev_enc = {k: (to_dev_u8(v[0], dev), to_dev_u8(v[1], dev),
                   torch.tensor([v[2]], dtype=torch.float32, device=dev)) for k, v in enc.items()}

    def copies(kind, n):
        return [tuple(t.clone() for t in dev_enc[kind]) for _ in range(n)]
    L = {"gate": copies("gate", layers), "up": copies("up", layers), "down": copies("down", layers),
         "q": copies("sq", layers), "k": copies("sq", layers), "v": copies("sq", layers),
         "o": copies("sq", layers)}
    reps = (V + H - 1) // H
    head = (torch.cat([dev_enc["sq"][0]] * reps)[:V].contiguous(),
            torch.cat([dev_enc["sq"][1]] * reps)[:V].contiguous(), dev_enc["sq"][2].clone())
    del dev_enc
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
            # greedy decoding: the head's argmax, without materialising logits
            w4.gemm_argmax(head[0], head[1], head[2], x, idx=tok_idx, val=tok_val, workspace=wk_hd,
                           stream=s)

        t = graph_time([token], replays, stream)
        t_head = graph_time([lambda s: w4.gemm(head[0], head[1], head[2], x0, y=logits, workspace=wk_hd0,
                                               stream=s)] * 8, replays, stream)
        t_head_am = graph_time([lambda s: w4.gemm_argmax(head[0], head[1], head[2], x0, idx=tok_idx, val=tok_val,
                                                         workspace=wk_hd, stream=s)] * 8, replays, stream)
        bh = weight_bytes(V, H)
        out[f"head_M{M}"] = dict(us_per_call=t_head * 1e6, gbs=bh / t_head / 1e9,
                                 argmax_us_per_call=t_head_am * 1e6, argmax_gbs=bh / t_head_am / 1e9)
        log(f"[bench] head 5120->{V} M={M}: logits {t_head*1e6:.1f} us ({bh/t_head/1e9:.0f} GB/s), "
            f"fused argmax {t_head_am*1e6:.1f} us ({bh/t_head_am/1e9:.0f} GB/s)")
        per_layer = 6  # captured MLP blocks run as two launches (gate/up, down)
        out[f"tower_M{M}"] = dict(ms_per_token=t * 1e3, tokens_per_s=1.0 / t,
                                  launches_per_token=per_layer * layers + 1,
                                  head="fused greedy argmax",
                                  bytes_per_token=b_token, gbs=b_token / t / 1e9,
                                  pct_peak=100 * b_token / t / 1e9 / HBM_PEAK_GBS)
        log(f"[bench] tower M={M}: {t*1e3:.3f} ms/token ({1/t:.1f} tok/s), {b_token/t/1e9:.0f} GB/s "
            f"over {b_token/1e9:.2f} GB")
    return out


def calibration(dev, stream, copies, call_bytes=5120 * 5120 // 2 + 5120 * 5120 // 16):
    """Achievable HBM read rates, from a plain 128-bit non-temporal streaming
    read (libw4a16_calib.so, not the matmul library): once on a 4 GiB buffer
    (32 workgroups of 1024 threads per CU: the fastest launch shape of a sweep
    on MI355X, 6.6-7.0 TB/s), and over `copies` buffers of one
    square call's weight bytes cycled like the weight copies, with the GEMV's
    grid (one workgroup of 512 threads per CU), in a HIP graph like the
    benchmark.  The second rate includes the same per-call fixed costs."""
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
    t_big = graph_time([lambda s: read(big, big_bytes, 32 * cus, 1024, s)], 10, stream)
    del big
    bufs = [torch.ones(call_bytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
    t_call = graph_time([lambda s, i=i: read(bufs[i], call_bytes, cus, 512, s) for i in range(copies)], 10, stream)
    del bufs
    return {"kind": "plain 128-bit non-temporal streaming read (libw4a16_calib.so)",
            "stream_4gib_gbs": round(big_bytes / t_big / 1e9, 1),
            "call_sized_bytes": call_bytes, "call_sized_copies": copies,
            "call_sized_us_per_call": round(t_call * 1e6, 3),
            "call_sized_gbs": round(call_bytes / t_call / 1e9, 1)}


def cpu_baseline(seconds_target=12.0):
    """The CPU oracle timed on a bounded sample of the square workload."""
    import oracle
    import synth
    c = synth.CONFIGS["square"]
    N, K = c["N"], c["K"]
    wq, ws, g = synth.nvfp4_weights(c["seed_w"], N, K)
    x = synth.activations(c["seed_x"], 1, K)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.gemm(wq, ws, g, x, 1, N, K, nthreads=threads)
    one = time.perf_counter() - t0
    reps = max(1, min(64, int(seconds_target / max(one, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.gemm(wq, ws, g, x, 1, N, K, nthreads=threads)
    dt = (time.perf_counter() - t0) / reps
    return dict(value=weight_bytes(N, K) / dt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{reps} calls of the square GEMV (M=1, K=N=5120) by the fp64 C oracle "
                       f"with {threads} OpenMP threads; {dt*1e3:.1f} ms/call")


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


def ingest_pmc(d):
    """Calibrated HBM traffic of the square GEMV from four rocprofv3 --pmc runs
    under `d`: pmc_bench_FETCH_SIZE, pmc_bench_WRITE_SIZE (this script's default
    workload) and pmc_copy_FETCH_SIZE, pmc_copy_WRITE_SIZE (--mode copy, a
    256 MiB device copy).  Each counter (KiB per dispatch) is scaled by
    (known copy bytes) / (what the counter reads for the copy)."""
    import csv
    import glob
    import statistics

    def values(sub, pred):
        f = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)[0]
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(f)) if pred(r["Kernel_Name"])]

    copy_kib = 256 * 1024
    out = {"kernel_source_hash": kernel_source_hash(), "unit": "bytes per launch"}
    total = 0.0
    for ctr, copy_pred in (("FETCH_SIZE", lambda n: "copyBuffer" in n),
                           ("WRITE_SIZE", lambda n: "copyBuffer" in n)):
        # the square GEMV at M = 1 (the run also has the M = 7 calls, on the MFMA kernel)
        gemm = statistics.median(values(f"pmc_bench_{ctr}", lambda n: "k_gemm_valu" in n))
        cal = statistics.median(values(f"pmc_copy_{ctr}", copy_pred))
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--extra", action="store_true", help="also time the gate/up and down configs")
    ap.add_argument("--tower", action="store_true",
                    help="also time the full-tower decode sweep (64 layers + head, 14.1 GB, M = 1 and 7)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the achievable-read-bandwidth calibration")
    ap.add_argument("--mode", choices=["bench", "copy", "ingest-pmc"], default="bench",
                    help="copy: run only the PMC calibration copy kernel; ingest-pmc: turn rocprofv3 "
                         "FETCH_SIZE/WRITE_SIZE outputs (--pmc-dir) into profiles/traffic_square_m1.json")
    ap.add_argument("--pmc-dir", default=None)
    args = ap.parse_args()
    if args.mode == "ingest-pmc":
        ingest_pmc(args.pmc_dir)
        return
    if args.mode == "copy":
        import torch
        copy_calibration(torch.device("cuda:0"))
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
    r = bench_square(args, dev, stream)
    log(f"[bench] square (graph replay): {r['per_call']*1e6:.3f} us/call, {r['gbs']:.1f} GB/s; "
        f"eager: {r['eager_per_call']*1e6:.3f} us/call, {r['eager_gbs']:.1f} GB/s; "
        f"M=7: {r['m7_per_call']*1e6:.3f} us/call, {r['m7_gbs']:.1f} GB/s")
    cal = None if args.no_calibration else calibration(dev, stream, r["copies"])
    if cal is not None:
        cal["value_frac_of_stream"] = round(r["gbs"] / cal["stream_4gib_gbs"], 4)
        cal["value_frac_of_call_sized"] = round(r["gbs"] / cal["call_sized_gbs"], 4)
        log(f"[bench] calibration: streaming read {cal['stream_4gib_gbs']} GB/s (4 GiB), "
            f"{cal['call_sized_gbs']} GB/s ({cal['call_sized_us_per_call']} us per 14.7 MB call)")
    extra = bench_extra(dev, stream) if args.extra else None
    if args.tower:
        extra = dict(extra or {}, **bench_tower(dev, stream))
    cpu = None if args.no_cpu_baseline else cpu_baseline()
    line = {
        "metric": "effective weight GB/s (NVFP4 codes + E4M3 scales + g per call / time per call), W4A16 GEMV",
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"] / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4(e2m1+e4m3) x bf16 -> fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights NVFP4-encoded, N(0,1) bf16 activations)",
        "config": {"workload": "square projection GEMV, K=5120 N=5120 M=1, 64 byte-identical "
                               "weight copies (943.7 MB) cycled per call; one step = the 64 calls "
                               "captured in one HIP graph and replayed",
                   "K": r["K"], "N": r["N"], "M": 1, "copies": r["copies"], "calls_timed": r["calls"],
                   "us_per_call": round(r["per_call"] * 1e6, 3),
                   "eager_us_per_call": round(r["eager_per_call"] * 1e6, 3),
                   "eager_gbs": round(r["eager_gbs"], 1)},
        "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), "traffic": stored_traffic()},
        "cpu_baseline": cpu,
        # the metric's second operating point: the same workload for a verify
        # block of M = 7 activation rows (not the `value`)
        "square_M7": {"us_per_call": round(r["m7_per_call"] * 1e6, 3), "gbs": round(r["m7_gbs"], 2),
                      "frac": round(r["m7_gbs"] / HBM_PEAK_GBS, 4), "calls_timed": 10 * r["copies"]},
        # achievable read rates on this box: `value` against them is "% of achievable"
        "calibration": cal,
    }
    if extra is not None:
        line["extra"] = extra
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
