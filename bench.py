"""Benchmark of the varlen chunkwise gated-delta-rule prefill forward on one MI355X.

One step = the whole hot path over one batch: device chunk metadata (built
from cu_seqlens inside the map kernel's prologue for up to 64 sequences, by
build_chunk_meta's kernel beyond), the chunk-parallel map and the sequential
reduce + output, captured once in a HIP graph and replayed (the fixed-capacity graph-replay mode
of the FLA graph-capture RFC, section "Performance evaluation").  Inputs are
seeded synthetic tensors already resident in HBM.

Prints ONE JSON line.  ``value`` is tokens/s of graph replays; ``roofline``
describes the dominant kernel (average duration measured live with HIP events
on the launch stream); ``cpu_baseline`` is the fp64 oracle timed on this
host's cores.  ``--gpus N`` with N > 1 exits: this build runs on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published

WORKLOADS = {
    "c1": (1, None, "GDN varlen prefill: bf16 q/k/v, fp32 g/beta/state, H=16, d_k=d_v=128, "
                    "BT=64, T=8192 cut into 8 sequences by 7 uniform cut points, "
                    "h0~N(0,0.1), seed 1"),
    "c2": (2, None, "KDA: bf16, one sequence T=4096, H=16, d_k=d_v=128, BT=64, zero state, seed 2"),
    "c4g": (4, False, "GDN: bf16, one sequence T=65536, H=10, d=128, BT=64, zero state, seed 4"),
    "c4k": (4, True, "KDA: bf16, one sequence T=65536, H=10, d=128, BT=64, zero state, seed 4"),
    "c4g_short": (4, False, "GDN: bf16, one sequence T=2048, H=10, d=128, zero state, seed 4"),
    "c4k_short": (4, True, "KDA: bf16, one sequence T=2048, H=10, d=128, zero state, seed 4"),
    "c3": (3, None, "fixed-capacity bucket: T_max=16384, N_max=64, GDN bf16, H=32, d=128, "
                    "no initial state; one graph capture, replays over fresh layouts "
                    "(N ~ U{1..64}, Dirichlet lengths), seeds 3000+r"),
    "dec": (None, False, "GDN decode step: 64 sequences x 1 token, bf16 q/k/v, H=16, "
                         "d_k=d_v=128, fp32 state N(0,0.1) updated in place, seed 5"),
    "deck": (None, True, "KDA decode step: 64 sequences x 1 token, bf16 q/k/v, H=16, "
                         "d_k=d_v=128, fp32 state N(0,0.1) updated in place, seed 5"),
    "bwd": (1, None, "GDN chunk backward on the 8K varlen workload: bf16 q/k/v, fp32 g/beta, "
                     "H=16, d_k=d_v=128, h0~N(0,0.1), dout~N(0,1) fp32, no dht, seed 1"),
    "bwdk": (2, True, "KDA chunk backward on the 4K KDA workload: bf16 q/k/v, bf16-valued "
                      "g/beta, one sequence T=4096, H=16, d_k=d_v=128, zero state, "
                      "dout~N(0,1) fp32, no dht, seed 2"),
    "conv": (None, None, "varlen causal short convolution: bf16 x [8192, 6144] (q, k, v "
                         "projections of H=16, d=128) in the 8 sequences of the 8K varlen "
                         "layout, W=4, bias, SiLU, bf16 states N(0,1) updated in place, "
                         "BT=64 chunk metadata built once, seed 7"),
}

def kernel_source_hash(files):
    """Hash of the shared device headers plus ``files`` (a name or a list)."""
    h = hashlib.sha256()
    files = [files] if isinstance(files, str) else list(files)
    for f in ["la_device.h", "kernels.h"] + files:
        with open(os.path.join(ROOT, "chunkwise_gated_delta_chunk_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def alg_bytes(inp, kind):
    """Algorithmic HBM bytes of one launch.

    "op": the whole forward, T*H*[(2 d_k + d_v) s_qkv + s_g + 4 + 4 d_v] plus
    4 d_k d_v per (non-empty sequence, head) for each of h0 / ht.  This is the
    figure the headline roofline divides by the step time.
    Per kernel (diagnostics), the part of those bytes a kernel has to touch
    itself: the map reads q, k, g and beta; the reduce reads v (and h0) and
    writes o (and ht), and with 16-bit GDN inputs it reads the q and k rows
    too -- it takes the chunk matrices (and otherwise the staged keys and
    queries) from the map's workspace images, which are implementation
    overhead and not counted."""
    T = int(inp["cu_seqlens"][-1])
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    s_qkv = 2 if inp["dtype"] == "bf16" else 4
    s_g = 4 * dk if inp["kda"] else 4
    lens = np.diff(inp["cu_seqlens"].astype(np.int64))
    nonempty = int((lens > 0).sum())
    state = nonempty * H * dk * dv * 4 * ((inp["h0"] is not None) + 1)
    if kind == "op":
        return T * H * ((2 * dk + dv) * s_qkv + s_g + 4 + 4 * dv) + state
    if kind == "map":
        return T * H * (2 * dk * s_qkv + s_g + 4)
    if kind == "reduce":
        qk = 2 * dk * s_qkv if (s_qkv == 2 and not inp["kda"]) else 0
        return T * H * (qk + dv * s_qkv + 4 * dv) + state
    raise ValueError(kind)


def alg_flops(inp):
    """Dense chunk GEMM flops + 2/3 C^3 for the inverse, per chunk-head (C=64)."""
    lens = np.diff(inp["cu_seqlens"].astype(np.int64))
    chunks = int((-(-lens // 64)).sum())
    C, dk, dv = 64, inp["dk"], inp["dv"]
    per = (2 * C * C * dk * 3 + 2 * C * C * dv + 3 * 2 * C * dk * dv + 2 * C * C * dv
           + 2 * C ** 3 / 3)
    return chunks * inp["H"] * per


def kernel_sources(kind, inp=None):
    """The source files (besides the shared headers) of a kernel kind; 16-bit
    inputs run the 32-column reduce of its own file or the general one."""
    if kind == "reduce":
        sixteen = inp is None or inp["dtype"] != "f32"
        return ["reduce_work.h"] + (["chunk_reduce16.hip"] if sixteen else []) + ["chunk_reduce.hip"]
    return [{"map": "chunk_map.hip", "recurrent": "recurrent.hip", "conv": "short_conv.hip"}[kind]]

# decode workloads: sequences (one token each), heads, head dim
DECODE_N, DECODE_H, DECODE_D = 64, 16, 128


def decode_alg_bytes(kda):
    """Algorithmic bytes of one decode step: the state read and written, q, k,
    v, g, beta and o."""
    N, H, d = DECODE_N, DECODE_H, DECODE_D
    return N * H * (2 * d * d * 4 + 3 * d * 2 + (4 * d if kda else 4) + 4 + 4 * d)


def load_traffic(kernel_kind, workload, inp=None):
    """HBM traffic of the dominant kernel from the committed counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_src_sha") != kernel_source_hash(kernel_sources(kernel_kind, inp)):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s=12.0):
    """Time the fp64 oracle (as it stands) on this host: whole workload, repeated
    until ~budget_s of wall time or 3 runs."""
    from oracle import recurrence
    T = int(inp["cu_seqlens"][-1])
    units = int((np.diff(inp["cu_seqlens"]) > 0).sum()) * inp["H"]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    omp = int(os.environ.get("OMP_NUM_THREADS", cores))
    threads = max(1, min(cores, omp, units))
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 and (time.perf_counter() - t_all) < budget_s:
        t0 = time.perf_counter()
        recurrence.gated_delta_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                   inp["cu_seqlens"], inp["h0"], kda=inp["kda"],
                                   nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": T / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({T} tokens x {inp['H']} heads), median of "
                      f"{len(times)} run(s) of the fp64 token recurrence, {threads} OpenMP "
                      f"threads of {cores} host cores"}


def bench_bucket(args, torch, la, synth, dev):
    """Fixed-capacity bucket: capture once, then for each of ``--layouts``
    fresh layouts copy cu_seqlens and inputs into the static buffers (outside
    the timed region) and time ``--steps`` replays of that layout."""
    T_max, N_max, H, d = 16384, 64, 32, 128
    bf = torch.bfloat16
    q = torch.zeros((T_max, H, d), dtype=bf, device=dev)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    g = torch.zeros((T_max, H), device=dev)
    beta = torch.zeros((T_max, H), device=dev)
    cu = torch.zeros((N_max + 1,), dtype=torch.int32, device=dev)
    NT = la.nt_max(T_max, N_max)
    ci = torch.empty((NT, 2), dtype=torch.int32, device=dev)
    co = torch.empty((N_max + 1,), dtype=torch.int32, device=dev)
    st = torch.empty((1,), dtype=torch.int32, device=dev)
    o = torch.empty((T_max, H, d), device=dev)
    ht = torch.empty((N_max, H, d, d), device=dev)
    ws = torch.empty((la.workspace_bytes(T_max, N_max, H, d, d, bf, False, seg_len=args.seg_len,
                                         dv_split=args.dv_split),),
                     dtype=torch.uint8, device=dev)
    kw = dict(o=o, ht=ht, workspace=ws, dv_split=args.dv_split, seg_len=args.seg_len)

    def fill(inp):
        for t, key in ((q, "q"), (k, "k"), (v, "v")):
            t.copy_(torch.from_numpy(inp[key]).to(bf))
        g.copy_(torch.from_numpy(inp["g"]))
        beta.copy_(torch.from_numpy(inp["beta"]))
        cu.copy_(torch.from_numpy(inp["cu_seqlens"].astype(np.int32)))

    def step():
        # the call builds the chunk layout of cu into ci / co itself
        la.gdn_chunk_fwd(q, k, v, g, beta, cu, ci, co, build_meta=True, meta_status=st, **kw)

    fill(synth.config(3, replay=0))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    tc = time.perf_counter()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    capture_ms = (time.perf_counter() - tc) * 1e3

    rows = []
    graph_eq = True
    for r in range(args.layouts):
        inp = synth.config(3, replay=r)
        fill(inp)
        tokens = int(inp["cu_seqlens"][-1])
        for _ in range(max(1, args.warmup)):
            graph.replay()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            graph.replay()
            ev[i + 1].record()
        torch.cuda.synchronize()
        t = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
        o_g, ht_g = o.clone(), ht.clone()
        step()
        torch.cuda.synchronize()
        graph_eq &= bool(torch.equal(o, o_g) and torch.equal(ht, ht_g))
        ab = alg_bytes(inp, "op")
        p50 = float(np.median(t))
        rows.append({"replay": r, "sequences": int((np.diff(inp["cu_seqlens"]) > 0).sum()),
                     "tokens": tokens, "p50_ms": round(p50, 5),
                     "p95_ms": round(float(np.percentile(t, 95)), 5),
                     "hbm_frac": round(ab / (p50 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        print(f"layout {r}: {rows[-1]}", file=sys.stderr, flush=True)
    tok = sum(x["tokens"] for x in rows)
    ms_total = sum(x["p50_ms"] for x in rows)
    fr = sorted(x["hbm_frac"] for x in rows)
    out = {
        "metric": "GDN/KDA chunk-fwd tokens/s (H=16,d=128,8K varlen); % of HBM/MFMA roofline",
        "value": round(tok / (ms_total * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_total / len(rows), 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 inputs; fp16 MFMA operands, fp32 accumulation and state",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": WORKLOADS["c3"][2],
                   "mode": "graph-replay of map (building the chunk layout) + reduce",
                   "layouts": len(rows), "nt_max": NT},
        "op_hbm_frac": {"median": fr[len(fr) // 2], "min": fr[0], "max": fr[-1]},
        "capture_ms": round(capture_ms, 3), "graph_equals_eager": graph_eq,
        "replays": rows,
    }
    print(json.dumps(out), flush=True)


CONV_T, CONV_D, CONV_W = 8192, 6144, 4


def conv_alg_bytes(N, esz=2):
    """Algorithmic bytes of one short-convolution launch: x read and y written
    once, the states read and written, weights and bias."""
    T, D, W = CONV_T, CONV_D, CONV_W
    return 2 * T * D * esz + 2 * N * (W - 1) * D * esz + D * W * 4 + D * 4


def bench_conv(args, torch, la, synth, dev):
    """One short convolution per replay over the 8K varlen layout, the states
    updated in place; HIP events around the launches on the current stream,
    then a graph of one launch replayed."""
    desc = WORKLOADS[args.workload][2]
    cu_np = synth.config(1)["cu_seqlens"]
    N = len(cu_np) - 1
    inp = synth.make_conv_inputs(CONV_T, CONV_D, CONV_W, dtype="bf16", seed=7, cu_seqlens=cu_np,
                                 h0=True)
    bf = torch.bfloat16
    x = torch.from_numpy(inp["x"]).to(dev, bf)
    w = torch.from_numpy(inp["weight"]).to(dev)
    b = torch.from_numpy(inp["bias"]).to(dev)
    state0 = torch.from_numpy(inp["h0"]).to(dev, bf)
    state = state0.clone()
    y = torch.empty_like(x)
    cu = torch.from_numpy(cu_np.astype(np.int32)).to(dev)
    ci, _, _ = la.build_chunk_meta(cu, CONV_T)

    def step():
        la.short_conv_fwd(x, w, cu, ci, bias=b, h0=state, ht=state, y=y, activation="silu")

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / args.steps
    state.copy_(state0)
    step()
    torch.cuda.synchronize()
    eager_y, eager_state = y.clone(), state.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    state.copy_(state0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    graph_eq = bool(torch.equal(y, eager_y) and torch.equal(state, eager_state))
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    ab = conv_alg_bytes(N)
    achieved = ab / (launch_ms * 1e-3) / 1e9
    # a plain device copy of x into y moves the same bytes: the practical
    # ceiling of a read-once, write-once kernel on this GPU
    y2 = torch.empty_like(x)
    for _ in range(3):
        y2.copy_(x)
    e0.record()
    for _ in range(20):
        y2.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * x.numel() * 2 / (e0.elapsed_time(e1) / 20 * 1e-3) / 1e9
    out = {
        "metric": "GDN/KDA chunk-fwd tokens/s (H=16,d=128,8K varlen); % of HBM/MFMA roofline",
        "value": round(CONV_T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 data; fp32 weights and arithmetic",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": desc, "mode": "graph-replay of one short convolution",
                   "tokens": CONV_T, "channels": CONV_D, "width": CONV_W, "sequences": N},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("conv", args.workload),
                     "kernel": "short_conv_kernel", "alg_bytes_per_launch": ab,
                     "avg_launch_ms": round(launch_ms, 5)},
        "graph_equals_eager": graph_eq,
        "copy_same_bytes_gbs": round(copy_gbs, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = conv_cpu_baseline(inp)
    print(json.dumps(out), flush=True)


def conv_cpu_baseline(inp, budget_s=12.0):
    """The fp64 short-convolution oracle on the whole workload, repeated until
    ~budget_s of wall time or 3 runs (numpy, one thread of vector work)."""
    from oracle.short_conv import short_conv_fwd
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 and (time.perf_counter() - t_all) < budget_s:
        t0 = time.perf_counter()
        short_conv_fwd(inp["x"], inp["weight"], inp["cu_seqlens"], b=inp["bias"], h0=inp["h0"],
                       activation="silu")
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    return {"value": CONV_T / t, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload ({CONV_T} tokens x {CONV_D} channels), median of "
                      f"{len(times)} run(s) of the fp64 numpy token loop"}


def bwd_alg_flops(cells, d, kda=False):
    """Algorithmic flops of the chunk backward per (chunk, head) cell, summed:
    the per-chunk products of the state-gradient pass (3 x 64 d^2 + 2 x 64^2 d
    MACs), of the dV / partial-product pass (5 x 64 d^2 + 5 x 64^2 d), of the
    final pass (4 x 64^2 d + 2 x 64^3), of the prep (2 x 64^2 d + 64^3 / 3) and
    of the forward state recompute (2 x 64 d^2 + 64^2 d + the map's 2 x 64^2 d
    + 64^3 / 3); 2 flops per MAC."""
    c = 64
    macs = (3 * c * d * d + 2 * c * c * d) + (5 * c * d * d + 5 * c * c * d) + \
        (4 * c * c * d + 2 * c ** 3) + (2 * c * c * d + c ** 3 / 3) + \
        (2 * c * d * d + c * c * d + 2 * c * c * d + c ** 3 / 3)
    # KDA: the per-channel E-weighted sums of the final pass (four sums of
    # C^2 / 2 d terms) count as the 4 x 64^2 d products they replace; the
    # decay is inside S and M, whose 2 x 64^2 d products the prep counts
    return 2 * macs * cells


def bench_bwd(args, torch, la, synth, dev):
    """One chunk backward per step (forward recompute + the backward
    launches: prep, dh and the fused per-chunk kernel for GDN; prep, dh, part
    and final for KDA) on the workload's inputs; HIP events around the calls,
    then a graph of one call replayed.  GDN's bf16 path runs on bf16 MFMA
    (operands split into bf16 high and low halves) and is priced against the
    bf16 peak; KDA's prep, part and final run on fp32 MFMA (its dh on split
    bf16) and the call is priced against the fp32 peak."""
    cfg, kda, desc = WORKLOADS[args.workload]
    kda = bool(kda)
    inp = synth.config(cfg)
    T, H, d = inp["q"].shape[0], inp["H"], inp["dk"]
    bf = torch.bfloat16
    q, k, v = (torch.from_numpy(inp[x]).to(dev, bf) for x in ("q", "k", "v"))
    g = torch.from_numpy(inp["g"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    h0 = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).to(dev)
    rng = np.random.default_rng(1)
    dout = torch.from_numpy(rng.standard_normal((T, H, d)).astype(np.float32)).to(dev)
    cu = torch.from_numpy(inp["cu_seqlens"].astype(np.int32)).to(dev)
    N = cu.numel() - 1
    ci, co, _ = la.build_chunk_meta(cu, T)
    ws = torch.empty((la.bwd_workspace_bytes(T, N, H, d, d, bf, kda=kda),), dtype=torch.uint8,
                     device=dev)
    outs = dict(dq=torch.empty((T, H, d), device=dev), dk=torch.empty((T, H, d), device=dev),
                dv=torch.empty((T, H, d), device=dev), dg=torch.empty(g.shape, device=dev),
                dbeta=torch.empty((T, H), device=dev))
    if h0 is not None:
        outs["dh0"] = torch.empty_like(h0)
    fn = la.kda_chunk_bwd if kda else la.gdn_chunk_bwd
    # the reverse pass runs beside the forward recompute on a second stream
    # (the caller's stream, fork and join events)
    aux = torch.cuda.Stream()
    evs = la.fork_join_events()

    def step():
        fn(q, k, v, g, beta, cu, ci, co, dout, h0=h0, workspace=ws, aux_stream=aux, events=evs,
           **outs)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    call_ms = e0.elapsed_time(e1) / args.steps
    eager = {key: t.clone() for key, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    graph_eq = all(torch.equal(outs[key], eager[key]) for key in outs)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    cells = int(np.ceil(np.diff(inp["cu_seqlens"]) / 64).sum()) * H
    fl = bwd_alg_flops(cells, d, kda)
    achieved = fl / (call_ms * 1e-3) / 1e12
    peak = MFMA_F32_PEAK_TFLOPS if kda else MFMA_F16_PEAK_TFLOPS
    out = {
        "metric": "GDN/KDA chunk-fwd tokens/s (H=16,d=128,8K varlen); % of HBM/MFMA roofline",
        "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16 inputs; dh on bf16 MFMA with split operands, prep/part/final on fp32 "
                  "MFMA and VALU" if kda else
                  "bf16 inputs; bf16 MFMA on split operands, fp32 accumulation"),
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": desc, "mode": "graph-replay of one backward call",
                   "tokens": T, "heads": H, "d": d, "sequences": N},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "kda_chunk_bwd (whole call: map, reduce, prep, dh, part, final)" if kda
                               else "gdn_chunk_bwd (whole call: map, reduce, prep, dh, fused part+final)",
                     "alg_flops_per_call": fl, "avg_call_ms": round(call_ms, 5)},
        "graph_equals_eager": graph_eq,
    }
    print(json.dumps(out), flush=True)


def bench_decode(args, torch, la, synth, dev):
    """One recurrent (decode) step per replay: a token for each of N sequences,
    the state updated in place; HIP events around the launch, then a graph of
    one step replayed."""
    _, kda, desc = WORKLOADS[args.workload]
    N, H, d = DECODE_N, DECODE_H, DECODE_D
    inp = synth.make_inputs(N, H, d, d, kda=kda, dtype="bf16", seed=5,
                            cu_seqlens=np.arange(N + 1, dtype=np.int32), h0_std=0.1)
    bf = torch.bfloat16
    q, k, v = (torch.from_numpy(inp[x]).to(dev, bf) for x in ("q", "k", "v"))
    g = torch.from_numpy(inp["g"]).to(dev)
    beta = torch.from_numpy(inp["beta"]).to(dev)
    state0 = torch.from_numpy(inp["h0"]).to(dev)
    state = state0.clone()
    o = torch.empty((N, H, d), device=dev)
    fwd = la.kda_recurrent_fwd if kda else la.gdn_recurrent_fwd

    def step():
        fwd(q, k, v, g, beta, h0=state, ht=state, o=o)

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    launch_ms = e0.elapsed_time(e1) / args.steps
    # eager reference step from a known state
    state.copy_(state0)
    step()
    torch.cuda.synchronize()
    eager_o, eager_state = o.clone(), state.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    state.copy_(state0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    graph_eq = bool(torch.equal(o, eager_o) and torch.equal(state, eager_state))
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    ab = decode_alg_bytes(kda)
    achieved = ab / (launch_ms * 1e-3) / 1e9
    out = {
        "metric": "GDN/KDA chunk-fwd tokens/s (H=16,d=128,8K varlen); % of HBM/MFMA roofline",
        "value": round(N * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 inputs; fp32 state and arithmetic",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": desc, "mode": "graph-replay of one recurrent step",
                   "sequences": N, "heads": H, "d": d},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": load_traffic("recurrent", args.workload),
                     "kernel": "recurrent_kernel", "alg_bytes_per_launch": ab,
                     "avg_launch_ms": round(launch_ms, 5)},
        "graph_equals_eager": graph_eq,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


def env_record(torch):
    """Versions and device of this run (the RFC's CI plan records them)."""
    props = torch.cuda.get_device_properties(0)
    rocm = None
    if os.path.exists("/opt/rocm/.info/version"):
        rocm = open("/opt/rocm/.info/version").read().strip()
    return {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
            "rocm": rocm, "gfx_arch": getattr(props, "gcnArchName", None),
            "device": props.name, "compute_units": props.multi_processor_count}


class FwdBucket:
    """Static device buffers of one fixed-capacity bucket (T_max, N_max) of a
    forward workload, and the step on them: the chunk forward, which builds
    the chunk layout of cu_seqlens into ci / co itself (in the map kernel up
    to 64 sequences, else with the metadata kernel first) (the FLA
    graph-capture RFC, "Static buffer contract" and "Device-side metadata")."""

    def __init__(self, torch, la, inp, T_max, N_max, dev, dv_split=0, seg_len=0):
        self.torch, self.la = torch, la
        H, dk, dv = inp["H"], inp["dk"], inp["dv"]
        tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
        self.kda = bool(inp["kda"])
        z = lambda shape, dt=torch.float32: torch.zeros(shape, dtype=dt, device=dev)  # noqa: E731
        self.q, self.k, self.v = (z((T_max, H, dk), tdt) for _ in range(3))
        self.g = z((T_max, H, dk) if self.kda else (T_max, H))
        self.beta = z((T_max, H))
        self.cu = z((N_max + 1,), torch.int32)
        self.has_h0 = inp["h0"] is not None
        self.h0 = z((N_max, H, dk, dv)) if self.has_h0 else None
        NT = la.nt_max(T_max, N_max)
        self.ci = z((NT, 2), torch.int32)
        self.co = z((N_max + 1,), torch.int32)
        self.st = z((1,), torch.int32)
        self.o = z((T_max, H, dv))
        self.ht = z((N_max, H, dk, dv))
        self.ws = torch.empty((la.workspace_bytes(T_max, N_max, H, dk, dv, tdt, self.kda,
                                                  seg_len=seg_len, dv_split=dv_split),),
                              dtype=torch.uint8, device=dev)
        self.kw = dict(h0=self.h0, o=self.o, ht=self.ht, workspace=self.ws, dv_split=dv_split,
                       seg_len=seg_len)
        self.T_max, self.N_max, self.NT = T_max, N_max, NT
        self.split = la.dv_split_for(T_max, N_max, H, dk, dv, tdt, dv_split, seg_len=seg_len)
        self.seg = la.seg_len_for(T_max, N_max, H, dk, dv, tdt, seg_len=seg_len)
        self.fwd = la.kda_chunk_fwd if self.kda else la.gdn_chunk_fwd
        self.graph = None

    def load(self, src, cu_host):
        """Write one layout into the static buffers: device inputs ``src`` (the
        rows of real tokens) and cu_seqlens from pinned host memory."""
        T = int(cu_host[-1])
        for name in ("q", "k", "v", "g", "beta"):
            getattr(self, name)[:T].copy_(src[name][:T], non_blocking=True)
        if self.has_h0:
            n = src["h0"].shape[0]
            self.h0[:n].copy_(src["h0"], non_blocking=True)
        self.cu.copy_(cu_host, non_blocking=True)

    def step(self):
        self.fwd(self.q, self.k, self.v, self.g, self.beta, self.cu, self.ci, self.co,
                 build_meta=True, meta_status=self.st, **self.kw)

    def capture(self):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        tc = time.perf_counter()
        with torch.cuda.graph(self.graph):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - tc) * 1e3


def padded_cu(cu, N_max):
    out = np.full(N_max + 1, cu[-1], dtype=np.int32)
    out[:len(cu)] = cu
    return out


def event_times(torch, fn, steps, warmup):
    """p50, p95 and mean (ms) of ``steps`` calls of fn, each bracketed by HIP
    events on the current stream."""
    for _ in range(warmup):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[2 * i].record()
        fn()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    t = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)])
    return float(np.median(t)), float(np.percentile(t, 95)), float(t.mean())


def wall_ms(torch, fn, steps, warmup):
    """Wall-clock ms per call of ``steps`` back-to-back calls (host dispatch
    included), synchronised at both ends."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def device_inputs(torch, inp, dev):
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    d = {x: torch.from_numpy(inp[x]).to(dev, tdt) for x in ("q", "k", "v")}
    d["g"] = torch.from_numpy(inp["g"]).to(dev)
    d["beta"] = torch.from_numpy(inp["beta"]).to(dev)
    d["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).to(dev)
    return d


def timing_protocol(args, torch, la, inp, src, dev, exact_replay_p50):
    """The RFC's four modes on this workload ("Performance evaluation"):
    eager-live (the exact sizes, host dispatch included), eager-fixed and
    graph-replay in a fixed-capacity bucket (N_max = 64 sequence slots), and
    graph-update-replay (the layout's rows copied into the bucket's static
    buffers and cu_seqlens from pinned host memory, then the replay).  Also
    the padding cost of the bucket, the update overhead, and the break-even
    length: eager-live against graph-update-replay for one sequence of
    growing length in the same bucket."""
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int32)
    T, N = int(cu[-1]), len(cu) - 1
    N_max = max(64, N)
    b = FwdBucket(torch, la, inp, T, N_max, dev)
    cu_pin = torch.from_numpy(padded_cu(cu, N_max)).pin_memory()
    b.load(src, cu_pin)
    torch.cuda.synchronize()
    steps, warm = max(10, args.steps // 4), 3
    eager_fixed = wall_ms(torch, b.step, steps, warm)
    capture_ms = b.capture()
    rp50, rp95, _ = event_times(torch, b.graph.replay, steps, warm)

    def update_replay():
        b.load(src, cu_pin)
        b.graph.replay()

    up50, up95, _ = event_times(torch, update_replay, steps, warm)
    upd50, _, _ = event_times(torch, lambda: b.load(src, cu_pin), steps, warm)

    # break-even: one sequence of length L, eager-live (exact sizes) against
    # graph-update-replay in this bucket
    rows = []
    for L in (64, 256, 1024, 4096, T):
        if L > T:
            continue
        cu_l = np.array([0, L], dtype=np.int32)
        sub = {x: (None if src[x] is None else src[x][:L] if x != "h0" else src[x][:1])
               for x in src}
        ex = FwdBucket(torch, la, dict(inp, h0=inp["h0"]), L, 1, dev)
        ex.load(sub, torch.from_numpy(cu_l).pin_memory())
        live = wall_ms(torch, ex.step, steps, warm)
        cu_b = torch.from_numpy(padded_cu(cu_l, N_max)).pin_memory()

        def upd():
            b.load(sub, cu_b)
            b.graph.replay()

        gu50, _, _ = event_times(torch, upd, steps, warm)
        rows.append({"tokens": L, "eager_live_ms": round(live, 5),
                     "graph_update_replay_ms": round(gu50, 5)})
        del ex
    faster = [r["tokens"] for r in rows if r["graph_update_replay_ms"] < r["eager_live_ms"]]
    return {
        "bucket": {"T_max": T, "N_max": N_max, "nt_max": b.NT},
        "eager_fixed_ms": round(eager_fixed, 5),
        "graph_replay_bucket_p50_ms": round(rp50, 5), "graph_replay_bucket_p95_ms": round(rp95, 5),
        "graph_update_replay_p50_ms": round(up50, 5),
        "graph_update_replay_p95_ms": round(up95, 5),
        "update_ms": round(upd50, 5),
        "padding_cost_ms": round(rp50 - exact_replay_p50, 5),
        "bucket_capture_ms": round(capture_ms, 3),
        "break_even": {"rows": rows,
                       "graph_faster_up_to_tokens": max(faster) if faster else 0},
    }


def bucket_leg(args, torch, la, dev):
    """The fixed-capacity bucket (T_max = 16384, N_max = 64, GDN, H = 32,
    d = 128, no initial state) over its 20 replay layouts: one capture, each
    layout's cu_seqlens copied into the static buffer and replayed; per-layout
    op fraction (the layout's algorithmic bytes over its replay p50 at
    8 TB/s).  The layouts are the workload's own (synth.bucket_replay_layout);
    the token data are drawn on the device from a seeded generator with the
    workload's distributions (the timing does not depend on their values)."""
    import synth
    T_max, N_max, H, d = synth.BUCKET_T_MAX, synth.BUCKET_N_MAX, 32, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(3000)
    bf = torch.bfloat16

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float64)
        return (x / x.norm(dim=-1, keepdim=True).clamp_min(1e-6)).to(bf)

    src = {"q": unit((T_max, H, d)), "k": unit((T_max, H, d)),
           "v": torch.randn((T_max, H, d), generator=gen, device=dev).to(bf),
           "g": torch.nn.functional.logsigmoid(
               torch.randn((T_max, H), generator=gen, device=dev) + 3.0),
           "beta": torch.sigmoid(torch.randn((T_max, H), generator=gen, device=dev)),
           "h0": None}
    spec = dict(H=H, dk=d, dv=d, dtype="bf16", kda=False, h0=None)
    b = FwdBucket(torch, la, spec, T_max, N_max, dev)
    for x in ("q", "k", "v", "g", "beta"):
        getattr(b, x).copy_(src[x])
    b.cu.copy_(torch.from_numpy(synth.bucket_replay_layout(0)))
    b.capture()
    fr = []
    for r in range(args.layouts):
        cu = synth.bucket_replay_layout(r)
        b.cu.copy_(torch.from_numpy(cu))
        p50, _, _ = event_times(torch, b.graph.replay, 5, 2)
        ab = alg_bytes(dict(spec, cu_seqlens=cu), "op")
        fr.append(ab / (p50 * 1e-3) / 1e9 / HBM_PEAK_GBS)
    fr.sort()
    return {"workload": WORKLOADS["c3"][2], "layouts": len(fr),
            "op_hbm_frac_median": round(fr[len(fr) // 2], 4), "op_hbm_frac_min": round(fr[0], 4),
            "op_hbm_frac_max": round(fr[-1], 4)}


def bench_forward(args, torch, la, synth, dev):
    cfg, kda, desc = WORKLOADS[args.workload]
    T_arg = 2048 if args.workload.endswith("_short") else None
    inp = synth.config(cfg, kda=kda, T=T_arg) if cfg == 4 else synth.config(cfg)
    T = inp["q"].shape[0]
    H, dk, dv = inp["H"], inp["dk"], inp["dv"]
    cu_np = np.asarray(inp["cu_seqlens"], dtype=np.int32)
    N = len(cu_np) - 1
    src = device_inputs(torch, inp, dev)
    b = FwdBucket(torch, la, inp, T, N, dev, args.dv_split, args.seg_len)
    b.load(src, torch.from_numpy(cu_np).pin_memory())
    torch.cuda.synchronize()
    is_kda = bool(inp["kda"])
    split, seg = b.split, b.seg
    fwd_kw = b.kw
    args_t = (b.q, b.k, b.v, b.g, b.beta, b.cu, b.ci, b.co)
    stage_kw = dict(fwd_kw, build_meta=True, meta_status=b.st)
    # the standalone metadata kernel, timed for comparison only (not part of
    # the step), into arrays of its own
    ci_alone, co_alone = torch.empty_like(b.ci), torch.empty_like(b.co)
    st_alone = torch.empty_like(b.st)

    # ---- eager warmup + per-kernel HIP-event timing on the launch stream
    for _ in range(max(1, args.warmup)):
        b.step()
    torch.cuda.synchronize()
    assert int(b.st.item()) == 0
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        e = evs[i]
        e[0].record()
        la.build_chunk_meta(b.cu, T, chunk_indices=ci_alone, chunk_offsets=co_alone,
                            status=st_alone)
        e[1].record()
        la.chunk_fwd_stages(is_kda, la.STAGE_MAP, *args_t, **stage_kw)
        e[2].record()
        la.chunk_fwd_stages(is_kda, la.STAGE_REDUCE, *args_t, **stage_kw)
        e[3].record()
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])  # ms
    t_meta, t_map, t_red = (float(x) for x in per.mean(axis=0))
    eager_o = b.o.clone()
    eager_ht = b.ht.clone()

    # eager-live: whole steps at the exact sizes, host dispatch included
    eager_ms = wall_ms(torch, b.step, args.steps, 0)

    # ---- graph capture of one step, replay timing
    capture_ms = b.capture()
    for _ in range(args.warmup):
        b.graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        b.graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / args.steps
    # per-replay event pairs on the replay stream: p50 / p95 of one step and
    # the event-timed mean the headline roofline uses
    p50, p95, ev_mean = event_times(torch, b.graph.replay, args.steps, 0)
    graph_eq = bool(torch.equal(b.o, eager_o) and torch.equal(b.ht, eager_ht))
    # diagnostic: four steps in one graph, so the runtime's per-launch cost
    # is paid once per four steps (the headline is one step per replay)
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4):
        for _ in range(4):
            b.step()
    torch.cuda.synchronize()
    g4_ms = wall_ms(torch, g4.replay, args.steps, 5) / 4
    graph_eq = graph_eq and bool(torch.equal(b.o, eager_o) and torch.equal(b.ht, eager_ht))
    del g4

    tokens = int(cu_np[-1])
    value = tokens * args.steps / elapsed
    nt_actual = int(np.ceil(np.diff(cu_np) / 64).sum())

    op_bytes = alg_bytes(inp, "op")
    op_flops = alg_flops(inp)
    kernels = {"map": t_map, "reduce": t_red}
    diag = {}
    for kind, t in kernels.items():
        ab = alg_bytes(inp, kind)
        diag[kind] = {"ms": round(t, 5), "alg_bytes": ab,
                      "hbm_frac": round(ab / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    fused = N <= 64
    diag["meta_standalone"] = {"ms": round(t_meta, 5), "in_step": not fused}
    # HBM traffic of one step: the sum of every kernel's counter-measured
    # bytes, when all were taken on the current sources (else null)
    tr = [load_traffic(kind, args.workload, inp) for kind in ("map", "reduce")]
    traffic = None if (any(x is None for x in tr) or seg) else float(sum(tr))
    achieved = op_bytes / (ev_mean * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": ("whole step (graph replay): chunk_map (building the chunk layout) + "
                       "chunk_reduce" if fused else
                       "whole step (graph replay): chunk_meta + chunk_map + chunk_reduce"
                       + ("" if seg == 0 else
                          f" x2 + chunk_combine (segments of {seg} chunks)")
                       + f", d_v split {split}"),
            "alg_bytes_per_launch": op_bytes, "avg_launch_ms": round(ev_mean, 5)}

    out = {
        "metric": "GDN/KDA chunk-fwd tokens/s (H=16,d=128,8K varlen); % of HBM/MFMA roofline",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 inputs; fp16 MFMA operands, fp32 accumulation and state"
        if inp["dtype"] == "bf16" else "fp32",
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": desc,
                   "mode": "graph-replay of map (building the chunk layout) + reduce" if fused
                   else "graph-replay of meta+map+reduce",
                   "tokens": tokens, "heads": H, "d": dk, "sequences": N, "nt_max": b.NT,
                   "dv_split": split, "seg_len": seg},
        "roofline": roof,
        "op_roofline": {
            "alg_bytes": op_bytes, "alg_flops": op_flops,
            "hbm_frac": round(op_bytes / (ev_mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(op_flops / (ev_mean * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)},
        "kernels": diag,
        "eager_live_ms": round(eager_ms, 5), "capture_ms": round(capture_ms, 3),
        "graph_x4_ms_per_step": round(g4_ms, 5),
        "replay_p50_ms": round(p50, 5), "replay_p95_ms": round(p95, 5),
        "kernels_per_step": (2 if seg == 0 else 4) + (not fused),
        "host_launches_per_step": {"eager": (2 if seg == 0 else 4) + (not fused), "graph": 1},
        "chunk_utilisation": round(nt_actual / b.NT, 4),
        "token_utilisation": round(tokens / T, 4),
        "workspace_bytes": int(b.ws.numel()),
        "graph_equals_eager": graph_eq,
        "env": env_record(torch),
    }
    if not args.no_protocol:
        out["protocol"] = timing_protocol(args, torch, la, inp, src, dev, p50)
        mem = torch.cuda.max_memory_allocated(dev)
        out["protocol"]["peak_allocated_bytes"] = int(mem)
    if args.workload == "c1" and not args.no_bucket:
        out["bucket_c3"] = bucket_leg(args, torch, la, dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c1", choices=sorted(WORKLOADS))
    ap.add_argument("--dv-split", type=int, default=0)
    ap.add_argument("--seg-len", type=int, default=0,
                    help="chunks per segment of the reduce (0 auto, -1 one pass per sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-protocol", action="store_true",
                    help="skip the eager-fixed / graph-update-replay / break-even timings")
    ap.add_argument("--no-bucket", action="store_true",
                    help="skip the bucket (20-layout) leg of the default workload")
    ap.add_argument("--layouts", type=int, default=20, help="bucket layouts (c3 only)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(see DESIGN.md, 'More than one GPU').", file=sys.stderr)
        sys.exit(2)

    import torch
    import chunkwise_gated_delta_chunk_amd as la
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4,
                          "launches": 3}))
        return

    if args.workload == "c3":
        bench_bucket(args, torch, la, synth, dev)
        return
    if args.workload in ("dec", "deck"):
        bench_decode(args, torch, la, synth, dev)
        return
    if args.workload == "conv":
        bench_conv(args, torch, la, synth, dev)
        return
    if args.workload in ("bwd", "bwdk"):
        bench_bwd(args, torch, la, synth, dev)
        return

    bench_forward(args, torch, la, synth, dev)


if __name__ == "__main__":
    main()
