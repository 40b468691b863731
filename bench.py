#!/usr/bin/env python3
"""Benchmark of biased full-graph attention on one MI355X.

One step = the whole hot path over one synthetic input: the forward (scores,
bias gathered from the uint8 code tile, online softmax, PV) and the backward
(delta, key-outer dK/dV/bucket partials, query-outer dQ, dtable reduction).
The distance codes are built once per graph before timing (graph preparation,
like loading the graph); every input is resident in device memory when the
timed region starts.

Prints ONE JSON line. Throughput is giga score-pairs per second,
L*H*N^2 / (fwd+bwd seconds) / 1e9 (L = 1 but for the stacked workload, whose step
is the forward and backward of all its layers, projections included).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload ba32768-bf16] [--cp P]

With --cp P the step is the key-block schedule of graph-aware context parallelism
(MegaGraph pages, Fig. 4) run on this one GPU: P virtual ranks each hold N/P query
rows; every rank processes every one of the P key blocks (with its slice of code
columns) in ring order, merging the partial forward results by log-sum-exp, then
the backward of every (rank, block) pair against the merged statistics. The step
covers all P*P block steps, i.e. the same N^2 pairs as the unsplit path.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "biased-attn fwd+bwd ms & Gpairs/s at N=32768,H=8,d=8; SPD-stream GB/s vs peak"
HBM_PEAK_GBS = 8000.0
# exp2 peak from the unit counts: 256 CUs x 4 SIMDs x 2.4 GHz, and a v_exp_f32 takes two
# quad-cycles of a SIMD (8 lanes per clock, half the rate of an ordinary fp32 instruction;
# rocprofv3's SQ_ACTIVE_INST_VALU shows it on the exp probe)
EXP_PEAK_TOPS = 256 * 4 * 8 * 2.4e9 / 1e12
# published dense bf16/fp16 matrix-core peak (the contractions run as 32x32x16 bf16/fp16 MFMA)
MFMA_PEAK_TFLOPS = 2500.0
# contractions over D per score entry: forward QK^T, PV; key-outer QK^T, dO V^T, P^T dO, dS^T Q;
# query-outer QK^T, dO V^T, dS K; the one-pass backward the key-outer four and dS K
CONTRACTIONS = {"fwd": 2, "bwd_kv": 4, "bwd_q": 3, "bwd_fused": 5}
ROOT = os.path.dirname(os.path.abspath(__file__))
# host cores one GPU's jobs may use on a shared GPU machine (the CPU baseline's worker cap)
CPU_SHARE_CORES = 16
# sources of the kernels the default workload runs (bf16, H = 8, D = 8: the MFMA path)
# matrix-core kernel sources by head dimension (what a recorded traffic figure was taken on)
KERNEL_SOURCES = {8: ["graph_transformer_attention_amd/csrc/attn_mfma.hip",
                      "graph_transformer_attention_amd/csrc/mfma_common.h"],
                  32: ["graph_transformer_attention_amd/csrc/attn_mfma_d32.hip",
                       "graph_transformer_attention_amd/csrc/mfma_common.h"]}


def kernel_source_hash(D: int = 8) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(D, KERNEL_SOURCES[8]):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str, D: int = 8):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(D):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def work_model(name: str, N: int, H: int, D: int, s_bytes: int):
    """Algorithmic work of one launch of a kernel: (flops, exps, hbm bytes).

    Per score entry (h, i, j): each contraction over D costs 2D flops; the softmax
    and bias bookkeeping are counted as the few extra operations the method needs
    (forward: bias add, max, subtract, sum = 4; backward: bias add, subtract lse,
    dS = P(dP - delta) = 4, plus the bucket accumulation in the key-outer pass).
    Bytes: the N^2 code matrix once per pass plus each node tensor read or written once.
    """
    E = H * N * N
    node = N * H * D * s_bytes
    f32node = N * H * D * 4
    if name == "fwd":
        return E * (4 * D + 4), E, N * N + 3 * node + f32node + N * H * 4
    if name == "bwd_kv":
        return E * (8 * D + 5), E, N * N + 4 * node + 2 * N * H * 4 + 2 * f32node
    if name == "bwd_q":
        return E * (6 * D + 4), E, N * N + 4 * node + 2 * N * H * 4 + f32node
    if name == "bwd_fused":     # the key-outer work plus dQ = dS K from the same dS
        return E * (10 * D + 5), E, N * N + 4 * node + 2 * N * H * 4 + 3 * f32node
    if name == "bwd_delta":
        return N * H * 2 * D, 0, 4 * node + f32node + N * H * 4
    hid = H * D
    if name == "qkv_fwd":      # X [N,hid] times three [hid,hid] weights
        return 2 * N * hid * 3 * hid, 0, node + 3 * hid * hid * s_bytes + 3 * node
    if name in ("qkv_bwd_dx", "qkv_bwd_dw"):
        return 2 * N * hid * 3 * hid, 0, 3 * f32node + 3 * hid * hid * s_bytes + f32node
    if name == "store":        # float32 -> storage type
        return 0, 0, f32node + node
    if name in ("layer_fwd", "layer_bwd"):   # one side of a full layer: three 64x64 products per node
        return 3 * 2 * N * hid * hid, 0, 6 * f32node
    if name == "layer_wgrad":                # eight sums over nodes of 64x64 outer products
        return 8 * 2 * N * hid * hid, 0, 16 * f32node
    if name == "merge":        # two partial (out, lse) in, one out
        return 3 * N * H * D, 2 * N * H, 3 * f32node + 3 * N * H * 4
    return 0, 0, 0


def cpu_baseline(inp, n_rows: int, cores: int):
    """Time the float64 oracle's forward+backward on a bounded row sample (for a stacked
    workload: the first layer's attention, its Q/K/V from the oracle's projection)."""
    import oracle
    w = inp.workload
    rows = np.sort(np.random.default_rng(12345).choice(w.N, size=min(n_rows, w.N), replace=False))
    t0 = time.perf_counter()
    codes = oracle.bfs_codes_parallel(inp.indptr, inp.indices, w.C, rows, workers=cores)
    t_bfs = time.perf_counter() - t0
    if w.model == "gt":
        from oracle import gt_layer as gl
        g = {k: v.value[0] for k, v in inp.gt_params.items()}
        a = gl.layer_norm(inp.x0.value, g["g1"], g["b1"])[0]
        q, k, v = (oracle.round_bf16(a @ g[t]).reshape(w.N, w.H, w.D) for t in ("wq", "wk", "wv"))
        table, dout = inp.table.value[0], oracle.round_bf16(inp.dout.value).reshape(w.N, w.H, w.D)
    elif w.layers > 1:
        q, k, v = (t.reshape(w.N, w.H, w.D) for t in oracle.qkv_projection(inp.x0.value, inp.w_qkv.value[0]))
        table, dout = inp.table.value[0], inp.dout.value.reshape(w.N, w.H, w.D)
    else:
        q, k, v, table, dout = inp.q.value, inp.k.value, inp.v.value, inp.table.value, inp.dout.value
    t0 = time.perf_counter()
    oracle.full_backward(q[rows], k, v, codes, table, dout[rows], block=16, workers=cores)
    t_attn = time.perf_counter() - t0
    pairs = len(rows) * w.H * w.N
    return {
        "value": round(pairs / t_attn / 1e9, 6),
        "unit": "Gpairs/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{len(rows)} query rows x {w.N} keys x {w.H} heads of {w.name} "
                   f"(float64 NumPy forward+backward, {t_attn:.1f} s; the oracle's BFS for "
                   f"those rows took another {t_bfs:.1f} s and is not in the rate)"),
        "seconds": round(t_attn, 3),
        "extrapolated_full_step_s": round(t_attn * (w.N / len(rows)), 1),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="ba32768-bf16")
    ap.add_argument("--cp", type=int, default=1,
                    help="time the key-block (context-parallel) schedule with P virtual ranks")
    ap.add_argument("--cpu-rows", type=int, default=6144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays; per-kernel averages then come "
                         "from the same number of eager steps run after the timed replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (the reference for FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the benchmark measures one GPU "
              "(the path shards by query rows across GPUs, but no multi-GPU run is made).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import graph_transformer_attention_amd as gta
    from workloads import WORKLOADS, make_inputs

    byname = {w.name: w for w in WORKLOADS.values()}
    w = byname[args.workload]
    print(f"[bench] {w.describe()}", file=sys.stderr, flush=True)
    inp = make_inputs(w.number)
    N, H, D, C, NB = w.N, w.H, w.D, w.C, w.NB

    t0 = time.perf_counter()
    spd_host = gta.spd_build(inp.indptr, inp.indices, N, C)
    t_spd = time.perf_counter() - t0
    print(f"[bench] distance codes built on the host in {t_spd:.2f} s", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")

    def put(st):
        if st.dtype == "f32":
            return torch.from_numpy(np.ascontiguousarray(st.raw)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(st.raw).view(np.int16)).to(dev).view(torch.bfloat16)

    spd = torch.from_numpy(spd_host).to(dev)
    hist = np.bincount(spd_host.ravel(), minlength=NB)
    del spd_host
    # the same codes built on the GPU (graph preparation, outside the timed step): one
    # untimed run, then one timed with events; it must equal the host build byte for byte
    spd_dev = torch.empty_like(spd)
    spd_ws = torch.empty(max(int(gta.lib().gt_spd_build_device_workspace_bytes(N, int(inp.indptr[-1]), C)), 256),
                         dtype=torch.uint8, device=dev)
    gta.spd_build_device(inp.indptr, inp.indices, N, C, out=spd_dev, workspace=spd_ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gta.spd_build_device(inp.indptr, inp.indices, N, C, out=spd_dev, workspace=spd_ws)
    e1.record()
    torch.cuda.synchronize()
    t_spd_dev = e0.elapsed_time(e1) * 1e-3
    spd_dev_equal = bool(torch.equal(spd_dev, spd))
    print(f"[bench] distance codes built on the GPU in {t_spd_dev * 1e3:.1f} ms (equal to host: {spd_dev_equal})",
          file=sys.stderr, flush=True)
    del spd_dev, spd_ws
    dt = gta.GT_BF16 if w.dtype == "bf16" else gta.GT_F32
    L = w.layers
    P = args.cp
    if P > 1 and (L != 1 or N % (32 * P) != 0):
        print(f"bench.py: --cp {P} needs a single-layer workload with N a multiple of {32 * P}", file=sys.stderr)
        sys.exit(2)
    if P > 1:
        q, k, v, do, table = put(inp.q), put(inp.k), put(inp.v), put(inp.dout), put(inp.table)
        spd_t = spd  # undirected graphs: the code matrix is its own transpose
        Nb = N // P
        cuts = [(i * Nb, (i + 1) * Nb) for i in range(P)]
        out = torch.empty((N, H, D), dtype=torch.float32, device=dev)
        lse = torch.empty((N, H), dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty((N, H, D), dtype=torch.float32, device=dev) for _ in range(3))
        dtab = torch.empty((H, NB), dtype=torch.float32, device=dev)
        ws = torch.empty(gta.bwd_block_workspace_bytes(Nb, Nb, H, D, NB, dt), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(gta.fwd_block_workspace_bytes(Nb, Nb, H, D, NB, dt), 256), dtype=torch.uint8,
                          device=dev)

        def step():
            for r, (r0, r1) in enumerate(cuts):
                for t in range(P):
                    c0, c1 = cuts[(r - t) % P]
                    # the first block overwrites the rank's out/lse, later ones merge into them
                    gta.fwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], table,
                                  out=out[r0:r1], lse=lse[r0:r1], workspace=fws, accumulate=t > 0)
            for r, (r0, r1) in enumerate(cuts):
                for t in range(P):
                    c0, c1 = cuts[(r - t) % P]
                    acc = ((gta.ACC_DQ if t > 0 else 0) | (gta.ACC_DKV if r > 0 else 0)
                           | (gta.ACC_DTABLE if (r, t) != (0, 0) else 0))
                    gta.bwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], spd_t[c0:c1, r0:r1], table,
                                  out[r0:r1], lse[r0:r1], do[r0:r1], dq[r0:r1], dk[c0:c1], dv[c0:c1], dtab,
                                  accumulate=acc, workspace=ws)

        def outputs():
            return [out, dq, dk, dv], dtab
    elif w.model == "gt":
        # the full model: L pre-norm layers (attention with the bias, output projection,
        # residuals, norms, GELU feed-forward), forward and backward
        x0, do, tables = put(inp.x0), put(inp.dout), put(inp.table)
        params = torch.from_numpy(gta.model_pack({k: v.raw for k, v in inp.gt_params.items()}, w.hidden)).to(dev)
        ws = torch.empty(int(gta.lib().gt_model_workspace_bytes(N, L, H, D, NB, dt)), dtype=torch.uint8, device=dev)
        res = {}

        def step():
            res["r"] = gta.model_fwd_bwd(x0, params, tables, spd, do, H,
                                         dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32, workspace=ws)

        def outputs():
            x_last, dx0, dpar, dtl = res["r"]
            return [x_last, dx0, dpar], dtl.reshape(L * H, NB)
    elif L == 1:
        q, k, v, do, table = put(inp.q), put(inp.k), put(inp.v), put(inp.dout), put(inp.table)
        out = torch.empty((N, H, D), dtype=torch.float32, device=dev)
        lse = torch.empty((N, H), dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty((N, H, D), dtype=torch.float32, device=dev) for _ in range(3))
        dtab = torch.empty((H, NB), dtype=torch.float32, device=dev)
        ws = torch.empty(gta.bwd_workspace_bytes(N, H, D, NB, dt), dtype=torch.uint8, device=dev)
        fws = torch.empty(max(gta.fwd_workspace_bytes(N, H, D, NB, dt), 256), dtype=torch.uint8, device=dev)

        def step():
            gta.fwd(q, k, v, spd, table, out=out, lse=lse, workspace=fws)
            gta.bwd(q, k, v, spd, table, out, lse, do, dq=dq, dk=dk, dv=dv, dtable=dtab, workspace=ws)

        def outputs():
            return [out, dq, dk, dv], dtab
    else:
        # the stacked model: L layers of projections + attention, forward and backward
        x0, wq, tables, do = put(inp.x0), put(inp.w_qkv), put(inp.table), put(inp.dout)
        ws = torch.empty(gta.stack_workspace_bytes(N, L, H, D, NB, dt), dtype=torch.uint8, device=dev)
        res = {}

        def step():
            res["r"] = gta.stack_fwd_bwd(x0, wq, tables, spd, do, H, workspace=ws)

        def outputs():
            x_last, dx0, dw, dtl = res["r"]
            return [x_last.float(), dx0, dw], dtl.reshape(L * H, NB)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    exp_measured = gta.probe_peak(0) / 1e3   # T exp2/s, this device, this run
    exp_peak = EXP_PEAK_TOPS
    print(f"[bench] measured v_exp_f32 rate {exp_measured:.2f} T/s (derived peak {exp_peak:.2f})", file=sys.stderr,
          flush=True)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    graph = None
    if args.graph:
        # the library allocates nothing, never synchronises and records no memset, so a
        # whole step (every launch of every layer) can be captured and replayed
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print("[bench] one step captured in a HIP graph", file=sys.stderr, flush=True)

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph is None:
        gta.trace(True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        if graph is None:
            step()
        else:
            graph.replay()
    stop.record()
    torch.cuda.synchronize()
    if graph is not None:  # per-kernel averages from eager steps (the trace events are not captured)
        gta.trace(True)
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
    gta.trace(False)
    per_kernel = gta.trace_collect()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    # Invariants that hold at any size (cheap checks that the timed outputs are sane).
    tensors, dtab_t = outputs()
    dtab_h = dtab_t.double().cpu().numpy()
    absent = hist[:NB] == 0
    checks = {
        "finite": bool(all(torch.isfinite(t).all() for t in tensors)),
        "dtable_row_sum_max_abs": float(np.abs(dtab_h.sum(axis=1)).max()),
        "dtable_absent_buckets_exact_zero": bool(np.all(dtab_h[:, absent] == 0.0)),
    }

    s_bytes = 2 if w.dtype == "bf16" else 4
    kern = {}
    for name, (cnt, tot) in per_kernel.items():
        avg = tot / cnt
        fl, ex, by = work_model(name, N // P, H, D, s_bytes)
        kern[name] = {"launches": cnt, "avg_ms": round(avg, 4),
                      "tflops": round(fl / (avg * 1e-3) / 1e12, 2),
                      "gexp_per_s": round(ex / (avg * 1e-3) / 1e9, 1),
                      "gbs": round(by / (avg * 1e-3) / 1e9, 1)}
    dom = max(per_kernel, key=lambda n: per_kernel[n][1])
    fl, ex, by = work_model(dom, N // P, H, D, s_bytes)
    dom_s = per_kernel[dom][1] / per_kernel[dom][0] * 1e-3
    # the dominant kernel's binding unit: its exps at the exp2 peak, or (on the matrix-core
    # path) its contraction flops at the dense MFMA peak, whichever takes longer
    mfma_path = w.dtype == "bf16" and H == 8 and D in (8, 32)
    cfl = CONTRACTIONS.get(dom, 0) * 2 * D * H * (N // P) ** 2
    if mfma_path and cfl / (MFMA_PEAK_TFLOPS * 1e12) > ex / (exp_peak * 1e12):
        achieved = cfl / dom_s / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 4), "peak": MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                    "op": "contraction flops over D (2D per contraction and score entry); peak = published dense bf16",
                    "ops_per_launch": cfl}
    else:
        achieved = ex / dom_s / 1e12
        roofline = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 4),
                    "peak": round(exp_peak, 3), "peak_measured": round(exp_measured, 3), "unit": "TFLOP/s",
                    "frac": round(achieved / exp_peak, 4),
                    "op": "exp2 (one per score entry and pass; peak from unit counts: 1024 SIMDs x 8 lanes/clock x "
                          "2.4 GHz; peak_measured = this run's v_exp_f32 probe)",
                    "ops_per_launch": ex}
    roofline.update({"traffic": recorded_traffic(dom, w.name, w.D) if P == 1 else None,
                     "algorithmic_bytes_per_launch": by, "avg_launch_ms": round(dom_s * 1e3, 4)})

    pairs = L * H * N * N
    # per step: each kernel's average launch time times its launches per step
    fwd_ms = sum(kern[n]["avg_ms"] * kern[n]["launches"] / args.steps for n in ("fwd", "merge", "fwd_merge")
                 if n in kern)
    bwd_ms = sum(kern[n]["avg_ms"] * kern[n]["launches"] / args.steps for n in kern if n.startswith("bwd"))
    # passes over the code matrix (and exps per score entry) of the kernels that ran: the
    # forward, the key-outer pass and, unless the backward is fused, the query-outer pass.
    # The method itself needs two: one forward and one backward recompute.
    # (a launch that returned at once, such as the three-pass kernels gated behind the
    # one-pass backward, is not a pass: under 2% of the step)
    passes = sum(1 for n in ("fwd", "bwd_kv", "bwd_q", "bwd_fused")
                 if n in kern and kern[n]["avg_ms"] * kern[n]["launches"] / args.steps > 0.02 * ms_step)
    alg_passes = 2
    res = {
        "metric": METRIC,
        "value": round(pairs / (ms_step * 1e-3) / 1e9, 3),
        "unit": "Gpairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if (w.dtype == "bf16" and H == 8 and D in (8, 32)) else "f32",
        "data": "synthetic",
        "launch": "hip_graph" if graph is not None else "eager",
        "config": {"workload": w.name, "graph": f"{w.family} {w.graph_args}", "N": N, "H": H,
                   "D": D, "NB": NB, "storage": w.dtype, "layers": L,
                   **({"cp_ranks": P, "block": f"{N // P}x{N // P}"} if P > 1 else {})},
        "ms_fwd": round(fwd_ms, 4),
        "ms_bwd": round(bwd_ms, 4),
        "code_passes": passes,
        "spd_stream_gbs": round(L * passes * N * N / (ms_step * 1e-3) / 1e9, 1),
        "spd_stream_frac_of_hbm_peak": round(L * passes * N * N / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "spd_stream_gbs_algorithmic": round(L * alg_passes * N * N / (ms_step * 1e-3) / 1e9, 1),
        "exp_per_s": round(passes * pairs / (ms_step * 1e-3), 1),
        "kernels": kern,
        "roofline": roofline,
        "spd_build_host_s": round(t_spd, 2),
        "spd_build_device_ms": round(t_spd_dev * 1e3, 2),
        "spd_build_device_equals_host": spd_dev_equal,
        "exp_peak_tops": round(exp_peak, 3),
        "exp_peak_measured_tops": round(exp_measured, 3),
        "exp_frac_of_step": round(passes * pairs / (ms_step * 1e-3) / (exp_peak * 1e12), 4),
        "exp_frac_of_step_algorithmic": round(alg_passes * pairs / (ms_step * 1e-3) / (exp_peak * 1e12), 4),
        "kernel_source_hash": kernel_source_hash(w.D),
        "checks": checks,
    }
    if not args.no_cpu_baseline:
        # One worker per core of this process's CPU share. A GPU machine shares its host among
        # its GPUs and gives one GPU's jobs 16 cores, whatever the affinity mask lists, so
        # the pool is capped there; the record states both numbers.
        avail = len(os.sched_getaffinity(0))
        cores = min(avail, CPU_SHARE_CORES)
        print(f"[bench] timing the oracle on {cores} host cores ({avail} in the affinity mask)", file=sys.stderr,
              flush=True)
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows, cores)
        res["cpu_baseline"]["cores_in_affinity_mask"] = avail
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
