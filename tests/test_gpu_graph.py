"""HIP-graph capture of whole steps.

The library allocates nothing, never synchronises and records no memset, so a whole
forward + backward step can be captured once and replayed: the attention alone (split
along its inner loops, so merge and finish kernels are in the graph), the key-block
schedule of graph-aware context parallelism (MegaGraph pages, Fig. 4) with its
merges and accumulating block steps, the stacked layers and the full model. Every
kernel is deterministic, so each replay must reproduce the eager step bit for bit.
Between replays the outputs are poisoned with NaN and other eager library work runs on
other buffers, with synchronisations, so a replay that skipped a write or read stale
memory would show.
"""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from workloads import small_case
from workloads.configs import gt_params

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _capture(step):
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def _replays_match(g, outputs, eager_ref, other_work, replays=4):
    """outputs() -> the tensors the captured step writes; eager_ref: their eager values."""
    for r in range(replays):
        for t in outputs():
            t.fill_(float("nan"))
        other_work()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(), eager_ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs from the eager step"


def _attention_case(N, H, D, C, dtype, seed):
    inp = small_case(N, H, D, C, dtype, seed=seed)
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, C)).cuda()
    return dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table), spd


@pytest.mark.parametrize("N,H,D,C,dtype", [
    (777, 8, 8, 20, "bf16"),     # matrix cores, inner loops split: merge and finish kernels
    (1000, 8, 32, 12, "bf16"),   # matrix cores, D = 32
    (131, 4, 16, 6, "f32"),      # vector ALU
])
def test_attention_step_graph(N, H, D, C, dtype):
    print(f"graph attention N={N} H={H} D={D} C={C} {dtype}", flush=True)
    q, k, v, do, table, spd = _attention_case(N, H, D, C, dtype, seed=11)
    NB = table.shape[1]
    dt = gta.GT_BF16 if dtype == "bf16" else gta.GT_F32
    out = torch.empty((N, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty((N, H, D), dtype=torch.float32, device="cuda") for _ in range(3))
    dtab = torch.empty((H, NB), dtype=torch.float32, device="cuda")
    ws = torch.empty(gta.bwd_workspace_bytes(N, H, D, NB, dt), dtype=torch.uint8, device="cuda")
    fws = torch.empty(max(gta.fwd_workspace_bytes(N, H, D, NB, dt), 256), dtype=torch.uint8, device="cuda")

    def step():
        gta.fwd(q, k, v, spd, table, out=out, lse=lse, workspace=fws)
        gta.bwd(q, k, v, spd, table, out, lse, do, dq=dq, dk=dk, dv=dv, dtable=dtab, workspace=ws)

    def outputs():
        return [out, lse, dq, dk, dv, dtab]

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = _capture(step)
    # other work between replays: the same library on other inputs and buffers
    q2, k2, v2, do2, table2, spd2 = _attention_case(N, H, D, C, dtype, seed=12)
    o2, l2 = gta.fwd(q2, k2, v2, spd2, table2)

    def other():
        gta.fwd(q2, k2, v2, spd2, table2, out=o2, lse=l2)
        gta.bwd(q2, k2, v2, spd2, table2, o2, l2, do2)

    _replays_match(g, outputs, ref, other)


def test_block_schedule_graph():
    N, H, D, C = 1000, 8, 8, 16
    print(f"graph block schedule N={N}", flush=True)
    q, k, v, do, table, spd = _attention_case(N, H, D, C, "bf16", seed=21)
    NB = table.shape[1]
    cuts = [0, 320, 656, 1000]
    P = len(cuts) - 1
    blocks = list(zip(cuts, cuts[1:]))
    out = torch.empty((N, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty((N, H, D), dtype=torch.float32, device="cuda") for _ in range(3))
    dtab = torch.empty((H, NB), dtype=torch.float32, device="cuda")
    fws = torch.empty(max(max(gta.fwd_block_workspace_bytes(b1 - b0, c1 - c0, H, D, NB, gta.GT_BF16)
                              for b0, b1 in blocks for c0, c1 in blocks), 256), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(gta.bwd_block_workspace_bytes(b1 - b0, c1 - c0, H, D, NB, gta.GT_BF16)
                          for b0, b1 in blocks for c0, c1 in blocks), dtype=torch.uint8, device="cuda")

    def step():
        for r, (r0, r1) in enumerate(blocks):
            for t in range(P):
                c0, c1 = blocks[(r - t) % P]
                gta.fwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], table,
                              out=out[r0:r1], lse=lse[r0:r1], workspace=fws, accumulate=t > 0)
        for r, (r0, r1) in enumerate(blocks):
            for t in range(P):
                c0, c1 = blocks[(r - t) % P]
                acc = ((gta.ACC_DQ if t > 0 else 0) | (gta.ACC_DKV if r > 0 else 0)
                       | (gta.ACC_DTABLE if (r, t) != (0, 0) else 0))
                gta.bwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], spd[c0:c1, r0:r1], table,
                              out[r0:r1], lse[r0:r1], do[r0:r1], dq[r0:r1], dk[c0:c1], dv[c0:c1], dtab,
                              accumulate=acc, workspace=bws)

    def outputs():
        return [out, lse, dq, dk, dv, dtab]

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = _capture(step)
    o2, l2 = gta.fwd(k, q, v, spd, table)   # other work: attention with q and k swapped

    def other():
        gta.fwd(k, q, v, spd, table, out=o2, lse=l2)

    _replays_match(g, outputs, ref, other)


def test_stack_graph():
    N, H, D, C, L = 300, 8, 8, 10, 2
    print(f"graph stack N={N} L={L}", flush=True)
    inp = small_case(N, H, D, C, "bf16", seed=31)
    rng = np.random.default_rng(31)
    hid = H * D
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, C)).cuda()
    x0 = torch.from_numpy(rng.standard_normal((N, hid)).astype(np.float32)).cuda().to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((L, 3, hid, hid)) / 8).astype(np.float32)).cuda().to(torch.bfloat16)
    tables = torch.from_numpy((rng.standard_normal((L, H, C + 1)) * np.sqrt(0.5)).astype(np.float32)).cuda()
    dout = torch.from_numpy(rng.standard_normal((N, hid)).astype(np.float32)).cuda().to(torch.bfloat16)
    ws = torch.empty(gta.stack_workspace_bytes(N, L, H, D, C + 1, gta.GT_BF16), dtype=torch.uint8, device="cuda")
    res = {}

    def step():
        res["r"] = gta.stack_fwd_bwd(x0, w, tables, spd, dout, H, workspace=ws)

    def outputs():
        return list(res["r"])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = _capture(step)
    ws2 = torch.empty_like(ws)

    def other():
        gta.stack_fwd_bwd(dout, w, tables, spd, x0, H, workspace=ws2)

    _replays_match(g, outputs, ref, other)


def test_model_graph():
    N, H, D, C, L = 300, 8, 8, 10, 2
    print(f"graph model N={N} L={L}", flush=True)
    inp = small_case(N, H, D, C, "bf16", seed=41)
    rng = np.random.default_rng(41)
    hid = H * D
    named = gt_params(rng, L, hid)
    params = torch.from_numpy(gta.model_pack({k: v.raw for k, v in named.items()}, hid)).cuda()
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, C)).cuda()
    x0 = torch.from_numpy(rng.standard_normal((N, hid)).astype(np.float32)).cuda()
    dout = torch.from_numpy(rng.standard_normal((N, hid)).astype(np.float32)).cuda()
    tables = torch.from_numpy((rng.standard_normal((L, H, C + 1)) * np.sqrt(0.5)).astype(np.float32)).cuda()
    ws = torch.empty(int(gta.lib().gt_model_workspace_bytes(N, L, H, D, C + 1, gta.GT_BF16)), dtype=torch.uint8,
                     device="cuda")
    res = {}

    def step():
        res["r"] = gta.model_fwd_bwd(x0, params, tables, spd, dout, H, dtype=torch.bfloat16, workspace=ws)

    def outputs():
        return list(res["r"])

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    g = _capture(step)
    ws2 = torch.empty_like(ws)

    def other():
        gta.model_fwd_bwd(dout, params, tables, spd, x0, H, dtype=torch.bfloat16, workspace=ws2)

    _replays_match(g, outputs, ref, other)
