"""Workspaces are "contents ignored on entry" (include/gt_attn.h): results may not depend on
what a workspace held before the call. Every case runs once with a zeroed workspace and
then with workspaces filled with 0xFF bytes and with float NaNs (the D = 32 key-outer
pass's code-range flag word among them, which its prep kernel must clear); all outputs
must agree bit for bit. The cases split their inner loops, so the partial-result regions
are in use, and include a D = 32 graph whose codes force the shared-bin rerun."""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from workloads import small_case

from gpu_util import dev

pytestmark = pytest.mark.gpu

PATTERNS = {"ff": lambda t: t.fill_(0xFF),
            "nan": lambda t: t.view(torch.float32).fill_(float("nan")) if t.numel() % 4 == 0 else t.fill_(0xFF)}


def _run(inp, spd, fill):
    w = inp.workload
    N, H, D, NB = w.N, w.H, w.D, w.NB
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    fws = torch.zeros(max(gta.fwd_workspace_bytes(N, H, D, NB, gta.GT_BF16), 256), dtype=torch.uint8, device="cuda")
    bws = torch.zeros(max(gta.bwd_workspace_bytes(N, H, D, NB, gta.GT_BF16), 256), dtype=torch.uint8, device="cuda")
    if fill is not None:
        fill(fws)
        fill(bws)
    out, lse = gta.fwd(q, k, v, spd, table, workspace=fws)
    if fill is not None:
        fill(fws)
    res = [out, lse, *gta.bwd(q, k, v, spd, table, out, lse, do, workspace=bws)]
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("N,D,C,family", [(777, 8, 20, "er"), (1000, 32, 30, "er"), (40, 32, 30, "path"),
                                          (300, 8, 20, "er")])
def test_poisoned_workspaces_give_identical_results(N, D, C, family):
    print(f"poisoned workspace N={N} D={D} {family}", flush=True)
    inp = small_case(N, 8, D, C, "bf16", seed=9, family=family)
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, C)).cuda()
    ref = _run(inp, spd, None)
    for name, fill in PATTERNS.items():
        got = _run(inp, spd, fill)
        for t, a, b in zip(["out", "lse", "dq", "dk", "dv", "dtable"], got, ref):
            assert torch.equal(a, b), (name, t)


def test_poisoned_block_workspaces_give_identical_results():
    # one GA-CP block step of a 3-way key split, forward merging into a running result
    N, D, C = 600, 8, 20
    inp = small_case(N, 8, D, C, "bf16", seed=10)
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, C)).cuda()
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    r0, r1, c0, c1 = 0, 200, 200, 400

    def run(fill):
        fws = torch.zeros(max(gta.fwd_block_workspace_bytes(r1 - r0, c1 - c0, 8, D, C + 1, gta.GT_BF16), 256),
                          dtype=torch.uint8, device="cuda")
        bws = torch.zeros(max(gta.bwd_block_workspace_bytes(r1 - r0, c1 - c0, 8, D, C + 1, gta.GT_BF16), 256),
                          dtype=torch.uint8, device="cuda")
        if fill is not None:
            fill(fws)
            fill(bws)
        out, lse = gta.fwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], table, workspace=fws)
        o2, l2 = out.clone(), lse.clone()
        if fill is not None:
            fill(fws)
        gta.fwd_block(q[r0:r1], k[0:c0], v[0:c0], spd[r0:r1, 0:c0], table, out=o2, lse=l2, workspace=fws,
                      accumulate=True)
        g = gta.bwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], spd[c0:c1, r0:r1], table, o2, l2,
                          do[r0:r1], workspace=bws)
        torch.cuda.synchronize()
        return [o2, l2, *g]

    ref = run(None)
    for name, fill in PATTERNS.items():
        for t, a, b in zip(["out", "lse", "dq", "dk", "dv", "dtable"], run(fill), ref):
            assert torch.equal(a, b), (name, t)
