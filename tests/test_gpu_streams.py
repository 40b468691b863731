"""Calls on a caller's stream other than the current one.

The binding allocates outputs and temporary workspaces itself when the caller passes
none. Those must belong to the stream the kernels run on: a temporary dropped on
return must not be handed to other work while the kernels still use it. Here the
forward and backward run on a side stream while the current stream allocates and
overwrites memory; the results must equal a serial run bit for bit (the kernels are
deterministic).
"""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from workloads import small_case

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,D", [(777, 8), (1000, 32)])
def test_side_stream_calls_match_serial(N, D):
    # sizes at which every kernel splits its inner loop, so each call needs a workspace
    print(f"side stream N={N} D={D}", flush=True)
    inp = small_case(N, 8, D, 20, "bf16", seed=8)
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, inp.workload.C)).cuda()
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    out, lse = gta.fwd(q, k, v, spd, table)
    ref = [out, lse, *gta.bwd(q, k, v, spd, table, out, lse, do)]
    torch.cuda.synchronize()
    ref = [t.clone() for t in ref]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = []
    for rep in range(3):
        o2, l2 = gta.fwd(q, k, v, spd, table, stream=side)
        got = [o2, l2, *gta.bwd(q, k, v, spd, table, o2, l2, do, stream=side)]
        # the current stream meanwhile allocates and writes memory of the same sizes
        junk = [torch.empty(max(gta.bwd_workspace_bytes(N, 8, D, inp.workload.NB, gta.GT_BF16), 256) // 4 + s,
                            dtype=torch.float32, device="cuda").fill_(float("nan")) for s in range(8)]
        junk += [torch.full_like(t, float("nan")) for t in ref]
        del junk
    torch.cuda.synchronize()
    for name, a, b in zip(["out", "lse", "dq", "dk", "dv", "dtable"], got, ref):
        assert torch.equal(a, b), name
