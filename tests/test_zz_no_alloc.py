"""gt_attn_bwd_static (the backward with a fixed per-GPU scratch array, for callers that
cannot allocate) against gt_attn_bwd with a workspace: the same kernels, so the results
must agree bit for bit. Two calls in a row, the second on a smaller input, share the one
array; a size that needs more scratch than the array holds is refused before any launch."""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from workloads import small_case

from gpu_util import dev

pytestmark = pytest.mark.gpu


def _inputs(N, D, seed):
    inp = small_case(N, 8, D, 20, "bf16", seed=seed)
    spd = torch.from_numpy(gta.spd_build(inp.indptr, inp.indices, N, inp.workload.C)).cuda()
    t = [dev(inp.q), dev(inp.k), dev(inp.v), spd, dev(inp.table)]
    out, lse = gta.fwd(*t)
    return t, out, lse, dev(inp.dout)


@pytest.mark.parametrize("D,sizes", [(8, (4096, 777)), (32, (1000, 129))])
def test_static_scratch_matches_workspace_entry_point(D, sizes):
    for call, N in enumerate(sizes):
        print(f"no-alloc D={D} call {call} N={N}", flush=True)
        (q, k, v, spd, table), out, lse, do = _inputs(N, D, seed=60 + call)
        ref = gta.bwd(q, k, v, spd, table, out, lse, do)
        got = [torch.full_like(t, float("nan")) for t in ref]
        gta.bwd_static(q, k, v, spd, table, out, lse, do, *got)
        torch.cuda.synchronize()
        for name, a, b in zip(["dq", "dk", "dv", "dtable"], got, ref):
            assert torch.equal(a, b), (N, name)


def test_static_scratch_refuses_sizes_beyond_the_array():
    N, H, D, NB = 65536, 8, 32, 49
    assert gta.bwd_workspace_bytes(N, H, D, NB, gta.GT_BF16) > gta.BWD_STATIC_SCRATCH_BYTES
    # tiny stand-in tensors: the size check comes before any pointer is used
    lib = gta.lib()
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = x.data_ptr()
    import ctypes
    rc = lib.gt_attn_bwd_static(*([ctypes.c_void_p(p)] * 13), N, H, D, NB, gta.GT_BF16,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == gta.GT_EINVAL
    assert "scratch" in gta.last_error()
