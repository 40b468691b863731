"""Metamorphic checks of the GPU kernels, with no oracle in the loop (the oracle pins the
same identities on its own side):

* a per-head constant added to the bias table leaves out, dq, dk, dv and dtable unchanged
  (the softmax absorbs it, and each head's dS sums to zero) and moves lse by exactly that
  constant;
* relabelling the nodes (q, k, v, dout rows and both axes of the code matrix by one
  permutation) permutes out, lse, dq, dk and dv the same way and leaves dtable unchanged.

Both runs go through the same kernels, so they may differ only by floating-point rounding.
A table shift keeps every tile's order, and the runs then agree to a tenth of the stated
parity bound for bfloat16 inputs (2e-5 absolute for float32). Relabelling reorders the keys
within tiles, so the lazily rescaled half-precision P of the matrix-core paths is rounded at
other points: each run sits within the parity bound of the exact result (measured 2-5e-3 of
the RMS apart), so they are held to that bound, which an indexing mistake exceeds by far
(float32: 2e-5 absolute). The cases cover the matrix-core paths (bf16, D = 8 with its
one-pass backward, D = 32) and the vector-ALU path (float32, D = 16), at sizes that split
the inner loops.
"""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from workloads import small_case

from gpu_util import TOL_BF16_REL, dev, host64

pytestmark = pytest.mark.gpu

CASES = [(600, 8, 8, 20, "bf16"), (300, 8, 32, 20, "bf16"), (200, 8, 16, 12, "f32")]
NAMES = ["out", "lse", "dq", "dk", "dv", "dtable"]


def _run(q, k, v, spd, table, do):
    out, lse = gta.fwd(q, k, v, spd, table)
    grads = gta.bwd(q, k, v, spd, table, out, lse, do)
    torch.cuda.synchronize()
    return [host64(t) for t in (out, lse, *grads)]


def _check(name, got, ref, dtype, rel):
    e = float(np.max(np.abs(got - ref)))
    if dtype == "f32":
        assert e <= 2e-5, f"{name}: max-abs {e:.2e}"
    else:
        rms = float(np.sqrt(np.mean(ref ** 2)))
        assert e <= rel * rms, f"{name}: max-abs/rms {e / rms:.2e} > {rel:.0e}"


def _inputs(N, H, D, C, dtype, seed):
    inp = small_case(N, H, D, C, dtype, seed=seed)
    spd = gta.spd_build(inp.indptr, inp.indices, N, C)
    return inp, spd


@pytest.mark.parametrize("N,H,D,C,dtype", CASES)
def test_table_shift_moves_only_lse(N, H, D, C, dtype):
    print(f"table shift N={N} D={D} {dtype}", flush=True)
    inp, spd_h = _inputs(N, H, D, C, dtype, seed=41)
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    spd = torch.from_numpy(spd_h).cuda()
    table = dev(inp.table)
    shift = np.linspace(-2.5, 7.0, H)  # one constant per head
    shifted = table + torch.from_numpy(shift).float().cuda()[:, None]
    ref = _run(q, k, v, spd, table, do)
    got = _run(q, k, v, spd, shifted, do)
    for name, g, r in zip(NAMES, got, ref):
        if name == "lse":
            e = float(np.max(np.abs(g - r - shift[None, :])))
            assert e <= 1e-4 * (1.0 + float(np.max(np.abs(r)))), f"lse - shift: max-abs {e:.2e}"
        else:
            _check(name, g, r, dtype, 0.1 * TOL_BF16_REL)


@pytest.mark.parametrize("N,H,D,C,dtype", CASES)
def test_node_relabelling_permutes_outputs(N, H, D, C, dtype):
    print(f"relabelling N={N} D={D} {dtype}", flush=True)
    inp, spd_h = _inputs(N, H, D, C, dtype, seed=42)
    perm = np.random.default_rng(43).permutation(N)
    tp = torch.from_numpy(perm).cuda()
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    table = dev(inp.table)
    ref = _run(q, k, v, torch.from_numpy(spd_h).cuda(), table, do)
    spd_p = torch.from_numpy(np.ascontiguousarray(spd_h[perm][:, perm])).cuda()
    got = _run(q[tp].contiguous(), k[tp].contiguous(), v[tp].contiguous(), spd_p, table, do[tp].contiguous())
    for name, g, r in zip(NAMES, got, ref):
        _check(name, g, r if name == "dtable" else r[perm], dtype, TOL_BF16_REL)
