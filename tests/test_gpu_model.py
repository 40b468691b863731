"""GPU parity of the full Graph-Transformer model (pre-norm attention with the topology
bias, output projection, residuals, norms and GELU feed-forward; gt_model_fwd_bwd)
against the float64 oracle, small stacks element by element.

Tolerance per tensor: max |GPU - oracle| / rms(oracle) <= 1e-4 with float32 storage
(float32 against float64 arithmetic, no rounding points), and <= 2e-2 with bfloat16
storage of Q, K, V and the attention's output gradient (the same rounding points on
both sides; the float32 path may round a value near a bfloat16 tie the other way)."""
import numpy as np
import pytest
import torch

import graph_transformer_attention_amd as gta
from oracle import gt_layer as gl
from workloads import small_case
from workloads.configs import gt_params

from gpu_util import host64

pytestmark = pytest.mark.gpu


def _rel(got, ref):
    """max |got - ref| / rms(ref); for a reference that is exactly zero (one node: the table
    gradients vanish) the plain max |got|, held to 1e-4 by _bound."""
    ref = np.asarray(ref, np.float64)
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return err / rms if rms > 0 else err


def _case(N, H, D, C, L, dtype, seed):
    inp = small_case(N, H, D, C, dtype, seed=seed)
    rng = np.random.default_rng(seed + 7)
    hid = H * D
    named = gt_params(rng, L, hid)
    x0 = rng.standard_normal((N, hid)).astype(np.float32)
    dout = rng.standard_normal((N, hid)).astype(np.float32)
    tables = (rng.standard_normal((L, H, C + 1)) * np.sqrt(0.5)).astype(np.float32)
    codes = gta.spd_build(inp.indptr, inp.indices, N, C)
    return named, x0, dout, tables, codes


@pytest.mark.parametrize("N,H,D,C,L,dtype", [
    (200, 8, 8, 20, 2, "bf16"),    # matrix-core attention
    (777, 8, 8, 20, 2, "bf16"),    # matrix-core attention split along its inner loops
    (131, 8, 8, 12, 3, "f32"),     # vector-ALU attention, float32 storage
    (97, 4, 16, 6, 2, "f32"),
    (150, 2, 32, 9, 2, "bf16"),    # vector-ALU attention with bfloat16 storage
    (1, 8, 8, 3, 1, "bf16"),       # one node, one layer
    (70, 1, 64, 5, 2, "f32"),      # a single head of 64
])
def test_model_matches_oracle(N, H, D, C, L, dtype):
    print(f"model N={N} H={H} D={D} C={C} L={L} {dtype}", flush=True)
    named, x0, dout, tables, codes = _case(N, H, D, C, L, dtype, seed=N)
    hid = H * D
    params = gta.model_pack({k: v.raw for k, v in named.items()}, hid)
    ref_params = np.stack([gl.pack({k: v.value[l] for k, v in named.items()}, hid, hid) for l in range(L)])
    np.testing.assert_array_equal(params.astype(np.float64), ref_params)   # both layouts agree
    ref = gl.model_forward_backward(x0.astype(np.float64), ref_params, tables.astype(np.float64), codes,
                                    dout.astype(np.float64), H=H, rounding=dtype == "bf16")
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x_last, dx0, dparams, dtables = gta.model_fwd_bwd(t(x0), t(params), t(tables), t(codes), t(dout), H,
                                                      dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    bound = 2e-2 if dtype == "bf16" else 1e-4
    errs = {}
    pairs = [("x_last", host64(x_last), ref["x"][-1]), ("dx0", host64(dx0), ref["dx0"]),
             ("dparams", host64(dparams), ref["dparams"]), ("dtables", host64(dtables), ref["dtables"])]
    # per-parameter-block errors of the first layer, so a wrong block is named
    lay, _ = gl.param_layout(hid, hid)
    g = pairs[2][1]
    for k, (o, s) in lay.items():
        n = int(np.prod(s))
        pairs.append((f"d{k}[0]", g[0, o:o + n], ref["dparams"][0, o:o + n]))
    for name, got, r in pairs:
        errs[name] = (_rel(got, r), bound if np.any(r != 0) else 1e-4)
    print("errors:", {k: f"{v:.2e}" for k, (v, _) in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v[0] <= v[1]}
    assert not bad, f"above bound: {bad}"


def test_gt16_ba6800_full_size():
    """The pages' model at its Fig. 8 size: 16 layers, 8 heads, hidden = FFN = 64, 6800
    nodes, against values stored from the oracle (final features and dX0 on 512 sampled
    rows; every layer's parameter and table gradients). Bound per tensor, and per layer for
    the gradients: max(2e-2, 3 x the oracle's own spread when its values before each
    bfloat16 rounding carry a float32-sized relative error)."""
    import hashlib
    import os
    from workloads import make_inputs
    inp = make_inputs(6)
    w = inp.workload
    g = np.load(os.path.join(os.path.dirname(__file__), "golden", f"{w.name}.npz"), allow_pickle=False)
    print(f"model full size {w.name}", flush=True)
    spd_host = gta.spd_build(inp.indptr, inp.indices, w.N, w.C)
    assert hashlib.sha256(spd_host.tobytes()).hexdigest() == str(g["codes_sha256"])
    dev = "cuda"
    params = gta.model_pack({k: v.raw for k, v in inp.gt_params.items()}, w.hidden)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x_last, dx0, dparams, dtables = gta.model_fwd_bwd(t(inp.x0.raw), t(params), t(inp.table.raw), t(spd_host),
                                                      t(inp.dout.raw), w.H, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = g["rows"]
    got = dict(x_last=host64(x_last)[rows], dx0=host64(dx0)[rows], dparams=host64(dparams), dtables=host64(dtables))
    errs = {}
    for k in ("x_last", "dx0", "dparams", "dtables"):
        bound = max(2e-2, 3 * float(g[f"spread_{k}"]))
        errs[k] = (_rel(got[k], g[k].astype(np.float64)), bound)
    print("errors (err, bound):", {k: f"{e:.2e} / {b:.2e}" for k, (e, b) in errs.items()}, flush=True)
    assert all(e <= b for e, b in errs.values()), errs
    # Layer by layer, each against its own RMS: at 2e-2 wherever that layer's spread allows
    # it (3 x spread <= 2e-2), so no layer hides behind a bound set by another.
    bad = []
    for k in ("dparams", "dtables"):
        sp = g[f"spread_{k}_layer"]
        line = []
        for l in range(sp.shape[0]):
            bound = max(2e-2, 3 * float(sp[l]))
            e = _rel(got[k][l], g[k][l].astype(np.float64))
            line.append(f"{l}:{e:.1e}/{bound:.1e}")
            if not e <= bound:
                bad.append((k, l, e, bound))
        print(f"{k} per layer (error/bound):", " ".join(line), flush=True)
    assert not bad, f"per-layer errors above bound: {bad}"
