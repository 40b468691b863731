"""GPU parity of the stacked model's parts (MegaGraph pages, Fig. 8 caption: 16 layers,
8 heads, hidden 64): the Q/K/V projections, the float32 -> bfloat16 storage rounding
and the whole 16-layer stack, through the C ABI, against the float64 oracle."""
import os

import numpy as np
import pytest
import torch

import oracle
import graph_transformer_attention_amd as gta
from workloads import graphs, make_inputs
from workloads.tensors import normal, store

from gpu_util import TOL_BF16_REL, TOL_F32_ABS, check, dev, err, host64

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("N,hid,dtype", [(1, 8, "f32"), (77, 64, "bf16"), (300, 64, "f32"),
                                         (129, 24, "bf16"), (200, 200, "bf16"), (65, 512, "f32")])
def test_qkv_projection_matches_oracle(N, hid, dtype):
    rng = np.random.default_rng(np.random.SeedSequence([7, N, hid]))
    x = store(normal(rng, (N, hid)), dtype)
    w = store(normal(rng, (3, hid, hid), 1.0 / hid), dtype)
    g = [normal(rng, (N, hid)) for _ in range(3)]
    q, k, v = gta.qkv_fwd(dev(x), dev(w))
    dq, dk, dv = (torch.from_numpy(t.astype(np.float32)).cuda() for t in g)
    dx, dw = gta.qkv_bwd(dev(x), dev(w), dq, dk, dv)
    torch.cuda.synchronize()
    ref = oracle.qkv_projection(x.value, w.value, rounding=(dtype == "bf16"))
    for name, got, r in zip("qkv", (q, k, v), ref):
        check(name, host64(got), r, dtype)
    g32 = [t.astype(np.float32).astype(np.float64) for t in g]
    rdx, rdw = oracle.qkv_projection_backward(x.value, w.value, *g32)
    # dx and dw are float32 results of float32 inputs: held to the float32 bound
    # relative to their scale (dw sums N products)
    scale_dw = max(1.0, float(np.sqrt(N)))
    check("dx", host64(dx), rdx, "f32")
    check("dw", host64(dw) / scale_dw, rdw / scale_dw, "f32")


def test_store_rounds_to_nearest_even_bit_exact():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, 10000),
                        1 + np.arange(-64, 64) * 2.0 ** -8, -(1 + np.arange(-64, 64) * 2.0 ** -8),
                        [0.0, -0.0, 3.0e38, -3.0e38, 1.0e-37]]).astype(np.float32)
    src = torch.from_numpy(x).cuda()
    got = gta.store(src, torch.bfloat16)
    got_f32 = gta.store(src, torch.float32)
    torch.cuda.synchronize()
    ref = oracle.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(host64(got), ref)
    np.testing.assert_array_equal(host64(got_f32), x.astype(np.float64))


def _stack_case(N, L, H, D, C, dtype, seed):
    rng = np.random.default_rng(np.random.SeedSequence([seed, N, L, H, D]))
    indptr, indices = graphs.erdos_renyi(N, 4.0, rng)
    hid = H * D
    x0 = store(normal(rng, (N, hid)), dtype)
    w = store(normal(rng, (L, 3, hid, hid), 1.0 / hid), dtype)
    tables = store(normal(rng, (L, H, C + 1), 0.5), "f32")
    dout = store(normal(rng, (N, hid)), dtype)
    return indptr, indices, x0, w, tables, dout


def _run_stack(indptr, indices, x0, w, tables, dout, N, H, C):
    spd_host = gta.spd_build(indptr, indices, N, C)
    spd = torch.from_numpy(spd_host).cuda()
    x_last, dx0, dw, dtab = gta.stack_fwd_bwd(dev(x0), dev(w), dev(tables), spd, dev(dout), H)
    torch.cuda.synchronize()
    return spd_host, dict(x_last=host64(x_last), dx0=host64(dx0), dw=host64(dw), dtable=host64(dtab))


# Stacked bfloat16 layers round every activation to bfloat16 between layers. A value
# close to a bfloat16 tie rounds either way under a float32-sized error, so the outputs
# are only as well determined as the oracle's own spread over runs whose pre-rounding
# values carry such an error (oracle.stack_forward_backward(pre_round_noise=...)).
# Each output tensor is compared as a whole (max-abs over its RMS) at the stated
# bfloat16 tolerance, or at three times that spread where the spread is larger.
NOISE_EPS = 2.0 ** -21
NOISE_RUNS = 3
# a layer whose oracle gradient RMS is this far below the largest layer's is zero in
# exact arithmetic (rounding noise of the oracle's float64 sums)
ZERO_LAYER_RMS = 1e-9


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b ** 2)))


def _stack_outputs(r, rows=None):
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    return dict(x_last=sel(r["x"][-1]), dx0=sel(r["dx0"]), dw=r["dw"], dtable=r["dtable"])


def _compare_stack(got, ref, spread, dtype, layer_spread=None):
    rep = {}
    for name in ("x_last", "dx0", "dw", "dtable"):
        bound = None if dtype == "f32" else max(TOL_BF16_REL, 3.0 * float(spread[name]))
        check(name, got[name], ref[name], dtype, rep, bound)
    print("errors:", {k: f"{v:.2e}" for k, v in rep.items()},
          "spread:", {k: f"{float(v):.2e}" for k, v in spread.items()}, flush=True)
    if layer_spread is None:
        return
    # Layer by layer: each layer's dW and dtable against its own RMS, at the stated 2e-2
    # wherever the oracle's spread for that layer allows it (3 x spread <= 2e-2), and at
    # 3 x spread only past that point. A whole-tensor bound set by the deep layers would
    # otherwise let the well-determined early layers drift unnoticed.
    # Without a residual path the layers average every row of X into the same vector (by
    # layer 6 of ba6800); from there on every dS, so dtable, is exactly zero in real
    # arithmetic and the oracle's values are float64 rounding noise (RMS ~1e-17, eleven
    # orders below the last nonzero layer). A ratio to that RMS compares noise with noise,
    # so such a layer is held like an exactly zero reference: max |GPU| <= 1e-4.
    bad = []
    for name in ("dw", "dtable"):
        rms = np.sqrt(np.mean(ref[name].reshape(ref[name].shape[0], -1) ** 2, axis=1))
        line = []
        for l in range(ref[name].shape[0]):
            if rms[l] < ZERO_LAYER_RMS * rms.max():
                e = float(np.abs(got[name][l]).max())
                bound, ok = TOL_F32_ABS, e <= TOL_F32_ABS
                line.append(f"{l}:|{e:.1e}|/{bound:.0e}")
            else:
                bound = max(TOL_BF16_REL, 3.0 * float(layer_spread[name][l]))
                e, ok = err(got[name][l], ref[name][l], dtype, bound)
                line.append(f"{l}:{e:.1e}/{bound:.1e}")
            if not ok:
                bad.append((name, l, e, bound))
        print(f"{name} per layer (error/bound; |max| for a zero layer):", " ".join(line), flush=True)
    assert not bad, f"per-layer errors above bound: {bad}"


@pytest.mark.parametrize("N,L,H,D,C,dtype", [(200, 3, 8, 8, 20, "bf16"), (131, 2, 8, 8, 12, "f32"),
                                             (97, 2, 2, 16, 6, "bf16")])
def test_stack_small_matches_oracle(N, L, H, D, C, dtype):
    indptr, indices, x0, w, tables, dout = _stack_case(N, L, H, D, C, dtype, seed=3)
    codes, got = _run_stack(indptr, indices, x0, w, tables, dout, N, H, C)
    np.testing.assert_array_equal(codes, oracle.bfs_codes(indptr, indices, C, range(N)))
    args = (x0.value, w.value, tables.value, codes, dout.value)
    ref = _stack_outputs(oracle.stack_forward_backward(*args, rounding=(dtype == "bf16")))
    spread = {k: 0.0 for k in ref}
    if dtype == "bf16":
        for r in range(NOISE_RUNS):
            pr = _stack_outputs(oracle.stack_forward_backward(
                *args, pre_round_noise=(np.random.default_rng(1000 + r), NOISE_EPS)))
            spread = {k: max(spread[k], _rel(pr[k], ref[k])) for k in ref}
    _compare_stack(got, ref, spread, dtype)


def test_stack_ba6800_16_layers_full_size():
    """The 16-layer workload at its full size against stored oracle values and spreads
    (tests/golden/make_golden.py): final features and dX0 on 512 sampled rows, and all
    layers' dW and dtable as whole tensors. Buckets that occur nowhere must have exactly
    zero gradient in every layer."""
    import hashlib
    inp = make_inputs(3)
    w_ = inp.workload
    g = np.load(os.path.join(GOLDEN, f"{w_.name}.npz"))
    codes, got = _run_stack(inp.indptr, inp.indices, inp.x0, inp.w_qkv, inp.table, inp.dout, w_.N, w_.H, w_.C)
    assert hashlib.sha256(codes.tobytes()).hexdigest() == str(g["codes_sha256"])
    absent = np.bincount(codes.ravel(), minlength=w_.NB)[:w_.NB] == 0
    rows = g["rows"]
    got = dict(x_last=got["x_last"][rows], dx0=got["dx0"][rows], dw=got["dw"], dtable=got["dtable"])
    ref = {k: g[k] for k in ("x_last", "dx0", "dw", "dtable")}
    spread = {k: g[f"spread_{k}"] for k in ref}
    layer_spread = {"dw": g["spread_dw_layer"], "dtable": g["spread_dtable_layer"]}
    # the stated 2e-2 holds, by the stored spreads, for dW of layers 0-3 and dtable of layers
    # 0-1; dtable of layers 6-15 is zero in exact arithmetic
    assert np.all(3 * layer_spread["dw"][:4] <= TOL_BF16_REL) and np.all(3 * layer_spread["dtable"][:2] <= TOL_BF16_REL)
    dt_rms = np.sqrt(np.mean(ref["dtable"].reshape(16, -1) ** 2, axis=1))
    assert np.all(dt_rms[6:] < ZERO_LAYER_RMS * dt_rms.max()) and np.all(dt_rms[:6] > 1e-6 * dt_rms.max())
    _compare_stack(got, ref, spread, "bf16", layer_spread)
    assert absent.any() and np.all(got["dtable"][:, :, absent] == 0.0)
