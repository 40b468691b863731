"""The value range of the matrix-core paths (bf16, H = 8, D in {8, 32}).

Those paths carry q, k, v and dout, and the backward's lse*sqrt(D), delta and score
gradients dS, as IEEE half precision in their contractions (include/gt_attn.h,
conventions). Inside the stated range they match the float64 oracle at the bf16
bound; beyond it the affected outputs must not be finite, so that an out-of-range
call is never silently wrong.
"""
import numpy as np
import pytest
import torch

import oracle
import graph_transformer_attention_amd as gta
from workloads import small_case
from workloads.tensors import Stored, bf16_bits_to_f64, store

from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu


def _case(D, seed):
    return small_case(300, 8, D, 20, "bf16", seed=seed)


def _run(inp):
    w = inp.workload
    spd_host = gta.spd_build(inp.indptr, inp.indices, w.N, w.C)
    spd = torch.from_numpy(spd_host).cuda()
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    out, lse = gta.fwd(q, k, v, spd, table)
    dq, dk, dv, dtab = gta.bwd(q, k, v, spd, table, out, lse, do)
    torch.cuda.synchronize()
    got = dict(out=host64(out), lse=host64(lse), dq=host64(dq), dk=host64(dk), dv=host64(dv), dtable=host64(dtab))
    return got, spd_host


@pytest.mark.parametrize("D", [8, 32])
@pytest.mark.parametrize("big", ["v", "dout"])
def test_near_half_limit_matches_oracle(D, big):
    """One of v and dout spread over +-6e4 (bf16 values up to 60160, inside half's
    65504), the other small enough that |dout| |v| 2D stays inside it too."""
    print(f"range: D={D} large {big}", flush=True)
    inp = _case(D, seed=31)
    rng = np.random.default_rng(32)
    shape = inp.v.shape
    large = store(rng.uniform(-6.0e4, 6.0e4, shape), "bf16")
    small = store(rng.standard_normal(shape) * 1e-3, "bf16")
    assert np.abs(large.value).max() < 65504 and np.abs(large.value).max() > 5.9e4
    inp.v, inp.dout = (large, small) if big == "v" else (small, large)
    got, codes = _run(inp)
    ref = oracle.full_backward(inp.q.value, inp.k.value, inp.v.value, codes, inp.table.value, inp.dout.value)
    rep = {}
    for name, r in zip(["out", "lse", "dq", "dk", "dv", "dtable"], ref):
        check(name, got[name], r, "bf16", rep)
    print("errors:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("D", [8, 32])
def test_value_beyond_half_gives_non_finite_output(D):
    # one value of v past half's range (bf16 69632): every query's out for that head and
    # dimension takes it with a nonzero weight
    inp = _case(D, seed=33)
    raw = inp.v.raw.copy()
    raw[5, 3, 1] = 0x4788  # bf16 bits of 69632
    inp.v = Stored("bf16", raw, bf16_bits_to_f64(raw))
    got, _ = _run(inp)
    assert not np.isfinite(got["out"][:, 3, 1]).any()
    assert np.isfinite(np.delete(got["out"], 3, axis=1)).all()  # other heads untouched


@pytest.mark.parametrize("D", [8, 32])
def test_lse_beyond_half_gives_non_finite_gradients(D):
    """A table of 3e4 puts lse*sqrt(D) past 65504. The forward's scores are float32, so its
    output still matches (adding a constant to the table moves only lse); the backward's
    half-precision lse terms overflow, and its gradients must then come out as NaN, not
    as the zeros an infinite lse would give."""
    inp = _case(D, seed=34)
    tab = np.full(inp.table.shape, 3.0e4)
    inp.table = store(tab, "f32")
    got, codes = _run(inp)
    ref = oracle.full_backward(inp.q.value, inp.k.value, inp.v.value, codes, inp.table.value, inp.dout.value)
    rms = np.sqrt(np.mean(ref[0] ** 2))
    assert np.abs(got["out"] - ref[0]).max() / rms <= 2e-2
    for name in ("dq", "dk", "dv"):
        assert not np.isfinite(got[name]).all(), name


@pytest.mark.parametrize("D", [8, 32])
def test_score_gradient_beyond_half_gives_non_finite_gradients(D):
    # dout and v of 1e3: dS = P (dout.v - delta) reaches ~1e6 on peaked rows
    inp = _case(D, seed=35)
    rng = np.random.default_rng(36)
    inp.v = store(rng.standard_normal(inp.v.shape) * 1e3, "bf16")
    inp.dout = store(rng.standard_normal(inp.v.shape) * 1e3, "bf16")
    got, codes = _run(inp)
    ref = oracle.full_backward(inp.q.value, inp.k.value, inp.v.value, codes, inp.table.value, inp.dout.value)
    assert np.abs(ref[2]).max() > 0  # a real gradient exists
    assert not (np.isfinite(got["dq"]).all() and np.isfinite(got["dk"]).all())
