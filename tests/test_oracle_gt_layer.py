"""Pins of the oracle's full Graph-Transformer layer (pre-norm attention with the
topology bias, output projection, residual, norm, GELU feed-forward, residual):
library special cases for its pieces, exact special cases of the layer, finite
differences of the whole stacked model and torch autograd of an independent
float64 formulation."""
import numpy as np
import pytest
import torch

import oracle
from oracle import gt_layer as gl

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _model(seed, N=12, H=2, D=4, L=2, NB=4, scale=0.5):
    rng = np.random.default_rng(seed)
    hid = H * D
    lay, P = gl.param_layout(hid, hid)
    params = np.zeros((L, P))
    for l in range(L):
        d = {}
        for k, (o, s) in lay.items():
            if k in ("g1", "g2"):
                d[k] = 1.0 + 0.2 * rng.standard_normal(s)
            elif len(s) == 1:
                d[k] = 0.1 * rng.standard_normal(s)
            else:
                d[k] = scale * rng.standard_normal(s) / np.sqrt(s[0])
        params[l] = gl.pack(d, hid, hid)
    x0 = rng.standard_normal((N, hid))
    tables = rng.standard_normal((L, H, NB)) * 0.5
    codes = rng.integers(0, NB, (N, N)).astype(np.uint8)
    dout = rng.standard_normal((N, hid))
    return x0, params, tables, codes, dout


def test_layer_norm_and_gelu_vs_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 16)) * 3 + 1
    g, b = rng.standard_normal(16), rng.standard_normal(16)
    y, xhat, rstd = gl.layer_norm(x, g, b)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (16,), torch.from_numpy(g), torch.from_numpy(b),
                                         eps=gl.LN_EPS).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(xhat.mean(axis=1), 0, atol=1e-12)
    z = np.linspace(-8, 8, 201)
    np.testing.assert_allclose(gl.gelu(z), torch.nn.functional.gelu(torch.from_numpy(z)).numpy(), rtol=1e-12,
                               atol=1e-15)
    assert gl.gelu(np.array(0.0)) == 0.0
    h = 1e-6
    np.testing.assert_allclose(gl.gelu_grad(z), (gl.gelu(z + h) - gl.gelu(z - h)) / (2 * h), rtol=1e-7, atol=1e-8)


def test_layer_norm_backward_finite_differences():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 8))
    g, b, dy = rng.standard_normal(8), rng.standard_normal(8), rng.standard_normal((5, 8))
    y, xhat, rstd = gl.layer_norm(x, g, b)
    dx, dg, db = gl.layer_norm_backward(dy, xhat, rstd, g)
    h = 1e-6
    for (i, j) in [(0, 0), (3, 5), (4, 7)]:
        xp, xm = x.copy(), x.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd = ((gl.layer_norm(xp, g, b)[0] - gl.layer_norm(xm, g, b)[0]) * dy).sum() / (2 * h)
        assert abs(fd - dx[i, j]) < 1e-7
    np.testing.assert_allclose(db, dy.sum(axis=0))
    np.testing.assert_allclose(dg, (dy * xhat).sum(axis=0))


def test_zero_branches_make_the_layer_the_identity():
    """With Wo = 0 and W2 = 0, c2 = 0 both residual branches vanish: X_L = X_0, and the
    gradient of X_0 is dout itself."""
    x0, params, tables, codes, dout = _model(3)
    lay, _ = gl.param_layout(8, 8)
    for name in ("wo", "w2", "c2"):
        o, s = lay[name]
        params[:, o:o + int(np.prod(s))] = 0.0
    r = gl.model_forward_backward(x0, params, tables, codes, dout, H=2, rounding=False)
    np.testing.assert_allclose(r["x"][-1], x0, atol=1e-14)
    np.testing.assert_allclose(r["dx0"], dout, atol=1e-14)


def test_model_finite_differences():
    x0, params, tables, codes, dout = _model(4)
    r = gl.model_forward_backward(x0, params, tables, codes, dout, H=2, rounding=False)

    def loss(x0_, params_, tables_):
        rr = gl.model_forward_backward(x0_, params_, tables_, codes, np.zeros_like(dout), H=2, rounding=False)
        return float((rr["x"][-1] * dout).sum())

    h = 1e-6
    lay, P = gl.param_layout(8, 8)
    picks = [(l, lay[k][0] + j) for l in (0, 1) for k, j in
             (("g1", 3), ("b1", 0), ("wq", 9), ("wk", 17), ("wv", 33), ("wo", 40), ("g2", 7), ("b2", 2),
              ("w1", 5), ("c1", 6), ("w2", 60), ("c2", 1))]
    for l, idx in picks:
        pp, pm = params.copy(), params.copy()
        pp[l, idx] += h
        pm[l, idx] -= h
        fd = (loss(x0, pp, tables) - loss(x0, pm, tables)) / (2 * h)
        assert abs(fd - r["dparams"][l, idx]) < 1e-6 * max(1.0, abs(fd)), (l, idx, fd, r["dparams"][l, idx])
    for (i, j) in [(0, 0), (7, 5), (11, 7)]:
        xp, xm = x0.copy(), x0.copy()
        xp[i, j] += h
        xm[i, j] -= h
        fd = (loss(xp, params, tables) - loss(xm, params, tables)) / (2 * h)
        assert abs(fd - r["dx0"][i, j]) < 1e-6 * max(1.0, abs(fd))
    for (l, hh, b) in [(0, 0, 1), (1, 1, 3)]:
        tp, tm = tables.copy(), tables.copy()
        tp[l, hh, b] += h
        tm[l, hh, b] -= h
        fd = (loss(x0, params, tp) - loss(x0, params, tm)) / (2 * h)
        assert abs(fd - r["dtables"][l, hh, b]) < 1e-6 * max(1.0, abs(fd))


def test_model_vs_torch_autograd():
    """An independent float64 torch formulation (library norm, GELU and softmax),
    differentiated by autograd."""
    x0, params, tables, codes, dout = _model(5, N=10, L=3)
    H, D, hid = 2, 4, 8
    r = gl.model_forward_backward(x0, params, tables, codes, dout, H=H, rounding=False)
    lay, _ = gl.param_layout(hid, hid)
    X = torch.tensor(x0, requires_grad=True)
    Pm = torch.tensor(params, requires_grad=True)
    T = torch.tensor(tables, requires_grad=True)
    cl = torch.from_numpy(np.minimum(codes, tables.shape[2] - 1).astype(np.int64))
    h = X
    for l in range(params.shape[0]):
        p = {k: Pm[l, o:o + int(np.prod(s))].reshape(s) for k, (o, s) in lay.items()}
        a = torch.nn.functional.layer_norm(h, (hid,), p["g1"], p["b1"], eps=gl.LN_EPS)
        heads = []
        for hh in range(H):
            sl = slice(hh * D, (hh + 1) * D)
            q, k, v = ((a @ p[w])[:, sl] for w in ("wq", "wk", "wv"))
            s = q @ k.T / np.sqrt(D) + T[l, hh][cl]
            heads.append(torch.softmax(s, dim=1) @ v)
        h1 = h + torch.cat(heads, dim=1) @ p["wo"]
        b = torch.nn.functional.layer_norm(h1, (hid,), p["g2"], p["b2"], eps=gl.LN_EPS)
        h = h1 + torch.nn.functional.gelu(b @ p["w1"] + p["c1"]) @ p["w2"] + p["c2"]
    (h * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(r["x"][-1], h.detach().numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(r["dx0"], X.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dparams"], Pm.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(r["dtables"], T.grad.numpy(), rtol=1e-9, atol=1e-11)
