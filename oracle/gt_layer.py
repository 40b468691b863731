"""Oracle: the full Graph-Transformer layer around the biased attention (test infrastructure).

The MegaGraph pages evaluate a 16-layer, 8-head Graph Transformer whose hidden and
feed-forward dimensions are both 64 (Fig. 8 caption), and describe each layer as
the attention with a topology-aware bias followed by a feed-forward block (abstract,
Fig. 4). They do not spell the layer out; it is read here as the pre-norm Transformer
layer with the bias inside the attention:

    A   = LN(X; g1, b1)
    Q, K, V = store(A Wq), store(A Wk), store(A Wv)        (heads: hidden index h*D + d)
    O   = attention(Q, K, V; table, codes)                 (float64 here, float32 on the GPU)
    X1  = X + O Wo
    B   = LN(X1; g2, b2)
    X2  = X1 + gelu(B W1 + c1) W2 + c2

LN(x) = (x - mean(x)) / sqrt(var(x) + 1e-5) * g + b over the hidden dimension (biased
variance); gelu(x) = x * Phi(x) with Phi the standard normal distribution function.
store(.) is the bf16 rounding at the points where the GPU stores bfloat16 (Q, K, V
and the attention's output gradient); everything else stays float64.

Parameters of one layer are one flat vector in this order (hid = ffn = 64 in the
pages' model): g1[hid], b1[hid], Wq, Wk, Wv [hid, hid], Wo [hid, hid], g2[hid],
b2[hid], W1 [hid, ffn], c1[ffn], W2 [ffn, hid], c2[hid]; a matrix W[a][b] multiplies
input column a into output column b.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from .attention import full_backward
from .bf16 import round_bf16

LN_EPS = 1e-5


def param_layout(hid: int, ffn: int):
    """name -> (offset, shape) in one layer's parameter vector, and the vector length."""
    out, o = {}, 0
    for name, shape in (("g1", (hid,)), ("b1", (hid,)), ("wq", (hid, hid)), ("wk", (hid, hid)),
                        ("wv", (hid, hid)), ("wo", (hid, hid)), ("g2", (hid,)), ("b2", (hid,)),
                        ("w1", (hid, ffn)), ("c1", (ffn,)), ("w2", (ffn, hid)), ("c2", (hid,))):
        out[name] = (o, shape)
        o += int(np.prod(shape))
    return out, o


def unpack(p, hid: int, ffn: int):
    lay, n = param_layout(hid, ffn)
    p = np.asarray(p, np.float64)
    assert p.shape == (n,)
    return {k: p[o:o + int(np.prod(s))].reshape(s) for k, (o, s) in lay.items()}


def pack(d, hid: int, ffn: int):
    lay, n = param_layout(hid, ffn)
    p = np.zeros(n)
    for k, (o, s) in lay.items():
        p[o:o + int(np.prod(s))] = np.asarray(d[k], np.float64).ravel()
    return p


def layer_norm(x, g, b):
    """Row-wise normalisation over the last axis: returns y, the normalised xhat and
    1/sqrt(var + eps) per row."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + LN_EPS)
    xhat = (x - mu) * rstd
    return xhat * g + b, xhat, rstd


def layer_norm_backward(dy, xhat, rstd, g):
    """Gradient of LN with respect to its input, and of g and b (sums over rows). With
    dxhat = dy * g: dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))."""
    dxhat = dy * g
    dx = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True) - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return dx, (dy * xhat).sum(axis=0), dy.sum(axis=0)


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def gelu_grad(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x)."""
    return 0.5 * (1.0 + erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def _rounder(rounding: bool, noise=None):
    base = round_bf16 if rounding else (lambda a: np.asarray(a, np.float64))
    if noise is None:
        return base
    nrng, eps = noise
    return lambda a: base(np.asarray(a, np.float64) * (1.0 + eps * nrng.standard_normal(np.shape(a))))


def model_forward_backward(x0, params, tables, codes, dout, H: int, ffn: int | None = None, rounding: bool = True,
                           workers: int = 1, block: int = 256, pre_round_noise=None):
    """L layers forward, then the backward of sum(dout * X_L).

    x0 [N, hid]; params [L, P] (layout above); tables [L, H, NB]; codes [N, N];
    dout [N, hid]. Returns a dict with x (X_0..X_L), dx0, dparams [L, P], dtables
    [L, H, NB] and per-layer saved values. ``rounding=False`` removes the bf16 storage
    points (a smooth function, for finite differences); ``pre_round_noise=(rng, eps)``
    perturbs every value by a relative N(0, eps) just before it is rounded (see
    oracle.stack for why).
    """
    rnd = _rounder(rounding, pre_round_noise)
    x0 = np.asarray(x0, np.float64)
    params = np.asarray(params, np.float64)
    tables = np.asarray(tables, np.float64)
    L = params.shape[0]
    N, hid = x0.shape
    ffn = hid if ffn is None else ffn
    D = hid // H
    xs, saved = [x0], []
    for l in range(L):
        p = unpack(params[l], hid, ffn)
        X = xs[-1]
        A, ahat, r1 = layer_norm(X, p["g1"], p["b1"])
        q, k, v = (rnd(A @ p[w]).reshape(N, H, D) for w in ("wq", "wk", "wv"))
        out, lse, *_ = full_backward(q, k, v, codes, tables[l], np.zeros((N, H, D)), block=block, workers=workers)
        O = out.reshape(N, hid)
        X1 = X + O @ p["wo"]
        B, bhat, r2 = layer_norm(X1, p["g2"], p["b2"])
        Hd = B @ p["w1"] + p["c1"]
        G = gelu(Hd)
        X2 = X1 + G @ p["w2"] + p["c2"]
        saved.append(dict(A=A, ahat=ahat, r1=r1, q=q, k=k, v=v, O=O, lse=lse, X1=X1, B=B, bhat=bhat, r2=r2,
                          Hd=Hd, G=G))
        xs.append(X2)
    dX = np.asarray(dout, np.float64)
    dparams = np.zeros_like(params)
    dtables = np.zeros_like(tables)
    for l in reversed(range(L)):
        p = unpack(params[l], hid, ffn)
        s = saved[l]
        g = {}
        # X2 = X1 + gelu(Hd) W2 + c2
        g["w2"] = s["G"].T @ dX
        g["c2"] = dX.sum(axis=0)
        dHd = (dX @ p["w2"].T) * gelu_grad(s["Hd"])
        g["w1"] = s["B"].T @ dHd
        g["c1"] = dHd.sum(axis=0)
        dB = dHd @ p["w1"].T
        dX1_ln, g["g2"], g["b2"] = layer_norm_backward(dB, s["bhat"], s["r2"], p["g2"])
        dX1 = dX + dX1_ln
        # X1 = X + O Wo
        g["wo"] = s["O"].T @ dX1
        dO = rnd(dX1 @ p["wo"].T).reshape(N, H, D)
        _, _, dq, dk, dv, dt = full_backward(s["q"], s["k"], s["v"], codes, tables[l], dO, block=block,
                                             workers=workers)
        dtables[l] = dt
        dq, dk, dv = (t.reshape(N, hid) for t in (dq, dk, dv))
        g["wq"], g["wk"], g["wv"] = s["A"].T @ dq, s["A"].T @ dk, s["A"].T @ dv
        dA = dq @ p["wq"].T + dk @ p["wk"].T + dv @ p["wv"].T
        dX_ln, g["g1"], g["b1"] = layer_norm_backward(dA, s["ahat"], s["r1"], p["g1"])
        dX = dX1 + dX_ln
        dparams[l] = pack(g, hid, ffn)
    return dict(x=xs, dx0=dX, dparams=dparams, dtables=dtables, saved=saved)
