"""Oracle: a stack of biased-attention layers with Q/K/V projections (test infrastructure).

The MegaGraph pages evaluate a 16-layer, 8-head Graph Transformer with hidden
size 64 (Fig. 8 caption). Only the attention layers and their 64 -> 64 Q/K/V
projections are modelled here; there is no residual, norm, feed-forward or
output projection. Per layer l, with X_0 the node features:

    Q, K, V = bf16(X_l W_q), bf16(X_l W_k), bf16(X_l W_v)     (heads: hidden index h*D + d)
    X_{l+1} = bf16(attention_l(Q, K, V))                     (own bias table per layer)

bf16(.) is round-to-nearest-even at the points where the GPU path stores
bfloat16. The backward starts from dOut on X_L; each layer's attention
gradient input is bf16(dX_{l+1}); dq, dk, dv, dW, dX and dtable stay in float64.
"""
from __future__ import annotations

import numpy as np

from .attention import full_backward
from .bf16 import round_bf16


def _rounder(rounding: bool):
    return round_bf16 if rounding else (lambda a: np.asarray(a, np.float64))


def qkv_projection(x, w_l, rounding: bool = True):
    """One layer's projections: (Q, K, V) = store(X W_t) for t = q, k, v.
    x [N, hid]; w_l [3, hid, hid] with w_l[t][a][b] multiplying column a of X into column b."""
    rnd = _rounder(rounding)
    x = np.asarray(x, np.float64)
    w_l = np.asarray(w_l, np.float64)
    return tuple(rnd(x @ w_l[t]) for t in range(3))


def qkv_projection_backward(x, w_l, dq, dk, dv):
    """Gradients of the projections for output gradients dq, dk, dv [N, hid]:
    dW_t = X^T dT and dX = sum_t dT W_t^T (the chain rule of T = X W_t)."""
    x = np.asarray(x, np.float64)
    w_l = np.asarray(w_l, np.float64)
    dw = np.stack([x.T @ dq, x.T @ dk, x.T @ dv])
    dx = dq @ w_l[0].T + dk @ w_l[1].T + dv @ w_l[2].T
    return dx, dw


def stack_forward_backward(x0, w_qkv, tables, codes, dout, workers: int = 1, block: int = 256,
                           rounding: bool = True, pre_round_noise=None):
    """x0 [N, hid]; w_qkv [L, 3, hid, hid]; tables [L, H, NB]; codes [N, N]; dout [N, hid].

    Returns a dict with x (list of X_0..X_L), per-layer out/lse, dtable [L,H,NB],
    dw [L,3,hid,hid], dx0 [N,hid] and the per-layer attention dq/dk/dv.
    ``rounding=False`` drops the bf16 storage points (a smooth function, for
    finite-difference checks).

    ``pre_round_noise=(rng, eps)`` multiplies every value by (1 + eps * z), z ~ N(0,1)
    drawn from rng, just before it is rounded to bf16. It models an implementation
    whose pre-rounding values carry a relative error of order eps (float32
    accumulation: a few units of 2^-24), which may round values near a bf16 tie the
    other way. Comparing such runs with the unperturbed one measures how far each
    output is fixed by the method itself at bf16 storage.
    """
    base_rnd = _rounder(rounding)
    if pre_round_noise is None:
        rnd = base_rnd
    else:
        nrng, eps = pre_round_noise

        def rnd(a):
            a = np.asarray(a, np.float64)
            return base_rnd(a * (1.0 + eps * nrng.standard_normal(a.shape)))
    x0 = np.asarray(x0, np.float64)
    w = np.asarray(w_qkv, np.float64)
    tables = np.asarray(tables, np.float64)
    L, H = tables.shape[0], tables.shape[1]
    N, hid = x0.shape
    D = hid // H
    xs = [x0]
    qkv = []
    lses = []
    for l in range(L):
        X = xs[-1]
        q, k, v = (rnd(t).reshape(N, H, D) for t in qkv_projection(X, w[l], rounding=False))
        qkv.append((q, k, v))
        out, lse, *_ = full_backward(q, k, v, codes, tables[l], np.zeros((N, H, D)),
                                     block=block, workers=workers)
        lses.append(lse)
        xs.append(rnd(out.reshape(N, hid)))
    G = np.asarray(dout, np.float64)
    dw = np.zeros_like(w)
    dtab = np.zeros_like(tables)
    grads = [None] * L
    for l in reversed(range(L)):
        q, k, v = qkv[l]
        dO = rnd(G).reshape(N, H, D)
        _, _, dq, dk, dv, dt = full_backward(q, k, v, codes, tables[l], dO,
                                             block=block, workers=workers)
        dtab[l] = dt
        X = xs[l]
        dq2, dk2, dv2 = (t.reshape(N, hid) for t in (dq, dk, dv))
        G, dw[l] = qkv_projection_backward(X, w[l], dq2, dk2, dv2)
        grads[l] = (dq, dk, dv)
    return dict(x=xs, lse=lses, dtable=dtab, dw=dw, dx0=G, grads=grads, qkv=qkv)
