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


def stack_forward_backward(x0, w_qkv, tables, codes, dout, workers: int = 1, block: int = 256,
                           rounding: bool = True):
    """x0 [N, hid]; w_qkv [L, 3, hid, hid]; tables [L, H, NB]; codes [N, N]; dout [N, hid].

    Returns a dict with x (list of X_0..X_L), per-layer out/lse, dtable [L,H,NB],
    dw [L,3,hid,hid], dx0 [N,hid] and the per-layer attention dq/dk/dv.
    ``rounding=False`` drops the bf16 storage points (a smooth function, for
    finite-difference checks).
    """
    rnd = round_bf16 if rounding else (lambda a: np.asarray(a, np.float64))
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
        q, k, v = (rnd(X @ w[l, t]).reshape(N, H, D) for t in range(3))
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
        dw[l, 0], dw[l, 1], dw[l, 2] = X.T @ dq2, X.T @ dk2, X.T @ dv2
        G = dq2 @ w[l, 0].T + dk2 @ w[l, 1].T + dv2 @ w[l, 2].T
        grads[l] = (dq, dk, dv)
    return dict(x=xs, lse=lses, dtable=dtab, dw=dw, dx0=G, grads=grads, qkv=qkv)
