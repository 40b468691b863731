"""Oracle: biased multi-head attention forward and backward in float64 (test infrastructure).

Follows the MegaGraph pages' statement that each Graph-Transformer layer
forms an attention score matrix plus a topology-aware bias matrix (abstract),
with the bias read as B[h,i,j] = table[h, code(i,j)] and the scores as
QK^T/sqrt(D) + B. Both matrices are materialised here, one block of query
rows at a time; softmax is the two-pass definition over the whole row.

Layouts: q, k, v, dout, out, dq, dk, dv are [rows or N, H, D]; lse is [rows, H];
codes is [rows, N] uint8 (row = query node, column = key node); table and
dtable are [H, NB]. A code >= NB is clamped to NB - 1.
"""
from __future__ import annotations

import numpy as np


def _bias(table: np.ndarray, codes: np.ndarray, h: int) -> np.ndarray:
    nb = table.shape[1]
    return table[h][np.minimum(codes, nb - 1)]


def forward(q, k, v, codes, table):
    """out [R,H,D], lse [R,H] for the R query rows given (q and codes hold those rows)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    table = np.asarray(table, np.float64)
    R, H, D = q.shape
    out = np.empty((R, H, D))
    lse = np.empty((R, H))
    for h in range(H):
        S = q[:, h, :] @ k[:, h, :].T / np.sqrt(D) + _bias(table, codes, h)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        P = E / l
        out[:, h, :] = P @ v[:, h, :]
        lse[:, h] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def backward(q, k, v, codes, table, dout):
    """Forward and backward for the R query rows given.

    Returns out, lse, dq for those rows, plus the contributions of those rows to
    dk [N,H,D], dv [N,H,D] and dtable [H,NB] (sums over rows; add blocks to get
    the full gradients). The loss is sum(dout * out).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    table = np.asarray(table, np.float64)
    R, H, D = q.shape
    N = k.shape[0]
    NB = table.shape[1]
    sc = 1.0 / np.sqrt(D)
    cl = np.minimum(codes, NB - 1)
    out = np.empty((R, H, D))
    lse = np.empty((R, H))
    dq = np.empty((R, H, D))
    dk = np.zeros((N, H, D))
    dv = np.zeros((N, H, D))
    dtable = np.zeros((H, NB))
    for h in range(H):
        S = q[:, h, :] @ k[:, h, :].T * sc + table[h][cl]
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        l = E.sum(axis=1, keepdims=True)
        P = E / l
        out[:, h, :] = P @ v[:, h, :]
        lse[:, h] = m[:, 0] + np.log(l[:, 0])
        dO = dout[:, h, :]
        dv[:, h, :] = P.T @ dO
        dP = dO @ v[:, h, :].T
        delta = (P * dP).sum(axis=1, keepdims=True)
        dS = P * (dP - delta)
        dq[:, h, :] = dS @ k[:, h, :] * sc
        dk[:, h, :] = dS.T @ q[:, h, :] * sc
        dtable[h] = np.bincount(cl.ravel(), weights=dS.ravel(), minlength=NB)
    return out, lse, dq, dk, dv, dtable


def merge(out_a, lse_a, out_b, lse_b):
    """Attention over the union of two disjoint key sets from the results over each.

    MegaGraph pages, Fig. 4 and its caption: under graph-aware context parallelism
    each key/value block (with its slice of bias columns) yields a partial result,
    and the partial results are combined through their softmax statistics. With
    lse the log of a set's softmax denominator, the union's denominator is the sum
    of the two, and each partial output enters with the share of the denominator
    its keys hold. A side with lse = -inf (no keys) has share 0.
    """
    lse_a = np.asarray(lse_a, np.float64)
    lse_b = np.asarray(lse_b, np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    wa = np.exp(lse_a - lse)[..., None]
    wb = np.exp(lse_b - lse)[..., None]
    return wa * np.asarray(out_a, np.float64) + wb * np.asarray(out_b, np.float64), lse


def backward_block(q, k, v, codes, table, out, lse, dout):
    """Gradient contributions of one key block, given the forward over ALL keys.

    q, dout: [R,H,D] query rows; k, v: [K,H,D] the block's keys; codes: [R,K] the
    bias columns of the block; out, lse: [R,H,D], [R,H] the merged forward results
    over every key. The block's probabilities are the full softmax's entries in
    its columns, P = exp(S - lse), and with delta = rowsum(dout * out) the score
    gradient is dS = P (dout v^T - delta). Returns dq [R,H,D] (this block's share:
    summing over blocks gives the full dq), dk, dv [K,H,D] (the block's keys'
    gradients from these rows) and dtable [H,NB] (this block's share).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    out = np.asarray(out, np.float64)
    lse = np.asarray(lse, np.float64)
    table = np.asarray(table, np.float64)
    R, H, D = q.shape
    K = k.shape[0]
    NB = table.shape[1]
    sc = 1.0 / np.sqrt(D)
    cl = np.minimum(codes, NB - 1)
    dq = np.empty((R, H, D))
    dk = np.empty((K, H, D))
    dv = np.empty((K, H, D))
    dtable = np.empty((H, NB))
    for h in range(H):
        S = q[:, h, :] @ k[:, h, :].T * sc + table[h][cl]
        P = np.exp(S - lse[:, h:h + 1])
        dO = dout[:, h, :]
        delta = (dO * out[:, h, :]).sum(axis=1, keepdims=True)
        dS = P * (dO @ v[:, h, :].T - delta)
        dq[:, h, :] = dS @ k[:, h, :] * sc
        dk[:, h, :] = dS.T @ q[:, h, :] * sc
        dv[:, h, :] = P.T @ dO
        dtable[h] = np.bincount(cl.ravel(), weights=dS.ravel(), minlength=NB)
    return dq, dk, dv, dtable


_G = {}


def _one_blas_thread():
    # one BLAS thread per pool worker, so the workers do not oversubscribe the cores
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _pool_init(q, k, v, codes, table, dout, one_thread=False):
    if one_thread:
        _one_blas_thread()
    _G.update(q=q, k=k, v=v, codes=codes, table=table, dout=dout)


def _pool_block(span):
    r0, r1 = span
    g = _G
    o, l, dq, dk, dv, dt = backward(g["q"][r0:r1], g["k"], g["v"], g["codes"][r0:r1],
                                    g["table"], g["dout"][r0:r1])
    return r0, o, l, dq, dk, dv, dt


def full_backward(q, k, v, codes, table, dout, block: int = 256, workers: int = 1, rows=None):
    """Forward + backward over query rows, in row blocks.

    q, codes and dout hold R query rows (codes [R, N]); k and v hold all N keys.
    With q/codes/dout covering all N rows the results are the full gradients. If
    ``rows`` is given it selects a subset of those R rows. dk/dv/dtable are the
    contributions of the rows processed. Blocks may be spread over a process pool;
    each block is the plain definition above and the partial sums are added in
    block order.
    """
    N = np.asarray(k).shape[0]
    H, D = k.shape[1], k.shape[2]
    NB = np.asarray(table).shape[1]
    if rows is None:
        qs, cs, ds = np.asarray(q), np.asarray(codes), np.asarray(dout)
    else:
        rows = np.asarray(rows)
        qs, cs, ds = np.asarray(q)[rows], np.asarray(codes)[rows], np.asarray(dout)[rows]
    R = qs.shape[0]
    spans = [(r0, min(r0 + block, R)) for r0 in range(0, R, block)]
    out = np.empty((R, H, D))
    lse = np.empty((R, H))
    dq = np.empty((R, H, D))
    dk = np.zeros((N, H, D))
    dv = np.zeros((N, H, D))
    dtable = np.zeros((H, NB))
    if workers <= 1:
        _pool_init(qs, k, v, cs, table, ds)
        results = map(_pool_block, spans)
    else:
        import multiprocessing as mp
        ctx = mp.get_context("fork")
        pool = ctx.Pool(workers, initializer=_pool_init, initargs=(qs, k, v, cs, table, ds, True))
        results = pool.imap(_pool_block, spans)  # in block order
    for r0, o, l, dqb, dkb, dvb, dtb in results:
        r1 = r0 + o.shape[0]
        out[r0:r1], lse[r0:r1], dq[r0:r1] = o, l, dqb
        dk += dkb
        dv += dvb
        dtable += dtb
    if workers > 1:
        pool.close()
        pool.join()
    return out, lse, dq, dk, dv, dtable
