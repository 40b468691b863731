"""Oracle: shortest-path-distance codes by breadth-first search (test infrastructure).

The topology-aware bias of the MegaGraph pages (abstract) is read here as a
lookup of a learned per-head table by the hop distance between two nodes.
The stored code of a pair (s, j) is

    min(dist(s, j), C - 1)   if j is reachable from s   (dist(s, s) = 0)
    C                        otherwise

so a table with NB = C + 1 columns holds C distance buckets (the last one
clipped) and one unreachable bucket.
"""
from __future__ import annotations

from collections import deque

import numpy as np


def _adjacency(indptr, indices):
    ind = np.asarray(indices).tolist()
    ptr = np.asarray(indptr).tolist()
    return [ind[ptr[u]:ptr[u + 1]] for u in range(len(ptr) - 1)]


def bfs_codes(indptr, indices, C: int, sources, adj=None) -> np.ndarray:
    """Codes of every node as seen from each source: FIFO breadth-first search
    from the source over the CSR adjacency, then the clip/unreachable rule above.
    Returns uint8 [len(sources), N]."""
    if not 2 <= C + 1 <= 256:
        raise ValueError("C must lie in [1, 255]")
    n = len(indptr) - 1
    if adj is None:
        adj = _adjacency(indptr, indices)
    out = np.empty((len(sources), n), dtype=np.uint8)
    for r, s in enumerate(sources):
        dist = [-1] * n
        dist[s] = 0
        todo = deque([s])
        while todo:
            u = todo.popleft()
            du = dist[u] + 1
            for w in adj[u]:
                if dist[w] < 0:
                    dist[w] = du
                    todo.append(w)
        d = np.array(dist, dtype=np.int64)
        out[r] = np.where(d < 0, C, np.minimum(d, C - 1)).astype(np.uint8)
    return out


_G = {}


def _one_blas_thread():
    # one BLAS thread per pool worker, so the workers do not oversubscribe the cores
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except ImportError:
        pass


def _pool_init(indptr, indices, C):
    _one_blas_thread()
    _G["adj"] = _adjacency(indptr, indices)
    _G["args"] = (indptr, indices, C)


def _pool_rows(chunk):
    indptr, indices, C = _G["args"]
    return chunk[0], bfs_codes(indptr, indices, C, chunk, adj=_G["adj"])


def bfs_codes_parallel(indptr, indices, C: int, sources, workers: int, chunk: int = 64) -> np.ndarray:
    """Same as bfs_codes, with sources spread over a process pool (each BFS is independent)."""
    import multiprocessing as mp

    sources = np.asarray(sources, dtype=np.int64)
    out = np.empty((len(sources), len(indptr) - 1), dtype=np.uint8)
    chunks = [sources[i:i + chunk] for i in range(0, len(sources), chunk)]
    pos = {int(c[0]): i * chunk for i, c in enumerate(chunks)}
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init, initargs=(indptr, indices, C)) as pool:
        for first, rows in pool.imap_unordered(_pool_rows, chunks):
            p = pos[int(first)]
            out[p:p + len(rows)] = rows
    return out


def components(indptr, indices) -> np.ndarray:
    """Connected-component label per node by union-find (path halving), independent of BFS."""
    n = len(indptr) - 1
    parent = list(range(n))

    def find(x):
        while parent[x] != x:
            parent[x] = parent[parent[x]]
            x = parent[x]
        return x

    ptr = np.asarray(indptr)
    ind = np.asarray(indices)
    src = np.repeat(np.arange(n), np.diff(ptr))
    for a, b in zip(src.tolist(), ind.tolist()):
        ra, rb = find(a), find(b)
        if ra != rb:
            parent[max(ra, rb)] = min(ra, rb)
    return np.array([find(x) for x in range(n)], dtype=np.int64)


def certify_codes(indptr, indices, C: int, sources, codes, comp=None) -> bool:
    """Check codes[r] (the row of source sources[r]) without running BFS.

    Holds iff, for every source s and node j:
      * code(s, s) = 0;
      * code(s, j) = C exactly when j lies in another component than s;
      * otherwise, for j != s, code(s, j) = min(C-1, 1 + min over neighbours k of code(s, k)).
    The last line is the Bellman equation of hop distance with the clip applied; by
    induction on the true distance its only solution is the clipped distance.
    """
    n = len(indptr) - 1
    ptr = np.asarray(indptr, dtype=np.int64)
    ind = np.asarray(indices, dtype=np.int64)
    if comp is None:
        comp = components(indptr, indices)
    codes = np.asarray(codes)
    sources = np.asarray(sources, dtype=np.int64)
    deg = np.diff(ptr)
    has_nb = deg > 0
    starts = ptr[:-1][has_nb]
    for r0 in range(0, len(sources), 256):
        src = sources[r0:r0 + 256]
        cod = codes[r0:r0 + 256].astype(np.int64)
        rr = np.arange(len(src))
        if np.any(cod[rr, src] != 0):
            return False
        other = comp[None, :] != comp[src][:, None]
        if np.any((cod == C) != other):
            return False
        nbmin = np.full(cod.shape, 10 ** 6, dtype=np.int64)
        if ind.size:
            nbmin[:, has_nb] = np.minimum.reduceat(cod[:, ind], starts, axis=1)
        want = np.minimum(C - 1, 1 + nbmin)
        check = ~other
        check[rr, src] = False
        if np.any(cod[check] != want[check]):
            return False
    return True
