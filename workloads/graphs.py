"""Seeded synthetic graphs (input generation only).

The pages evaluate biased Graph-Transformer attention on graphs they do not
name (MegaGraph, "Fig. 8" caption: a 16-layer, 8-head model, batch 6800).
These generators stand in for those datasets. Each returns an undirected,
simple graph in CSR form: ``indptr`` int64 [N+1] and ``indices`` int32 [2E],
every neighbour list sorted ascending, no self loops, no duplicates.

Nothing here computes distances, biases or attention: this module is shared
by the oracle side and the HIP side only as a source of inputs.
"""
from __future__ import annotations

import numpy as np


def csr_from_edges(n: int, u: np.ndarray, v: np.ndarray):
    """Symmetric CSR from an undirected edge list (self loops and duplicates dropped)."""
    u = np.asarray(u, dtype=np.int64)
    v = np.asarray(v, dtype=np.int64)
    keep = u != v
    u, v = u[keep], v[keep]
    src = np.concatenate([u, v])
    dst = np.concatenate([v, u])
    key = np.unique(src * n + dst)
    src = key // n
    dst = key % n
    indptr = np.zeros(n + 1, dtype=np.int64)
    np.add.at(indptr, src + 1, 1)
    indptr = np.cumsum(indptr)
    return indptr, dst.astype(np.int32)


def erdos_renyi(n: int, avg_degree: float, rng: np.random.Generator):
    """G(n, p) with p = avg_degree/(n-1); upper-triangle pairs drawn in row-major order."""
    p = avg_degree / (n - 1)
    iu, ju = np.triu_indices(n, k=1)
    hit = rng.random(iu.shape[0]) < p
    return csr_from_edges(n, iu[hit], ju[hit])


def random_geometric(n: int, avg_degree: float, rng: np.random.Generator):
    """n points uniform in the unit square; an edge joins the n*avg_degree/2 closest pairs.

    The radius is the (n*avg_degree/2)-th smallest pairwise distance, so the
    average degree is exact (the closed-form radius undershoots near the border).
    """
    pts = rng.random((n, 2))
    iu, ju = np.triu_indices(n, k=1)
    d2 = ((pts[iu] - pts[ju]) ** 2).sum(axis=1)
    m = int(round(n * avg_degree / 2))
    r2 = np.partition(d2, m - 1)[m - 1]
    hit = d2 <= r2
    return csr_from_edges(n, iu[hit], ju[hit])


def barabasi_albert(n: int, m: int, rng: np.random.Generator):
    """Preferential attachment: seed clique on m+1 nodes, then each new node links to
    m distinct earlier nodes drawn with probability proportional to degree
    (a duplicate draw is redrawn). Edge count is m*n - m*(m+1)/2."""
    seed = m + 1
    us, vs = [], []
    pool = np.empty(2 * (m * n), dtype=np.int64)  # node id repeated once per incident edge end
    plen = 0
    for a in range(seed):
        for b in range(a + 1, seed):
            us.append(a)
            vs.append(b)
            pool[plen] = a
            pool[plen + 1] = b
            plen += 2
    for x in range(seed, n):
        chosen = []
        while len(chosen) < m:
            t = int(pool[int(rng.integers(plen))])
            if t not in chosen:
                chosen.append(t)
        for t in chosen:
            us.append(x)
            vs.append(t)
            pool[plen] = x
            pool[plen + 1] = t
            plen += 2
    return csr_from_edges(n, np.array(us), np.array(vs))


def stochastic_block(n_blocks: int, block_size: int, p_in: float, p_out: float,
                     rng: np.random.Generator):
    """SBM over contiguous blocks. For each block pair (a <= b) the edge count is
    Binomial(M, p) and that many distinct node pairs are drawn uniformly, which is
    the exact SBM law."""
    n = n_blocks * block_size
    us, vs = [], []
    bs = block_size
    iu, ju = np.triu_indices(bs, k=1)
    for a in range(n_blocks):
        for b in range(a, n_blocks):
            if a == b:
                M = bs * (bs - 1) // 2
                k = int(rng.binomial(M, p_in))
                pick = rng.choice(M, size=k, replace=False)
                us.append(a * bs + iu[pick])
                vs.append(a * bs + ju[pick])
            else:
                M = bs * bs
                k = int(rng.binomial(M, p_out))
                pick = rng.choice(M, size=k, replace=False)
                us.append(a * bs + pick // bs)
                vs.append(b * bs + pick % bs)
    return csr_from_edges(n, np.concatenate(us), np.concatenate(vs))


def path_graph(n: int):
    """0-1-2-...-(n-1); used for long-distance edge cases."""
    a = np.arange(n - 1)
    return csr_from_edges(n, a, a + 1)


def clique_chain(n: int, size: int = 32):
    """Cliques of `size` consecutive ids (the last one ragged), each joined to the next by
    one edge (last id of a clique to the first of the next): the distance from a node to
    the nodes of the clique k places away grows by about 2 per clique."""
    u, v = [], []
    for c0 in range(0, n, size):
        ids = np.arange(c0, min(n, c0 + size))
        a, b = np.triu_indices(len(ids), 1)
        u.append(ids[a])
        v.append(ids[b])
        if c0 + size < n:
            u.append(np.array([c0 + size - 1]))
            v.append(np.array([c0 + size]))
    return csr_from_edges(n, np.concatenate(u), np.concatenate(v))


def degrees(indptr: np.ndarray) -> np.ndarray:
    return np.diff(indptr)
