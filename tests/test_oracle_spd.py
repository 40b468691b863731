"""Pins for the oracle's BFS distance codes (CPU only).

The codes are the clipped hop distances of the topology-aware bias; they are
pinned to Floyd-Warshall, to the matrix-power definition of hop distance, to
scipy's shortest_path, and to the Bellman certificate, which must also reject
planted mistakes.
"""
import itertools

import numpy as np
import pytest
from scipy.sparse import csr_matrix
from scipy.sparse.csgraph import shortest_path

import oracle
from workloads import graphs, make_inputs


def _codes_from_dist(dist, C):
    dist = np.asarray(dist, dtype=np.float64)
    out = np.where(np.isinf(dist), C, np.minimum(dist, C - 1))
    return out.astype(np.uint8)


def _floyd_warshall(n, edges):
    d = np.full((n, n), np.inf)
    np.fill_diagonal(d, 0)
    for a, b in edges:
        d[a, b] = d[b, a] = 1
    for k in range(n):
        d = np.minimum(d, d[:, k:k + 1] + d[k:k + 1, :])
    return d


def _matrix_power_dist(n, edges):
    """d(i,j) = min{k : ((A+I)^k)[i,j] > 0} — reachability within k steps."""
    a = np.eye(n, dtype=np.int64)
    for x, y in edges:
        a[x, y] = a[y, x] = 1
    d = np.full((n, n), np.inf)
    reach = np.eye(n, dtype=np.int64)
    for k in range(n):
        d[(reach > 0) & np.isinf(d)] = k
        reach = np.minimum(reach @ a, 1)
    return d


def _csr(n, edges):
    if edges:
        u, v = zip(*edges)
    else:
        u, v = [], []
    return graphs.csr_from_edges(n, np.array(u, dtype=np.int64), np.array(v, dtype=np.int64))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_every_labelled_graph_small(n):
    pairs = list(itertools.combinations(range(n), 2))
    for C in (n + 1, 2, 3):
        for mask in range(1 << len(pairs)):
            edges = [p for b, p in enumerate(pairs) if mask >> b & 1]
            indptr, indices = _csr(n, edges)
            got = oracle.bfs_codes(indptr, indices, C, range(n))
            fw = _floyd_warshall(n, edges)
            mp = _matrix_power_dist(n, edges)
            np.testing.assert_array_equal(fw, mp)
            np.testing.assert_array_equal(got, _codes_from_dist(fw, C))


def test_random_graphs_vs_scipy():
    rng = np.random.default_rng(7)
    for trial in range(60):
        n = int(rng.integers(2, 13))
        p = rng.random() * 0.6
        edges = [(a, b) for a, b in itertools.combinations(range(n), 2) if rng.random() < p]
        indptr, indices = _csr(n, edges)
        C = int(rng.integers(2, 8))
        got = oracle.bfs_codes(indptr, indices, C, range(n))
        m = csr_matrix((np.ones(len(indices)), indices, indptr), shape=(n, n))
        ref = shortest_path(m, unweighted=True, directed=False)
        np.testing.assert_array_equal(got, _codes_from_dist(ref, C))


@pytest.mark.parametrize("number", [1, 2])
def test_workload_graphs_vs_scipy(number):
    inp = make_inputs(number)
    w = inp.workload
    n = w.N
    src = np.arange(n) if n <= 256 else np.random.default_rng(0).choice(n, 64, replace=False)
    got = oracle.bfs_codes(inp.indptr, inp.indices, w.C, src)
    m = csr_matrix((np.ones(len(inp.indices)), inp.indices, inp.indptr), shape=(n, n))
    ref = shortest_path(m, unweighted=True, directed=False, indices=src)
    np.testing.assert_array_equal(got, _codes_from_dist(ref, w.C))


def test_symmetry_and_edges():
    inp = make_inputs(1)
    n, C = inp.workload.N, inp.workload.C
    codes = oracle.bfs_codes(inp.indptr, inp.indices, C, range(n))
    np.testing.assert_array_equal(codes, codes.T)
    adj = np.zeros((n, n), bool)
    src = np.repeat(np.arange(n), np.diff(inp.indptr))
    adj[src, inp.indices] = True
    np.testing.assert_array_equal(codes == 1, adj)
    assert np.all(np.diag(codes) == 0)


def test_clip_on_path_graph():
    n, C = 40, 6
    indptr, indices = graphs.path_graph(n)
    codes = oracle.bfs_codes(indptr, indices, C, range(n))
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    np.testing.assert_array_equal(codes, np.minimum(np.abs(i - j), C - 1))


def test_clique_chain_distances():
    # cliques of 32 consecutive ids, clique k's last id joined to clique k+1's first: from
    # i in clique a to j in a later clique b, leave a at its last id (one step unless i is
    # it), cross each join (b - a joins) and each clique in between (first to last), then
    # reach j from b's first id (one step unless j is it)
    n, s, C = 100, 32, 63
    indptr, indices = graphs.clique_chain(n, s)
    codes = oracle.bfs_codes(indptr, indices, C, range(n))
    want = np.zeros((n, n), np.int64)
    for i in range(n):
        for j in range(n):
            a, b = sorted((i // s, j // s))
            lo, hi = (i, j) if i // s <= j // s else (j, i)
            if a == b:
                want[i, j] = int(i != j)
            else:
                want[i, j] = int(lo != a * s + s - 1) + (b - a) + (b - a - 1) + int(hi != b * s)
    np.testing.assert_array_equal(codes, np.minimum(want, C - 1))


def test_unreachable_bucket():
    # two components {0,1,2} and {3,4}, plus an isolated node 5
    indptr, indices = _csr(6, [(0, 1), (1, 2), (3, 4)])
    C = 4
    codes = oracle.bfs_codes(indptr, indices, C, range(6))
    assert codes[0, 2] == 2 and codes[0, 3] == C and codes[3, 4] == 1
    assert np.all(codes[5, :5] == C) and codes[5, 5] == 0


def test_certificate_accepts_and_rejects():
    inp = make_inputs(1)
    n, C = inp.workload.N, inp.workload.C
    codes = oracle.bfs_codes(inp.indptr, inp.indices, C, range(n))
    assert oracle.certify_codes(inp.indptr, inp.indices, C, range(n), codes)
    rng = np.random.default_rng(3)
    for _ in range(20):
        bad = codes.copy()
        i, j = rng.integers(n, size=2)
        bad[i, j] = (int(bad[i, j]) + int(rng.choice([-1, 1, 2]))) % (C + 1)
        if bad[i, j] == codes[i, j]:
            continue
        assert not oracle.certify_codes(inp.indptr, inp.indices, C, range(n), bad)
    # two components: an unreachable pair labelled as far, and a far pair labelled unreachable
    indptr, indices = _csr(8, [(0, 1), (1, 2), (2, 3), (4, 5), (5, 6), (6, 7)])
    good = oracle.bfs_codes(indptr, indices, 3, range(8))
    assert oracle.certify_codes(indptr, indices, 3, range(8), good)
    bad = good.copy()
    bad[0, 5] = 2
    assert not oracle.certify_codes(indptr, indices, 3, range(8), bad)
    bad = good.copy()
    bad[0, 3] = 3
    assert not oracle.certify_codes(indptr, indices, 3, range(8), bad)


def test_components_vs_scipy():
    from scipy.sparse.csgraph import connected_components
    inp = make_inputs(2)
    n = inp.workload.N
    comp = oracle.components(inp.indptr, inp.indices)
    m = csr_matrix((np.ones(len(inp.indices)), inp.indices, inp.indptr), shape=(n, n))
    k, lab = connected_components(m, directed=False)
    # same partition: labels map one-to-one
    pairs = set(zip(comp.tolist(), lab.tolist()))
    assert len(pairs) == k == len(set(comp.tolist()))


def test_parallel_equals_serial():
    inp = make_inputs(2)
    src = np.arange(0, 4096, 37)
    a = oracle.bfs_codes(inp.indptr, inp.indices, 24, src)
    b = oracle.bfs_codes_parallel(inp.indptr, inp.indices, 24, src, workers=3, chunk=16)
    np.testing.assert_array_equal(a, b)
