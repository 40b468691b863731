"""Pins for the oracle's biased attention forward/backward (CPU only).

Each pin ties the oracle to something other than itself: a brute-force loop,
torch's scaled_dot_product_attention on the CPU in float64 (a library special
case), closed forms, permutation equivariance and central finite differences.
Chosen so that a dropped term, a wrong scale or sign, a transposed operand or a
wrong index fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import small_case


def _rand(seed, N, H=2, D=4, NB=5, sd=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((N, H, D)) * sd for _ in range(4))
    codes = rng.integers(0, NB, size=(N, N)).astype(np.uint8)
    table = rng.standard_normal((H, NB)) * 0.7
    return q, k, v, codes, table, do


def test_forward_brute_force_loops():
    for seed, N in [(0, 1), (1, 3), (2, 8)]:
        q, k, v, codes, table, _ = _rand(seed, N, H=2, D=3, NB=4)
        out, lse = oracle.forward(q, k, v, codes, table)
        H, D = 2, 3
        for h in range(H):
            for i in range(N):
                s = []
                for j in range(N):
                    dot = 0.0
                    for d in range(D):
                        dot += q[i, h, d] * k[j, h, d]
                    s.append(dot / math.sqrt(D) + table[h, codes[i, j]])
                z = sum(math.exp(x) for x in s)
                assert abs(lse[i, h] - math.log(z)) < 1e-12
                for d in range(D):
                    o = sum(math.exp(s[j]) * v[j, h, d] for j in range(N)) / z
                    assert abs(out[i, h, d] - o) < 1e-12


def _torch_reference(q, k, v, codes, table, do):
    N, H, D = q.shape
    NB = table.shape[1]
    tq, tk, tv = (torch.tensor(a.transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)
                  for a in (q, k, v))
    tt = torch.tensor(table, dtype=torch.float64, requires_grad=True)
    idx = torch.tensor(np.minimum(codes, NB - 1).astype(np.int64))
    mask = tt[:, idx]                                     # [H, N, N]
    mask.retain_grad()
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    tdo = torch.tensor(do.transpose(1, 0, 2), dtype=torch.float64)
    (out * tdo).sum().backward()
    # dtable from the gradient of the materialised mask, gathered per bucket by a plain loop
    dm = mask.grad.numpy()
    dtab = np.zeros((H, NB))
    for b in range(NB):
        sel = np.minimum(codes, NB - 1) == b
        dtab[:, b] = dm[:, sel].sum(axis=1)
    T = lambda x: x.detach().numpy().transpose(1, 0, 2)  # noqa: E731
    return T(out), T(tq.grad), T(tk.grad), T(tv.grad), dtab, tt.grad.numpy()


@pytest.mark.parametrize("N,H,D,NB", [(1, 1, 4, 2), (7, 2, 4, 5), (33, 3, 8, 9), (64, 8, 8, 21)])
def test_vs_torch_sdpa_float64(N, H, D, NB):
    q, k, v, codes, table, do = _rand(N + H, N, H, D, NB)
    out, lse, dq, dk, dv, dtab = oracle.backward(q, k, v, codes, table, do)
    rout, rdq, rdk, rdv, rdtab, rtgrad = _torch_reference(q, k, v, codes, table, do)
    for a, b in [(out, rout), (dq, rdq), (dk, rdk), (dv, rdv), (dtab, rdtab), (dtab, rtgrad)]:
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    out2, lse2 = oracle.forward(q, k, v, codes, table)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-14)


def test_zero_table_is_vanilla_attention_rows_sum_to_one():
    q, k, v, codes, table, _ = _rand(5, 40, H=3, D=8, NB=6)
    table[:] = 0
    out, lse = oracle.forward(q, k, v, codes, table)
    for h in range(3):
        s = torch.tensor(q[:, h] @ k[:, h].T / math.sqrt(8))
        p = torch.softmax(s, dim=-1).numpy()
        np.testing.assert_allclose(out[:, h], p @ v[:, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[:, h], torch.logsumexp(s, -1).numpy(), rtol=1e-13)
    ones = np.ones_like(v)
    out1, _ = oracle.forward(q, k, ones, codes, table)
    np.testing.assert_allclose(out1, 1.0, rtol=0, atol=1e-13)
    table2 = np.random.default_rng(1).standard_normal(table.shape)
    out1, _ = oracle.forward(q, k, ones, codes, table2)       # rows of P sum to one with a bias too
    np.testing.assert_allclose(out1, 1.0, rtol=0, atol=1e-13)


def test_constant_shift_per_head():
    q, k, v, codes, table, do = _rand(11, 20, H=3, D=4, NB=5)
    c = np.array([3.0, -2.5, 0.75])
    a = oracle.backward(q, k, v, codes, table, do)
    b = oracle.backward(q, k, v, codes, table + c[:, None], do)
    for x, y in zip(a[:1] + a[2:], b[:1] + b[2:]):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b[1], a[1] + c[None, :], rtol=1e-12)


def test_single_node():
    q, k, v, codes, table, do = _rand(12, 1, H=3, D=4, NB=4)
    codes[:] = 0
    out, lse, dq, dk, dv, dtab = oracle.backward(q, k, v, codes, table, do)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, (q * k).sum(-1) / 2.0 + table[:, 0][None, :], rtol=1e-14)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dtab == 0)
    np.testing.assert_allclose(dv, do, rtol=0, atol=1e-15)


def test_zero_query_bucket_histogram():
    q, k, v, codes, table, _ = _rand(13, 30, H=2, D=4, NB=6)
    q[:] = 0
    out, lse = oracle.forward(q, k, v, codes, table)
    for h in range(2):
        for i in range(30):
            hist = np.bincount(codes[i], minlength=6)
            z = (hist * np.exp(table[h])).sum()
            p = np.exp(table[h][codes[i]]) / z
            np.testing.assert_allclose(out[i, h], p @ v[:, h], rtol=1e-12)
            np.testing.assert_allclose(lse[i, h], np.log(z), rtol=1e-13)


def test_strong_neighbour_bias_is_mean_aggregation():
    inp = small_case(50, 2, 4, 8, "f32", seed=4, avg_degree=3)
    codes = oracle.bfs_codes(inp.indptr, inp.indices, 8, range(50))
    table = np.zeros((2, 9))
    table[:, 1] = 50.0
    zeros = np.zeros((50, 2, 4))
    v = inp.v.value
    out, _ = oracle.forward(zeros, zeros, v, codes, table)
    deg = np.diff(inp.indptr)
    for i in range(50):
        if deg[i] == 0:
            continue
        nb = inp.indices[inp.indptr[i]:inp.indptr[i + 1]]
        np.testing.assert_allclose(out[i], v[nb].mean(axis=0), rtol=0, atol=1e-14 + 50 * np.exp(-50))
    table = np.zeros((2, 9))
    table[:, 0] = 50.0
    out, _ = oracle.forward(zeros, zeros, v, codes, table)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-14 + 200 * np.exp(-50))


def test_permutation_equivariance():
    q, k, v, codes, table, do = _rand(14, 25, H=2, D=4, NB=5)
    pi = np.random.default_rng(0).permutation(25)
    a = oracle.backward(q, k, v, codes, table, do)
    b = oracle.backward(q[pi], k[pi], v[pi], codes[pi][:, pi], table, do[pi])
    for x, y in zip(a[:5], b[:5]):
        np.testing.assert_allclose(x[pi], y, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(a[5], b[5], rtol=1e-10, atol=1e-12)


def test_finite_differences():
    N, H, D, NB = 12, 2, 4, 5
    q, k, v, codes, table, do = _rand(15, N, H, D, NB)
    _, _, dq, dk, dv, dtab = oracle.backward(q, k, v, codes, table, do)

    def loss(q_, k_, v_, t_):
        out, _ = oracle.forward(q_, k_, v_, codes, t_)
        return float((out * do).sum())

    eps = 1e-6
    rng = np.random.default_rng(0)
    for name, arr, grad in [("q", q, dq), ("k", k, dk), ("v", v, dv), ("t", table, dtab)]:
        flat = list(np.ndindex(arr.shape))
        picks = [flat[i] for i in rng.choice(len(flat), size=min(20, len(flat)), replace=False)]
        for ix in picks:
            args = {"q": q, "k": k, "v": v, "t": table}
            p = arr.copy()
            p[ix] += eps
            m = arr.copy()
            m[ix] -= eps
            args[name] = p
            lp = loss(args["q"], args["k"], args["v"], args["t"])
            args[name] = m
            lm = loss(args["q"], args["k"], args["v"], args["t"])
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[ix]) <= 1e-6 * max(1.0, abs(grad[ix])), (name, ix, fd, grad[ix])


def test_dtable_rows_sum_to_zero_and_absent_buckets_exact():
    q, k, v, codes, table, do = _rand(16, 40, H=3, D=4, NB=8)
    codes = np.minimum(codes, 4)       # buckets 5, 6, 7 never occur
    codes[3, 7] = 9                    # an out-of-range code clamps to NB-1
    _, _, _, _, _, dtab = oracle.backward(q, k, v, codes, table, do)
    np.testing.assert_allclose(dtab.sum(axis=1), 0, atol=1e-12)
    assert np.all(dtab[:, 5:7] == 0.0)
    assert np.all(dtab[:, 7] != 0.0)


def test_code_clamp_matches_explicit_last_bucket():
    q, k, v, codes, table, do = _rand(17, 16, H=2, D=4, NB=5)
    big = codes.copy()
    big[big == 4] = 200
    a = oracle.backward(q, k, v, codes, table, do)
    b = oracle.backward(q, k, v, big, table, do)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_row_blocks_and_pool_match_single_block():
    q, k, v, codes, table, do = _rand(18, 70, H=2, D=4, NB=6)
    ref = oracle.backward(q, k, v, codes, table, do)
    for block, workers in [(16, 1), (7, 3), (70, 1)]:
        got = oracle.full_backward(q, k, v, codes, table, do, block=block, workers=workers)
        for x, y in zip(ref, got):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)
    rows = np.array([0, 5, 69])
    got = oracle.full_backward(q, k, v, codes, table, do, block=2, rows=rows)
    np.testing.assert_allclose(got[0], ref[0][rows], rtol=1e-13)
    np.testing.assert_allclose(got[2], ref[2][rows], rtol=1e-13)


def test_key_split_merge_by_lse():
    """Fig. 4 of the MegaGraph pages: attention over key blocks (bias columns sliced to
    each block) merged by log-sum-exp equals unsplit attention."""
    q, k, v, codes, table, _ = _rand(19, 30, H=2, D=4, NB=5)
    out, lse = oracle.forward(q, k, v, codes, table)
    cuts = [0, 7, 19, 30]
    parts = [oracle.forward(q, k[a:b], v[a:b], codes[:, a:b], table) for a, b in zip(cuts, cuts[1:])]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    merged = sum(np.exp(p[1] - L)[..., None] * p[0] for p in parts)
    np.testing.assert_allclose(L, lse, rtol=1e-13)
    np.testing.assert_allclose(merged, out, rtol=1e-11, atol=1e-13)


def test_merge_running_equals_unsplit():
    """oracle.merge applied block after block (a running merge, as each key block
    arrives) gives unsplit attention; the order of the blocks does not matter."""
    q, k, v, codes, table, _ = _rand(31, 41, H=3, D=4, NB=6)
    out, lse = oracle.forward(q, k, v, codes, table)
    cuts = [0, 1, 16, 29, 41]
    parts = [oracle.forward(q, k[a:b], v[a:b], codes[:, a:b], table) for a, b in zip(cuts, cuts[1:])]
    for order in ([0, 1, 2, 3], [3, 1, 0, 2]):
        o, l = parts[order[0]]
        for i in order[1:]:
            o, l = oracle.merge(o, l, *parts[i])
        np.testing.assert_allclose(l, lse, rtol=1e-13)
        np.testing.assert_allclose(o, out, rtol=1e-11, atol=1e-13)


def test_merge_with_empty_side_is_identity():
    rng = np.random.default_rng(32)
    o = rng.standard_normal((5, 2, 8))
    l = rng.standard_normal((5, 2))
    empty_o = rng.standard_normal((5, 2, 8))
    empty_l = np.full((5, 2), -np.inf)
    for got in (oracle.merge(o, l, empty_o, empty_l), oracle.merge(empty_o, empty_l, o, l)):
        np.testing.assert_array_equal(got[0], o)
        np.testing.assert_array_equal(got[1], l)


def test_backward_block_sums_to_full_backward():
    """Key blocks x query blocks (virtual ranks holding query rows, key/value blocks
    visiting each): dq summed over key blocks, dk/dv summed over query blocks and
    dtable summed over both equal the unsplit backward."""
    q, k, v, codes, table, do = _rand(33, 37, H=2, D=4, NB=5)
    out, lse, dq, dk, dv, dtable = oracle.backward(q, k, v, codes, table, do)
    kc = [0, 11, 12, 37]
    qc = [0, 20, 37]
    gdq = np.zeros_like(dq)
    gdk = np.zeros_like(dk)
    gdv = np.zeros_like(dv)
    gdt = np.zeros_like(dtable)
    for r0, r1 in zip(qc, qc[1:]):
        for c0, c1 in zip(kc, kc[1:]):
            a, b, c, d = oracle.backward_block(q[r0:r1], k[c0:c1], v[c0:c1], codes[r0:r1, c0:c1], table,
                                               out[r0:r1], lse[r0:r1], do[r0:r1])
            gdq[r0:r1] += a
            gdk[c0:c1] += b
            gdv[c0:c1] += c
            gdt += d
    np.testing.assert_allclose(gdq, dq, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gdk, dk, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gdv, dv, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(gdt, dtable, rtol=1e-10, atol=1e-13)


def test_bf16_rounding_vs_torch():
    rng = np.random.default_rng(20)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, -3.5, 65504.0]])
    ref = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(x.astype(np.float32).astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    # ties go to even: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert oracle.round_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert oracle.round_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_stack_finite_differences_without_rounding():
    N, H, D, NB, L = 9, 2, 2, 4, 3
    rng = np.random.default_rng(21)
    hid = H * D
    x0 = rng.standard_normal((N, hid))
    w = rng.standard_normal((L, 3, hid, hid)) * 0.5
    tables = rng.standard_normal((L, H, NB)) * 0.5
    codes = rng.integers(0, NB, size=(N, N)).astype(np.uint8)
    do = rng.standard_normal((N, hid))
    r = oracle.stack_forward_backward(x0, w, tables, codes, do, rounding=False)

    def loss(x0_, w_, t_):
        rr = oracle.stack_forward_backward(x0_, w_, t_, codes, np.zeros_like(do), rounding=False)
        return float((rr["x"][-1] * do).sum())

    eps = 1e-6
    for name, arr, grad in [("x", x0, r["dx0"]), ("w", w, r["dw"]), ("t", tables, r["dtable"])]:
        for ix in [tuple(rng.integers(s) for s in arr.shape) for _ in range(8)]:
            args = {"x": x0, "w": w, "t": tables}
            p, m = arr.copy(), arr.copy()
            p[ix] += eps
            m[ix] -= eps
            args[name] = p
            lp = loss(args["x"], args["w"], args["t"])
            args[name] = m
            lm = loss(args["x"], args["w"], args["t"])
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad[ix]) <= 1e-6 * max(1.0, abs(grad[ix])), (name, ix, fd, grad[ix])


def test_projection_identity_weights_round_inputs():
    # W_t = I: Q = K = V = store(X), so each is X rounded to bfloat16 (or X itself)
    rng = np.random.default_rng(31)
    x = rng.standard_normal((11, 16))
    w = np.stack([np.eye(16)] * 3)
    for t in oracle.qkv_projection(x, w):
        np.testing.assert_array_equal(t, oracle.round_bf16(x))
    for t in oracle.qkv_projection(x, w, rounding=False):
        np.testing.assert_array_equal(t, x)


def test_projection_backward_finite_differences():
    # loss = sum_t <G_t, X W_t>: its gradients are dW_t = X^T G_t and dX = sum_t G_t W_t^T
    rng = np.random.default_rng(32)
    N, hid = 7, 8
    x = rng.standard_normal((N, hid))
    w = rng.standard_normal((3, hid, hid))
    g = rng.standard_normal((3, N, hid))
    dx, dw = oracle.qkv_projection_backward(x, w, g[0], g[1], g[2])

    def loss(x_, w_):
        return sum(float((g[t] * tt).sum()) for t, tt in enumerate(oracle.qkv_projection(x_, w_, rounding=False)))

    eps = 1e-6
    for name, arr, grad in [("x", x, dx), ("w", w, dw)]:
        for ix in [tuple(rng.integers(s) for s in arr.shape) for _ in range(10)]:
            p, m = arr.copy(), arr.copy()
            p[ix] += eps
            m[ix] -= eps
            fd = (loss(p, w) - loss(m, w)) / (2 * eps) if name == "x" else (loss(x, p) - loss(x, m)) / (2 * eps)
            assert abs(fd - grad[ix]) <= 1e-7 * max(1.0, abs(grad[ix])), (name, ix, fd, grad[ix])
