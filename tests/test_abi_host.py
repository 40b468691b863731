"""The C-ABI library on the host (no GPU): it loads, exports every declared symbol,
rejects bad arguments before anything is enqueued, and its native distance-code
builder agrees bit for bit with the oracle's breadth-first search."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import graph_transformer_attention_amd as gta
from workloads import graphs, make_inputs, small_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gt_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gt_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"gt_attn_fwd", "gt_attn_bwd", "gt_attn_bwd_workspace_bytes", "gt_spd_build",
            "gt_last_error", "gt_version"} <= set(names)
    L = gta.lib()
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in gta.version()


P = 0x10000  # a 16-byte-aligned stand-in address; these calls never reach the GPU


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, spd=P, table=P, out=P, lse=P, N=100, H=8, D=8, NB=33, dt=1)
    a.update(kw)
    if "ws" in a:  # the workspace variant
        return gta.lib().gt_attn_fwd_ws(a["q"], a["k"], a["v"], a["spd"], a["table"], a["out"], a["lse"], a["ws"],
                                        a["wsb"], a["N"], a["H"], a["D"], a["NB"], a["dt"], None)
    return gta.lib().gt_attn_fwd(a["q"], a["k"], a["v"], a["spd"], a["table"], a["out"], a["lse"],
                                 a["N"], a["H"], a["D"], a["NB"], a["dt"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), gta.GT_EINVAL, "q is null"),
    (dict(spd=None), gta.GT_EINVAL, "spd is null"),
    (dict(lse=P + 4), gta.GT_EINVAL, "aligned"),
    (dict(N=0), gta.GT_EINVAL, "N="),
    (dict(N=1 << 31), gta.GT_EINVAL, "N="),
    (dict(H=0), gta.GT_EINVAL, "H="),
    (dict(NB=1), gta.GT_EINVAL, "NB="),
    (dict(NB=256), gta.GT_EINVAL, "NB="),
    (dict(dt=7), gta.GT_EINVAL, "dtype"),
    (dict(D=12), gta.GT_EUNSUPPORTED, "D=12"),
    (dict(H=65), gta.GT_EUNSUPPORTED, "H=65"),
    (dict(H=16, D=64), gta.GT_EUNSUPPORTED, "H*D"),
    (dict(NB=100), gta.GT_EUNSUPPORTED, "NB=100"),
])
def test_fwd_argument_errors(kw, code, msg):
    assert _fwd(**kw) == code
    assert msg in gta.last_error()


def test_bwd_argument_errors():
    L = gta.lib()
    N, H, D, NB = 1000, 8, 8, 33
    need = L.gt_attn_bwd_workspace_bytes(N, H, D, NB, 1)
    assert need >= N * H * 4
    assert L.gt_attn_bwd_workspace_bytes(0, H, D, NB, 1) == 0
    assert L.gt_attn_bwd_workspace_bytes(N, H, 12, NB, 1) == 0

    def call(ws=P, wsb=need, dout=P, dtable=P, **kw):
        return L.gt_attn_bwd(P, P, P, P, P, P, P, P, dout, P, P, P, dtable, ws, wsb,
                             kw.get("N", N), H, D, NB, 1, None)
    assert call(wsb=need - 1) == gta.GT_EINVAL and "workspace_bytes" in gta.last_error()
    assert call(ws=None) == gta.GT_EINVAL
    assert call(ws=P + 16) == gta.GT_EINVAL and "256-byte" in gta.last_error()
    assert call(dout=None) == gta.GT_EINVAL and "dout" in gta.last_error()
    assert call(dtable=P + 8) == gta.GT_EINVAL
    assert call(N=-5) == gta.GT_EINVAL


def test_split_workspaces():
    """Launches whose workgroups would not fill whole rounds split the inner loop: the
    forward then needs a workspace for its partial results, and the backward's grows.
    At 32768 nodes (D = 8) the forward's 1024 workgroups would be one full round, whose tail
    the model charges, so it splits 4 ways (4 rounds of 256 tiles)."""
    L = gta.lib()
    rows = 32768 * 8
    assert L.gt_attn_fwd_workspace_bytes(32768, 8, 8, 33, 1) == 4 * (rows * 8 * 4 + rows * 4)
    # D = 32, 65536 nodes: 2048 workgroups at 3 per CU would leave the third round two thirds
    # full; three key splits (8 rounds of 683 tiles) cost less than 3 rounds of 2048 tiles
    rows = 65536 * 8
    assert L.gt_attn_fwd_workspace_bytes(65536, 8, 32, 49, 1) == 3 * (rows * 32 * 4 + rows * 4)
    # 100000 nodes: 3128 workgroups would leave the last wave of resident workgroups 5% full; two splits do better
    assert L.gt_attn_fwd_workspace_bytes(100000, 8, 8, 33, 1) > 0
    assert L.gt_attn_fwd_workspace_bytes(6800, 8, 8, 33, 0) == 0         # vector-ALU path: no split
    need = L.gt_attn_fwd_workspace_bytes(6800, 8, 8, 33, 1)
    assert need >= 2 * 6800 * 8 * 8 * 4
    assert _fwd(N=6800, ws=None, wsb=0) == gta.GT_EINVAL and "workspace is null" in gta.last_error()
    assert _fwd(N=6800, ws=P, wsb=need - 1) == gta.GT_EINVAL and "workspace_bytes" in gta.last_error()
    assert L.gt_attn_fwd_block_workspace_bytes(4096, 4096, 8, 32, 49, 1) >= 2 * 4096 * 8 * 32 * 4
    # too few keys to split: one partial result's room (a block step may merge into out/lse)
    assert L.gt_attn_fwd_block_workspace_bytes(4096, 200, 8, 8, 33, 1) == 4096 * 8 * 8 * 4 + 4096 * 8 * 4
    # the small graph's backward holds split partial gradients on top of the unsplit needs;
    # at D = 8 (bf16, H = 8) the one-pass backward adds one dQ partial [N, H, D] per 512-key workgroup
    small, big = L.gt_attn_bwd_workspace_bytes(6800, 8, 8, 33, 1), L.gt_attn_bwd_workspace_bytes(32768, 8, 8, 33, 1)
    dq_partials = (32768 // 512) * 32768 * 8 * 8 * 4
    assert small > 3 * 6800 * 8 * 8 * 4 and dq_partials < big < dq_partials + 40 * 32768 * 8 * 8 * 4
    # the float32 path has no one-pass backward
    assert L.gt_attn_bwd_workspace_bytes(32768, 8, 8, 33, 0) < 40 * 32768 * 8 * 8 * 4


def test_workspace_query_keeps_last_error():
    _fwd(q=None)
    before = gta.last_error()
    gta.lib().gt_attn_bwd_workspace_bytes(0, 8, 8, 33, 1)
    assert gta.last_error() == before


def _oracle_all(indptr, indices, C):
    n = len(indptr) - 1
    return oracle.bfs_codes(indptr, indices, C, range(n))


@pytest.mark.parametrize("case", ["er1", "path", "components", "single", "empty", "ragged"])
def test_spd_build_matches_oracle_small(case):
    if case == "er1":
        inp = make_inputs(1)
        ip, ix, C = inp.indptr, inp.indices, inp.workload.C
    elif case == "path":
        ip, ix = graphs.path_graph(150)
        C = 30
    elif case == "components":
        a = graphs.path_graph(70)
        b = graphs.erdos_renyi(90, 3.0, np.random.default_rng(1))
        u = np.concatenate([np.repeat(np.arange(70), np.diff(a[0])), 70 + np.repeat(np.arange(90), np.diff(b[0]))])
        v = np.concatenate([a[1], 70 + b[1]])
        ip, ix = graphs.csr_from_edges(160, u, v)
        C = 5
    elif case == "single":
        ip, ix, C = np.array([0, 0], np.int64), np.zeros(0, np.int32), 3
    elif case == "empty":
        ip, ix, C = np.zeros(11, np.int64), np.zeros(0, np.int32), 2
    else:
        inp = small_case(131, 1, 8, 4, "f32", seed=2, avg_degree=2.5)
        ip, ix, C = inp.indptr, inp.indices, 4
    n = len(ip) - 1
    ref = _oracle_all(ip, ix, C)
    for nt in (1, 3):
        got = gta.spd_build(ip, ix, n, C, nthreads=nt)
        np.testing.assert_array_equal(got, ref)


def test_spd_build_c1_small_clip():
    inp = make_inputs(1)
    for C in (1, 2, 3):
        ref = _oracle_all(inp.indptr, inp.indices, C)
        got = gta.spd_build(inp.indptr, inp.indices, 256, C)
        np.testing.assert_array_equal(got, ref)


def test_spd_build_rgg4096_sampled_rows_and_certificate():
    inp = make_inputs(2)
    w = inp.workload
    got = gta.spd_build(inp.indptr, inp.indices, w.N, w.C)
    rows = np.random.default_rng(5).choice(w.N, 48, replace=False)
    ref = oracle.bfs_codes(inp.indptr, inp.indices, w.C, rows)
    np.testing.assert_array_equal(got[rows], ref)
    assert oracle.certify_codes(inp.indptr, inp.indices, w.C, np.arange(w.N), got)
    # unreachable pairs exist in this graph (two components)
    assert (got == w.C).any()


@pytest.mark.slow
def test_spd_build_ba32768_full_certificate():
    inp = make_inputs(4)
    w = inp.workload
    got = gta.spd_build(inp.indptr, inp.indices, w.N, w.C)
    ref = oracle.bfs_codes(inp.indptr, inp.indices, w.C, inp.rows[:40])
    np.testing.assert_array_equal(got[inp.rows[:40]], ref)
    src = np.arange(0, w.N, 8)   # certificate on every 8th row keeps this under a minute
    assert oracle.certify_codes(inp.indptr, inp.indices, w.C, src, got[src])


@pytest.mark.parametrize("bad", ["asym", "range", "order", "C0", "C255"])
def test_spd_build_rejects_malformed(bad):
    ip, ix = graphs.path_graph(10)
    C = 4
    if bad == "asym":
        ix = ix.copy()
        ix[0] = 5            # 0 -> 5 without 5 -> 0
    elif bad == "range":
        ix = ix.copy()
        ix[3] = 10
    elif bad == "order":
        ip = ip.copy()
        ip[4] = ip[5] + 1
    elif bad == "C0":
        C = 0
    else:
        C = 255
    with pytest.raises(gta.GtError) as e:
        gta.spd_build(ip, ix, 10, C)
    assert e.value.code == gta.GT_EINVAL


def test_projection_and_stack_argument_errors():
    L = gta.lib()
    assert L.gt_qkv_fwd(P, P, P, P, P, 100, 12, 1, None) == gta.GT_EINVAL and "hid=12" in gta.last_error()
    assert L.gt_qkv_fwd(P, P, P, P, P, 100, 1024, 1, None) == gta.GT_EINVAL
    assert L.gt_qkv_fwd(None, P, P, P, P, 100, 64, 1, None) == gta.GT_EINVAL and "x is null" in gta.last_error()
    assert L.gt_qkv_fwd(P, P, P, P, P, 0, 64, 1, None) == gta.GT_EINVAL
    assert L.gt_qkv_fwd(P, P, P, P, P, 100, 64, 5, None) == gta.GT_EINVAL
    need = L.gt_qkv_bwd_workspace_bytes(6800, 64)
    assert need >= 27 * 3 * 64 * 64 * 4 and L.gt_qkv_bwd_workspace_bytes(6800, 63) == 0
    assert L.gt_qkv_bwd(P, P, P, P, P, P, P, P, need - 1, 6800, 64, 1, None) == gta.GT_EINVAL
    assert "workspace_bytes" in gta.last_error()
    assert L.gt_qkv_bwd(P, P, P, P, P, P, P, P + 16, need, 6800, 64, 1, None) == gta.GT_EINVAL
    assert L.gt_store(P, P, -1, 1, None) == gta.GT_EINVAL
    assert L.gt_store(None, None, 0, 1, None) == gta.GT_OK
    assert L.gt_store(P, P + 2, 10, 1, None) == gta.GT_EINVAL and "aligned" in gta.last_error()
    sw = L.gt_stack_workspace_bytes(6800, 16, 8, 8, 33, 1)
    assert sw > 16 * 6800 * 64 * (3 * 2 + 4 + 2) and L.gt_stack_workspace_bytes(6800, 0, 8, 8, 33, 1) == 0

    def stack(L_=16, ws=P, wsb=sw, **kw):
        a = dict(x0=P, dout=P)
        a.update(kw)
        return L.gt_stack_fwd_bwd(a["x0"], P, P, P, P, a["dout"], P, P, P, P, ws, wsb, 6800, L_, 8, 8, 33, 1,
                                  None)
    assert stack(L_=0) == gta.GT_EINVAL and "L=0" in gta.last_error()
    assert stack(wsb=sw - 1) == gta.GT_EINVAL
    assert stack(x0=None) == gta.GT_EINVAL and "x0" in gta.last_error()
    assert stack(dout=P + 8) == gta.GT_EINVAL


def test_block_argument_errors():
    """Key-block steps: row strides, counts, the accumulate flag and the workspace are
    checked before anything is enqueued; code pointers may have any alignment."""
    L = gta.lib()
    Nq, Nk, H, D, NB = 700, 300, 8, 8, 33

    fwb = L.gt_attn_fwd_block_workspace_bytes(Nq, Nk, H, D, NB, 1)

    def fwd(ld=1000, Nq_=Nq, Nk_=Nk, spd=P + 3, q=P, acc=0):
        return L.gt_attn_fwd_block(q, P, P, spd, ld, P, P, P, P, fwb, Nq_, Nk_, H, D, NB, 1, acc, None)
    assert fwd(ld=Nk - 1) == gta.GT_EINVAL and "ld=299" in gta.last_error()
    assert fwd(Nk_=0) == gta.GT_EINVAL and "Nk=0" in gta.last_error()
    assert fwd(Nq_=0) == gta.GT_EINVAL and "Nq=0" in gta.last_error()
    assert fwd(spd=None) == gta.GT_EINVAL and "spd is null" in gta.last_error()
    assert fwd(q=P + 2) == gta.GT_EINVAL and "aligned" in gta.last_error()
    assert fwd(acc=2) == gta.GT_EINVAL and "accumulate" in gta.last_error()

    need = L.gt_attn_bwd_block_workspace_bytes(Nq, Nk, H, D, NB, 1)
    assert need >= Nq * H * 4
    assert L.gt_attn_bwd_block_workspace_bytes(Nq, 0, H, D, NB, 1) == 0
    # a square block needs exactly the whole-graph backward's workspace
    assert L.gt_attn_bwd_block_workspace_bytes(Nq, Nq, H, D, NB, 1) == L.gt_attn_bwd_workspace_bytes(Nq, H, D, NB, 1)

    def bwd(ld=1000, ldt=1000, acc=0, wsb=need, spdt=P + 5):
        return L.gt_attn_bwd_block(P, P, P, P + 1, ld, spdt, ldt, P, P, P, P, P, P, P, P, P, wsb,
                                   Nq, Nk, H, D, NB, 1, acc, None)
    assert bwd(ldt=Nq - 1) == gta.GT_EINVAL and "ld_t=699" in gta.last_error()
    assert bwd(ld=10) == gta.GT_EINVAL and "ld=10" in gta.last_error()
    assert bwd(acc=8) == gta.GT_EINVAL and "accumulate" in gta.last_error()
    assert bwd(acc=-1) == gta.GT_EINVAL
    assert bwd(wsb=need - 1) == gta.GT_EINVAL and "workspace_bytes" in gta.last_error()
    assert bwd(spdt=None) == gta.GT_EINVAL and "spd_t is null" in gta.last_error()

    def merge(Nq_=Nq, H_=H, D_=D, out=P):
        return L.gt_attn_merge(P, P, P, P, out, P, Nq_, H_, D_, None)
    assert merge(Nq_=0) == gta.GT_EINVAL
    assert merge(D_=12) == gta.GT_EUNSUPPORTED
    assert merge(H_=0) == gta.GT_EINVAL
    assert merge(out=None) == gta.GT_EINVAL and "out is null" in gta.last_error()
    assert gta.kernel_names()[9] == "merge"


def test_model_argument_errors():
    L = gta.lib()
    assert L.gt_model_param_count(64, 64) == 24960
    assert L.gt_model_param_count(32, 32) == 0
    need = L.gt_model_workspace_bytes(6800, 16, 8, 8, 33, 1)
    assert need > 16 * 6800 * 64 * 4 * 5
    assert L.gt_model_workspace_bytes(6800, 16, 8, 16, 33, 1) == 0   # hidden 128: no kernels
    assert L.gt_model_workspace_bytes(6800, 0, 8, 8, 33, 1) == 0

    def call(L_=16, H=8, D=8, wsb=need, x0=P):
        return L.gt_model_fwd_bwd(x0, P, P, P, P, P, P, P, P, P, P, wsb, 6800, L_, H, D, 33, 1, None)
    assert call(H=8, D=16) == gta.GT_EUNSUPPORTED and "64" in gta.last_error()
    assert call(L_=0) == gta.GT_EINVAL and "L=0" in gta.last_error()
    assert call(wsb=need - 1) == gta.GT_EINVAL and "workspace_bytes" in gta.last_error()
    assert call(x0=None) == gta.GT_EINVAL and "x0" in gta.last_error()


def test_last_error_is_per_thread_and_calls_are_reentrant():
    """gt_last_error() reports the calling thread's own last failure, and the host entry
    points run concurrently from several threads with the results of a serial run."""
    import threading
    inp = small_case(300, 1, 8, 6, "f32", seed=4, avg_degree=3.0)
    ref = gta.spd_build(inp.indptr, inp.indices, 300, 6, nthreads=1)
    barrier = threading.Barrier(4)
    results = {}

    def worker(k):
        barrier.wait()
        if k % 2 == 0:
            rc = _fwd(N=0) if k == 0 else _fwd(D=12)
            msg = gta.last_error()
        else:
            rc, msg = 0, None
        got = gta.spd_build(inp.indptr, inp.indices, 300, 6, nthreads=2)
        # a successful call leaves this thread's message as it was
        results[k] = (rc, msg, gta.last_error() if k % 2 == 0 else None, np.array_equal(got, ref))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert results[0][0] == gta.GT_EINVAL and "N=" in results[0][1] and results[0][2] == results[0][1]
    assert results[2][0] == gta.GT_EUNSUPPORTED and "D=12" in results[2][1] and results[2][2] == results[2][1]
    assert all(r[3] for r in results.values())
