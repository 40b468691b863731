"""GPU parity of the key-block steps (graph-aware context parallelism, MegaGraph pages,
Fig. 4 and its caption): virtual ranks hold query rows, key/value blocks with their
slice of bias columns visit every rank in ring order, partial results are merged by
log-sum-exp, and the backward of each block runs against the merged statistics.

Every (rank, block) step goes through the C ABI; the merged and summed results are
compared with the float64 oracle's unsplit forward/backward, and single blocks with
the oracle's block backward. Key cuts that are not multiples of 16 exercise the
unaligned code loads, cuts on multiples of 32 the aligned ones; one case uses a
non-symmetric code matrix so that the transposed codes are a separate input.
"""
import numpy as np
import pytest
import torch

import oracle
import graph_transformer_attention_amd as gta
from workloads import small_case, store
from workloads.tensors import normal

from gpu_util import check, dev, host64

pytestmark = pytest.mark.gpu


def _inputs(N, H, D, C, dtype, asym, seed=5):
    inp = small_case(N, H, D, C, dtype, seed=seed)
    if asym:
        rng = np.random.default_rng(seed + 1000)
        codes = rng.integers(0, C + 1, size=(N, N)).astype(np.uint8)
    else:
        codes = gta.spd_build(inp.indptr, inp.indices, N, C)
        np.testing.assert_array_equal(codes, oracle.bfs_codes(inp.indptr, inp.indices, C, range(N)))
    return inp, codes


def _ring(inp, codes, qcuts, kcuts):
    """Ring schedule on one GPU: rank r holds query rows [qcuts[r], qcuts[r+1]); at step t
    it receives key block (r - t) mod P and merges its partial result."""
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout)
    table = dev(inp.table)
    spd = torch.from_numpy(codes).cuda()
    spd_t = torch.from_numpy(np.ascontiguousarray(codes.T)).cuda()
    N, H, D = q.shape
    NB = table.shape[1]
    P = len(kcuts) - 1
    ranks = list(zip(qcuts, qcuts[1:]))
    blocks = list(zip(kcuts, kcuts[1:]))
    out = torch.empty((N, H, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((N, H), dtype=torch.float32, device="cuda")
    for r, (r0, r1) in enumerate(ranks):
        for t in range(P):
            c0, c1 = blocks[(r - t) % P]
            blk = (q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], table)
            if t == 0:
                gta.fwd_block(*blk, out=out[r0:r1], lse=lse[r0:r1])
            elif t % 2 == 1:   # separate merge call
                ob, lb = gta.fwd_block(*blk)
                gta.merge(out[r0:r1], lse[r0:r1], ob, lb, out[r0:r1], lse[r0:r1])
            else:              # merged by the block step itself
                gta.fwd_block(*blk, out=out[r0:r1], lse=lse[r0:r1], accumulate=True)
    # outputs start as NaN: each is overwritten on its first visit and added into after
    # (dq stays with its rank, dk/dv travel with their block, dtable is global)
    dq = torch.full((N, H, D), float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full_like(dq, float("nan"))
    dv = torch.full_like(dq, float("nan"))
    dtable = torch.full((H, NB), float("nan"), dtype=torch.float32, device="cuda")
    for r, (r0, r1) in enumerate(ranks):
        for t in range(P):
            c0, c1 = blocks[(r - t) % P]
            acc = ((gta.ACC_DQ if t > 0 else 0) | (gta.ACC_DKV if r > 0 else 0)
                   | (gta.ACC_DTABLE if (r, t) != (0, 0) else 0))
            gta.bwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], spd_t[c0:c1, r0:r1], table,
                          out[r0:r1], lse[r0:r1], do[r0:r1], dq[r0:r1], dk[c0:c1], dv[c0:c1], dtable,
                          accumulate=acc)
    torch.cuda.synchronize()
    return dict(out=host64(out), lse=host64(lse), dq=host64(dq), dk=host64(dk), dv=host64(dv),
                dtable=host64(dtable))


@pytest.mark.parametrize("N,H,D,C,dtype,asym,qcuts,kcuts", [
    # matrix-core paths (bf16, H = 8), unaligned and aligned cuts, ragged tails
    (300, 8, 8, 20, "bf16", False, [0, 150, 300], [0, 77, 200, 300]),
    (320, 8, 8, 20, "bf16", True, [0, 96, 320], [0, 128, 320]),
    (300, 8, 32, 30, "bf16", False, [0, 300], [0, 77, 200, 300]),
    (256, 8, 32, 30, "bf16", True, [0, 64, 256], [0, 32, 96, 256]),
    # vector-ALU paths
    (257, 4, 16, 12, "f32", True, [0, 100, 257], [0, 1, 130, 257]),
    (200, 8, 8, 20, "f32", False, [0, 200], [0, 64, 133, 200]),
    (90, 2, 64, 5, "bf16", True, [0, 46, 90], [0, 33, 90]),
    # blocks large enough that each block step splits its inner loop (2-3 splits)
    (1290, 8, 8, 20, "bf16", True, [0, 600, 1290], [0, 577, 1290]),
    (1200, 8, 32, 30, "bf16", False, [0, 1200], [0, 640, 1200]),
])
def test_ring_blocks_equal_oracle(N, H, D, C, dtype, asym, qcuts, kcuts):
    print(f"ring N={N} H={H} D={D} {dtype} asym={asym} qcuts={qcuts} kcuts={kcuts}", flush=True)
    inp, codes = _inputs(N, H, D, C, dtype, asym)
    got = _ring(inp, codes, qcuts, kcuts)
    ref = oracle.full_backward(inp.q.value, inp.k.value, inp.v.value, codes, inp.table.value, inp.dout.value)
    rep = {}
    for name, r in zip(["out", "lse", "dq", "dk", "dv", "dtable"], ref):
        check(name, got[name], r, dtype, rep)
    print("errors:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("N,D,dtype,r0,r1,c0,c1", [
    (300, 8, "bf16", 50, 290, 77, 200),
    (300, 32, "bf16", 0, 300, 0, 33),
    (300, 16, "f32", 10, 11, 3, 300),
    # one query row against one key, on each matrix-core path
    (300, 8, "bf16", 299, 300, 150, 151),
    (300, 32, "bf16", 0, 1, 299, 300),
])
def test_single_block_overwrite_equals_oracle_block(N, D, dtype, r0, r1, c0, c1):
    """One block without accumulation: out/lse of the block alone, and the block's
    backward shares against the merged (whole-graph) statistics."""
    print(f"block N={N} D={D} {dtype} rows=[{r0},{r1}) cols=[{c0},{c1})", flush=True)
    H = 8
    inp, codes = _inputs(N, H, D, 63, dtype, True, seed=9)   # the widest table, NB = 64
    Q, K, V, DO, T = (x.value for x in (inp.q, inp.k, inp.v, inp.dout, inp.table))
    out_all, lse_all = oracle.forward(Q[r0:r1], K, V, codes[r0:r1], T)
    ob_ref, lb_ref = oracle.forward(Q[r0:r1], K[c0:c1], V[c0:c1], codes[r0:r1, c0:c1], T)
    bref = oracle.backward_block(Q[r0:r1], K[c0:c1], V[c0:c1], codes[r0:r1, c0:c1], T, out_all, lse_all,
                                 DO[r0:r1])
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    spd = torch.from_numpy(codes).cuda()
    spd_t = torch.from_numpy(np.ascontiguousarray(codes.T)).cuda()
    ob, lb = gta.fwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], table)
    # the merged statistics come from the oracle here, so only the block step is tested
    out_m = torch.from_numpy(out_all.astype(np.float32)).cuda()
    lse_m = torch.from_numpy(lse_all.astype(np.float32)).cuda()
    fill = torch.full((r1 - r0, H, D), 7.0, device="cuda")
    dq, dk, dv, dt = gta.bwd_block(q[r0:r1], k[c0:c1], v[c0:c1], spd[r0:r1, c0:c1], spd_t[c0:c1, r0:r1],
                                   table, out_m, lse_m, do[r0:r1], dq=fill)
    torch.cuda.synchronize()
    rep = {}
    check("out", host64(ob), ob_ref, dtype, rep)
    check("lse", host64(lb), lb_ref, dtype, rep)
    for name, g, r in zip(["dq", "dk", "dv", "dtable"], (dq, dk, dv, dt), bref):
        check(name, host64(g), r, dtype, rep)
    print("errors:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


@pytest.mark.parametrize("Nk,NB", [(32788, 12), (32788, 33), (32800, 12)])
def test_block_with_many_keys_takes_two_key_sets(Nk, NB):
    """The one-pass backward gives each wave two 32-key sets once the key range fills 64
    workgroups of 512 keys (about 32256 keys); the sizes here reach that with only 100
    query rows, so the oracle stays cheap. Nk = 32788: the last workgroup's first wave has
    one live set, the others none, and the query tile is partial; Nk = 32800: that wave has
    both sets live. NB = 12 keeps every code in the private dtable bins; NB = 33 with codes
    up to 32 raises the flag, and the three-pass rerun overwrites every output. Codes are
    drawn directly (a block's slice needs no graph); the merged statistics are the block's
    own, so this is the whole backward of 100 queries against Nk keys. Queries are drawn
    N(0, 1/4): with N(0, 1) and only 100 of them, a few keys' dK and dV lie tens of times
    above their RMS, and half-precision operand rounding on those alone gives 2.1-2.8e-2 of
    the RMS (a float64 emulation of that rounding gives the GPU's 2.17e-2 for dK), past the
    bound; at variance 1/4 the emulation gives 3e-3 to 1e-2."""
    print(f"block Nq=100 Nk={Nk} NB={NB}", flush=True)
    Nq, H, D = 100, 8, 8
    rng = np.random.default_rng(np.random.SeedSequence([21, Nk, NB]))
    q = store(normal(rng, (Nq, H, D), 0.25), "bf16")
    k, v, do = (store(normal(rng, (n, H, D)), "bf16") for n in (Nk, Nk, Nq))
    table = store(normal(rng, (H, NB), 0.5), "f32")
    codes = rng.integers(0, NB, size=(Nq, Nk)).astype(np.uint8)
    Q, K, V, DO, T = (x.value for x in (q, k, v, do, table))
    out_all, lse_all = oracle.forward(Q, K, V, codes, T)
    bref = oracle.backward_block(Q, K, V, codes, T, out_all, lse_all, DO)
    spd = torch.from_numpy(codes).cuda()
    spd_t = torch.from_numpy(np.ascontiguousarray(codes.T)).cuda()
    out_m = torch.from_numpy(out_all.astype(np.float32)).cuda()
    lse_m = torch.from_numpy(lse_all.astype(np.float32)).cuda()
    got = gta.bwd_block(dev(q), dev(k), dev(v), spd, spd_t, dev(table), out_m, lse_m, dev(do))
    torch.cuda.synchronize()
    rep = {}
    for name, g, r in zip(["dq", "dk", "dv", "dtable"], got, bref):
        check(name, host64(g), r, "bf16", rep)
    print("errors:", {k: f"{v:.2e}" for k, v in rep.items()}, flush=True)


def test_accumulate_adds_into_given_values():
    """accumulate=True on buffers holding known values equals those values plus the
    overwrite-mode result, for every output."""
    N, H, D = 200, 8, 8
    inp, codes = _inputs(N, H, D, 20, "bf16", True, seed=4)
    q, k, v, do, table = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.dout), dev(inp.table)
    spd = torch.from_numpy(codes).cuda()
    spd_t = torch.from_numpy(np.ascontiguousarray(codes.T)).cuda()
    out, lse = gta.fwd(q, k, v, spd, table)
    args = (q[:150], k[40:], v[40:], spd[:150, 40:], spd_t[40:, :150], table, out[:150], lse[:150], do[:150])
    base = gta.bwd_block(*args)
    g = torch.Generator(device="cuda").manual_seed(0)
    init = [torch.randn(t.shape, generator=g, device="cuda") for t in base]
    got = gta.bwd_block(*args, *[t.clone() for t in init], accumulate=True)
    torch.cuda.synchronize()
    for name, a, b, c in zip(["dq", "dk", "dv", "dtable"], got, init, base):
        np.testing.assert_allclose(host64(a), host64(b) + host64(c), rtol=1e-6, atol=1e-6, err_msg=name)


def test_merge_kernel_equals_oracle():
    rng = np.random.default_rng(3)
    Nq, H, D = 1000, 8, 32
    oa, ob = (rng.standard_normal((Nq, H, D)).astype(np.float32) for _ in range(2))
    la, lb = (rng.standard_normal((Nq, H)).astype(np.float32) * 30 for _ in range(2))
    la[:5] = -np.inf           # empty first side
    lb[5:9] = -np.inf          # empty second side
    ref_o, ref_l = oracle.merge(oa, la, ob, lb)
    t = [torch.from_numpy(x).cuda() for x in (oa, la, ob, lb)]
    out, lse = gta.merge(*t)
    # in place, into the first side (a running merge)
    gta.merge(t[0], t[1], t[2], t[3], t[0], t[1])
    torch.cuda.synchronize()
    for o, l in ((out, lse), (t[0], t[1])):
        np.testing.assert_allclose(host64(o), ref_o, rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(host64(l), ref_l, rtol=2e-6, atol=2e-6)
