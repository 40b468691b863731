"""The GPU builder of the clipped hop-distance codes against the oracle's breadth-first
search (bit for bit) and against the host builder, from one node to the full 65536-node
graph (whose sources are searched in two groups)."""
import hashlib

import numpy as np
import pytest
import torch

import oracle
import graph_transformer_attention_amd as gta
from workloads import graphs, make_inputs, small_case

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(7)
    out = {}
    for name, N, C, family in [("single", 1, 5, "er"), ("pair", 2, 3, "er"), ("er65", 65, 6, "er"),
                               ("path130", 130, 20, "path"), ("path-clip", 130, 4, "path"),
                               ("empty", 70, 3, "empty"), ("er300-c1", 300, 1, "er"), ("er300-c2", 300, 2, "er")]:
        inp = small_case(N, 1, 8, C, "f32", seed=3, family=family)
        out[name] = (inp.indptr, inp.indices, N, C)
    # several components of different sizes, one of them an isolated node
    isolated = (np.zeros(2, np.int64), np.zeros(0, np.int32))
    parts = [graphs.erdos_renyi(40, 3.0, rng), isolated, graphs.erdos_renyi(57, 3.0, rng),
             graphs.erdos_renyi(33, 3.0, rng)]
    ip, ix, base = [0], [], 0
    for p_indptr, p_indices in parts:
        n = len(p_indptr) - 1
        ip.extend((p_indptr[1:] + len(ix)).tolist())
        ix.extend((p_indices + base).tolist())
        base += n
    out["components"] = (np.array(ip, np.int64), np.array(ix, np.int32), base, 9)
    return out


CASES = _cases()


@pytest.mark.parametrize("name", sorted(CASES))
def test_device_codes_equal_oracle(name):
    indptr, indices, N, C = CASES[name]
    print(f"spd device {name}: N={N} C={C}", flush=True)
    ref = oracle.bfs_codes(indptr, indices, C, range(N))
    got = gta.spd_build_device(indptr, indices, N, C)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.cpu().numpy(), ref)
    np.testing.assert_array_equal(gta.spd_build(indptr, indices, N, C), ref)


@pytest.mark.parametrize("number", [4, 5])
def test_device_codes_full_size(number):
    """ba32768 and sbm65536: the device codes equal the host builder's everywhere, and
    their digest equals the one stored from the oracle's search."""
    import os
    inp = make_inputs(number)
    w = inp.workload
    g = np.load(os.path.join(os.path.dirname(__file__), "golden", f"{w.name}.npz"), allow_pickle=False)
    print(f"spd device full size {w.name}: N={w.N} C={w.C}", flush=True)
    dev = gta.spd_build_device(inp.indptr, inp.indices, w.N, w.C)
    host = gta.spd_build(inp.indptr, inp.indices, w.N, w.C)
    assert hashlib.sha256(host.tobytes()).hexdigest() == str(g["codes_sha256"])
    assert torch.equal(dev, torch.from_numpy(host).cuda())
