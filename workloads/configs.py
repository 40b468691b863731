"""The synthetic workloads of biased full-graph attention and their seeded inputs.

Each workload fixes a graph family, the SPD clip C (codes 0..C-1 for reachable
pairs, C for unreachable ones, so the bias table has NB = C + 1 columns), the
head count H, the head dimension D and the storage type of Q/K/V/dOut.
Seeds: workload number k uses ``SeedSequence(k)`` spawned into eight streams,
in the order graph, q, k, v, dout, table, weights, samples.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import graphs
from .tensors import Stored, normal, store


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    family: str            # "er", "rgg", "ba", "sbm"
    N: int
    C: int
    H: int
    D: int
    dtype: str             # storage type of q, k, v, out, dout
    layers: int = 1        # >1: stacked layers with Q/K/V projections
    sample_rows: int = 0   # 0: compare every row against the oracle
    graph_args: dict = field(default_factory=dict)
    model: str = "attn"    # "attn": attention (+ projections when stacked); "gt": full layers

    @property
    def NB(self) -> int:
        return self.C + 1

    @property
    def hidden(self) -> int:
        return self.H * self.D

    def describe(self) -> str:
        g = ", ".join(f"{k}={v}" for k, v in self.graph_args.items())
        return (f"{self.name}: {self.family}({g}) N={self.N} C={self.C} NB={self.NB} "
                f"H={self.H} D={self.D} {self.dtype} layers={self.layers}")


WORKLOADS = {
    1: Workload(1, "er256-f32", "er", 256, 20, 8, 8, "f32", graph_args=dict(avg_degree=8)),
    2: Workload(2, "rgg4096-bf16", "rgg", 4096, 24, 8, 8, "bf16", graph_args=dict(avg_degree=10)),
    3: Workload(3, "ba6800-stack16-bf16", "ba", 6800, 32, 8, 8, "bf16", layers=16,
                graph_args=dict(m=4)),
    4: Workload(4, "ba32768-bf16", "ba", 32768, 32, 8, 8, "bf16", sample_rows=512,
                graph_args=dict(m=4)),
    5: Workload(5, "sbm65536-d32-bf16", "sbm", 65536, 48, 8, 32, "bf16", sample_rows=256,
                graph_args=dict(n_blocks=64, block_size=1024, p_in=0.01, p_out=2e-5)),
    6: Workload(6, "gt16-ba6800-bf16", "ba", 6800, 32, 8, 8, "bf16", layers=16, graph_args=dict(m=4),
                model="gt"),
}

_STREAMS = ("graph", "q", "k", "v", "dout", "table", "weights", "samples")


def streams(number: int) -> dict:
    ss = np.random.SeedSequence(number).spawn(len(_STREAMS))
    return {name: np.random.default_rng(s) for name, s in zip(_STREAMS, ss)}


def make_graph(w: Workload, rng: np.random.Generator):
    a = w.graph_args
    if w.family == "er":
        return graphs.erdos_renyi(w.N, a["avg_degree"], rng)
    if w.family == "rgg":
        return graphs.random_geometric(w.N, a["avg_degree"], rng)
    if w.family == "ba":
        return graphs.barabasi_albert(w.N, a["m"], rng)
    if w.family == "sbm":
        return graphs.stochastic_block(a["n_blocks"], a["block_size"], a["p_in"], a["p_out"], rng)
    raise ValueError(w.family)


@dataclass
class Inputs:
    workload: Workload
    indptr: np.ndarray
    indices: np.ndarray
    q: Stored = None
    k: Stored = None
    v: Stored = None
    dout: Stored = None
    table: Stored = None          # [H, NB] float32  (single layer) or [L, H, NB]
    x0: Stored = None             # stacked workload: node features [N, hidden]
    w_qkv: Stored = None          # stacked workload: [L, 3, hidden, hidden]
    gt_params: dict = None        # full layers: name -> Stored [L, ...] float32 (see gt_params)
    rows: np.ndarray = None       # sampled query rows (sorted, unique)


def make_inputs(w: Workload | int) -> Inputs:
    if isinstance(w, int):
        w = WORKLOADS[w]
    rs = streams(w.number)
    indptr, indices = make_graph(w, rs["graph"])
    inp = Inputs(w, indptr, indices)
    N, H, D, NB = w.N, w.H, w.D, w.NB
    if w.model == "gt":
        L, hid = w.layers, w.hidden
        inp.x0 = store(normal(rs["q"], (N, hid)), "f32")
        inp.dout = store(normal(rs["dout"], (N, hid)), "f32")
        inp.table = store(normal(rs["table"], (L, H, NB), 0.5), "f32")
        inp.gt_params = gt_params(rs["weights"], L, hid)
    elif w.layers == 1:
        inp.q = store(normal(rs["q"], (N, H, D)), w.dtype)
        inp.k = store(normal(rs["k"], (N, H, D)), w.dtype)
        inp.v = store(normal(rs["v"], (N, H, D)), w.dtype)
        inp.dout = store(normal(rs["dout"], (N, H, D)), w.dtype)
        inp.table = store(normal(rs["table"], (H, NB), 0.5), "f32")
    else:
        L, hid = w.layers, w.hidden
        inp.x0 = store(normal(rs["q"], (N, hid)), w.dtype)
        inp.dout = store(normal(rs["dout"], (N, hid)), w.dtype)
        inp.table = store(normal(rs["table"], (L, H, NB), 0.5), "f32")
        inp.w_qkv = store(normal(rs["weights"], (L, 3, hid, hid), 1.0 / hid), w.dtype)
    inp.rows = sample_rows(w, indptr, rs["samples"])
    return inp


def gt_params(rng: np.random.Generator, L: int, hid: int, ffn: int | None = None) -> dict:
    """Named float32 parameters of L full layers: norm gains near 1, norm shifts and
    biases near 0 (variance 0.01), weight matrices with variance 1/fan-in. Matrices are
    [L, fan_in, fan_out]."""
    ffn = hid if ffn is None else ffn
    shapes = (("g1", (hid,)), ("b1", (hid,)), ("wq", (hid, hid)), ("wk", (hid, hid)), ("wv", (hid, hid)),
              ("wo", (hid, hid)), ("g2", (hid,)), ("b2", (hid,)), ("w1", (hid, ffn)), ("c1", (ffn,)),
              ("w2", (ffn, hid)), ("c2", (hid,)))
    out = {}
    for name, shape in shapes:
        if len(shape) == 2:
            x = normal(rng, (L,) + shape, 1.0 / shape[0])
        elif name in ("g1", "g2"):
            x = 1.0 + normal(rng, (L,) + shape, 0.01)
        else:
            x = normal(rng, (L,) + shape, 0.01)
        out[name] = store(x, "f32")
    return out


def sample_rows(w: Workload, indptr: np.ndarray, rng: np.random.Generator) -> np.ndarray:
    """Query rows checked against the oracle: all rows, or a uniform sample without
    replacement plus rows 0 and N-1 and the highest- and lowest-degree nodes."""
    if w.sample_rows == 0:
        return np.arange(w.N, dtype=np.int64)
    deg = graphs.degrees(indptr)
    extra = [0, w.N - 1, int(np.argmax(deg)), int(np.argmin(deg))]
    pick = rng.choice(w.N, size=w.sample_rows, replace=False)
    return np.unique(np.concatenate([pick, extra])).astype(np.int64)


def small_case(N: int, H: int, D: int, C: int, dtype: str, seed: int, family: str = "er",
               avg_degree: float = 4.0, table_variance: float = 0.5) -> Inputs:
    """A small seeded case of any shape (edge cases, ragged tiles)."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, N, H, D, C]))
    w = Workload(0, f"case-N{N}-H{H}-D{D}-C{C}-{dtype}", family, N, C, H, D, dtype,
                 graph_args=dict(avg_degree=avg_degree))
    if N == 1:
        indptr, indices = np.zeros(2, np.int64), np.zeros(0, np.int32)
    elif family == "er":
        indptr, indices = graphs.erdos_renyi(N, min(avg_degree, N - 1), rng)
    elif family == "path":
        indptr, indices = graphs.path_graph(N)
    elif family == "empty":
        indptr, indices = np.zeros(N + 1, np.int64), np.zeros(0, np.int32)
    else:
        raise ValueError(family)
    inp = Inputs(w, indptr, indices)
    inp.q = store(normal(rng, (N, H, D)), dtype)
    inp.k = store(normal(rng, (N, H, D)), dtype)
    inp.v = store(normal(rng, (N, H, D)), dtype)
    inp.dout = store(normal(rng, (N, H, D)), dtype)
    inp.table = store(normal(rng, (H, C + 1), table_variance), "f32")
    inp.rows = np.arange(N, dtype=np.int64)
    return inp
