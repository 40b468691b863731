"""CPU float64 oracle for biased full-graph attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package
imports nothing from the product path; the two share only the seeded input
generators in ``workloads``.

What it computes (MegaGraph pages, abstract: attention scores plus a
topology-aware bias matrix per layer; Fig. 4 caption: the bias is sliced by
key columns to match each key/value block):

    B[h,i,j] = table[h, code(i,j)]                 code = clipped BFS distance
    S[h,i,j] = <q[i,h,:], k[j,h,:]> / sqrt(D) + B[h,i,j]
    P = softmax_j(S),  out[i,h,:] = sum_j P[h,i,j] v[j,h,:],  lse = log sum_j exp S

and its exact gradients. Everything is materialised per row block and
computed in float64; softmax is the two-pass definition (max, then exp/sum),
not an online update.

Pins (tests marked "not gpu") tie every function to something other than
itself: brute force on tiny inputs, scipy/torch library special cases,
closed forms, permutation equivariance and finite differences. The bf16
storage points of the multi-layer models (stack and full layer) are pinned
against torch autograd with torch's own bf16 conversion, and each point is
shown to change the result when left out. No function here is "parity
unpinned".
"""
from .spd import bfs_codes, bfs_codes_parallel, certify_codes, components  # noqa: F401
from .attention import forward, backward, backward_block, full_backward, merge  # noqa: F401
from .bf16 import round_bf16  # noqa: F401
from .stack import qkv_projection, qkv_projection_backward, stack_forward_backward  # noqa: F401
