"""Seeded synthetic inputs for biased full-graph attention: graphs (CSR) and tensors.

This package holds no part of the method's arithmetic. It is the only code
shared by the oracle side and the HIP side.
"""
from .configs import WORKLOADS, Workload, Inputs, make_inputs, small_case, sample_rows  # noqa: F401
from .tensors import Stored, store, f32_to_bf16_bits, bf16_bits_to_f64  # noqa: F401
from . import graphs  # noqa: F401
