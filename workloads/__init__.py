"""Seeded synthetic workloads shared by the tests, the benchmark and the oracle.

This package holds shapes, seeds and random draws only — none of the
method's arithmetic (no RoPE, no permute, no softmax).  Both the HIP path
and the oracle consume the exact host arrays produced here.
"""
from .configs import WORKLOADS, Workload, by_name, video_grid  # noqa: F401
from .inputs import make_inputs, sample_rows  # noqa: F401
