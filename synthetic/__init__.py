"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This package holds no arithmetic of the decoding method. It only produces
inputs: model shapes and seeds (``configs``), weight tensors (``weights``),
prompt token ids (``prompts``) and the Gumbel(0,1) noise rows that sampling
consumes (``noise``). Every value is a pure function of (seed, stream, index),
computed with integer hashing and a fixed float64 table, so the same call gives
bit-identical tensors on the CPU and on a GPU device.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
