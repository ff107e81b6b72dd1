"""Seeded synthetic inputs for shared-KV sparse flash MLA attention.

This package builds host-side numpy arrays (plus a parameter dict) for the
workloads the attention path is measured and checked on.  It is shared by the
CPU oracle, the GPU tests and the benchmark, and for that reason it holds none
of the attention arithmetic: no visibility rule, no index resolution, no
decoding of stored rows, no softmax.  What it does hold:

* seeded draws (numpy PCG64, one spawned child stream per tensor),
* fp32 -> bf16 rounding (round-to-nearest-even) of the drawn values,
* the packed-KV *writer* (per-128-tile INT8 / FP8-E4M3 quantiser and the
  656/528-byte row packer), which sits on the KV-cache writer side and is not
  part of the attention path that reads those rows,
* the workload recipes (shapes, lengths, block tables, index draws).

Index ranges in the recipes are written with each workload's own numbers
(e.g. "draw 512 of the 8192 compressed rows"), not derived from a mask rule.
"""

from .problem import Problem, bf16_bits
from .workloads import WORKLOADS, index_replicas, make_workload, random_tiny

__all__ = ["Problem", "bf16_bits", "WORKLOADS", "index_replicas", "make_workload", "random_tiny"]
