"""The benchmark prices a step by the rows each query row attends to, which
bench.py counts from how the workload is built (bench.recipe_rows), not
through the library.  These CPU checks pin that count to the oracle's
resolved lists on every benchmark recipe (the large pools at reduced size
where the recipe takes sizes; rows sampled on the largest)."""

import os
import sys

import numpy as np
import pytest

import oracle
import synth
from synth import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _oracle_counts(P, rows=None):
    want = None if rows is None else set(rows)
    out = {}
    for row, b, i in oracle.query_rows(P):
        if want is not None and row not in want:
            continue
        out[row] = len(oracle.resolve_rows(P, row, b, i)[2])
    return out


CASES = [
    ("swa_decode", lambda: W.swa_decode()),
    ("csa_decode_paged", lambda: W.csa_decode_paged()),
    ("csa_prefill", lambda: W.csa_prefill()),
    ("hca_prefill", lambda: W.rule_prefill(7, "hca")),
    ("swa_prefill", lambda: W.rule_prefill(8, "swa")),
    ("sfa_mla_rope (2 x 2 queries, 4096 tokens)",
     lambda: W.sfa_mla_rope(batch=2, q_s=2, kv_len=4096, topk=2048)),
    ("sfa_mla_rope block-wise 16 (2 x 2 queries, 4096 tokens)",
     lambda: W.sfa_mla_rope(batch=2, q_s=2, kv_len=4096, topk=2048, sbs=16)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
def test_recipe_rows_match_the_oracle(name, make):
    P = make()
    got = bench.recipe_rows(P)
    ref = _oracle_counts(P)
    assert len(got) == P.query_rows
    assert all(got[r] == n for r, n in ref.items()), name


@pytest.mark.parametrize("name", ["hca_varlen", "c8_packed_int8", "c8_packed_int8_q32",
                                  "hca_varlen_q32", "c8_packed_int8_value"])
def test_recipe_rows_match_the_oracle_full_size(name):
    P = synth.make_workload(name)
    got = bench.recipe_rows(P)
    rows = sorted(set(range(0, P.query_rows, max(1, P.query_rows // 16))) | {P.query_rows - 1})
    ref = _oracle_counts(P, rows)
    assert all(got[r] == n for r, n in ref.items()), name
    assert (got > 0).all()


def test_row_bytes_of_the_packed_value_workload():
    """A packed row with a value tensor moves its 656 key bytes and 512 value
    code bytes (the gathered bytes the roofline counts)."""
    P = synth.make_workload("c8_packed_int8_value")
    assert bench.row_bytes(P) == (656 + 512, 2 * (576 + 512))
