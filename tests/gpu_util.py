"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle (indices bit-exact, O within atol = rtol = 2e-2,
LSE within 1e-3 absolute)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

O_ATOL = 2e-2
O_RTOL = 2e-2
LSE_ATOL = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_gpu(P, call=None):
    import sparse_shared_kv_amd as s
    call = call or s.Call(P.params, P.arrays)
    out, lse = call.run()
    torch.cuda.synchronize()
    res = dict(O=out.float().cpu().numpy(), call=call,
               status=int(call.status.item()))
    res["lse"] = lse.cpu().numpy() if lse is not None else None
    return res


def check_outputs(P, res, ref, rows=None):
    """O and LSE of the given query rows against the oracle's."""
    rows = sorted(ref["lists"].keys()) if rows is None else rows
    g = res["O"][rows]
    r = ref["O"][rows]
    excess = np.abs(g - r) - (O_ATOL + O_RTOL * np.abs(r))
    assert np.isfinite(g).all(), "non-finite attention_out"
    assert (excess <= 0).all(), "O outside tolerance: max |d| %.3g (excess %.3g) at %s" % (
        np.abs(g - r).max(), excess.max(), np.unravel_index(np.argmax(excess), excess.shape))
    if res["lse"] is not None:
        gl, rl = res["lse"][rows], ref["lse"][rows]
        fin = np.isfinite(rl)
        assert (np.isfinite(gl) == fin).all(), "LSE finiteness differs"
        assert ((gl == rl) | fin).all(), "LSE -inf mismatch"
        if fin.any():
            d = np.abs(gl[fin] - rl[fin]).max()
            assert d <= LSE_ATOL, "LSE outside tolerance: %.3g" % d
    assert res["status"] == 0, "device status %d" % res["status"]
    return float(np.abs(g - r).max())


def check_lists(P, call, ref, rows=None):
    """Resolved physical rows (debug dump) bit-exact against the oracle's."""
    lists = ref["lists"]
    rows = sorted(lists.keys()) if rows is None else rows
    max_rows = max(1, max(len(lists[r]) for r in rows))
    got, counts = call.resolve(max_rows)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    counts = counts.cpu().numpy()
    for r in rows:
        exp = lists[r]
        assert counts[r] == len(exp), "row %d: %d resolved rows, oracle %d" % (r, counts[r], len(exp))
        assert np.array_equal(got[r, :len(exp)], exp), "row %d: resolved rows differ" % r
    return sum(len(lists[r]) for r in rows)
