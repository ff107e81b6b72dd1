"""sfmla_forward_static_workspace (the entry point for callers that cannot
allocate device memory) against sfmla_forward with a caller workspace: same
kernels and split policy, so the outputs must agree bit for bit (and with
the oracle within the stated tolerances), on two calls in a row whose second
input is smaller, plus the refusal of a workspace beyond the library's."""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_outputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_shared_kv_amd  # noqa: F401
    torch.cuda.set_device(0)


def _both(P):
    """(outputs through the caller workspace, outputs through the library's)."""
    import sparse_shared_kv_amd as s
    call = s.Call(P.params, P.arrays)
    ref = [None if t is None else t.clone() for t in call.run()]
    for t in (call.out, call.lse):
        if t is not None:
            t.fill_(float("nan"))
    call.status.zero_()
    call.plan()
    s.sfmla_forward_static_workspace(call.params, call.tensors, call.metadata, call.scale)
    torch.cuda.synchronize()
    assert int(call.status.item()) == 0
    return ref, [call.out, call.lse], call


def test_static_workspace_matches_caller_workspace_twice():
    cases = [synth.random_tiny(941, family="sfa", max_kv=4000, topk=2048, num_heads_q=128,
                               rope_head_dim=64, separate_v=True, lse=True, q_lens=[2, 2],
                               batch=2, layout_q="TND", layout_kv="PA_BSND", block_size=64),
             synth.random_tiny(942, family="csa", max_kv=1500, num_heads_q=64, lse=True,
                               topk=600, cmp_ratio=2)]
    import sparse_shared_kv_amd as s
    for P in cases:                     # the second call has the smaller input
        ws = s.sfmla_workspace_size(s.make_params(P.params, P.arrays))
        say("[no-alloc]", P.name, "workspace bytes", ws)
        assert ws > 0, "the case must use the split workspace"
        ref, got, call = _both(P)
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1]), P.name
        rows = [0, P.query_rows - 1]
        res = dict(O=got[0].float().cpu().numpy(), lse=got[1].cpu().numpy(),
                   status=int(call.status.item()))
        check_outputs(P, res, oracle.forward(P, rows=rows), rows)


def test_static_workspace_refuses_oversized_parameters():
    import sparse_shared_kv_amd as s
    P = synth.random_tiny(943, family="sfa", max_kv=600, topk=500, num_heads_q=128, lse=True,
                          layout_q="TND", layout_kv="PA_BSND")
    # many short splits of many query rows: beyond the library's buffer
    big = dict(P.params, split_rows=32)
    p = s.make_params(big, P.arrays)
    p.q_t = 4096
    need = s.sfmla_workspace_size(p)
    assert need > 64 << 20                           # SFMLA_STATIC_WORKSPACE_BYTES
    call = s.Call(P.params, P.arrays)
    with pytest.raises(s.SfmlaError, match="workspace"):
        s.sfmla_forward_static_workspace(p, call.tensors, call.metadata, call.scale)
