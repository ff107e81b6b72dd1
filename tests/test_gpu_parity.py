"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: resolved KV rows bit-exact (debug resolver dump), attention_out within
|gpu - oracle| <= 2e-2 + 2e-2 |oracle| (bf16 output against float64), LSE
within 1e-3 absolute, and -inf exactly where the oracle has it.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_lists, check_outputs, run_gpu, say
from helpers import logical, place, unplace_o

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_shared_kv_amd  # noqa: F401  (fails loudly without libsfmla.so)
    torch.cuda.set_device(0)


# ---------------------------------------------------------------------------
# the five measured configurations at full size
# ---------------------------------------------------------------------------

FULL = ["swa_decode", "csa_decode_paged", "hca_varlen", "sfa_mla_rope", "c8_packed_int8",
        "c8_packed_fp8", "csa_prefill", "sfa_mla_rope_fp16", "sfa_mla_rope_block16",
        "c8_packed_int8_q32", "hca_varlen_q32", "hca_prefill", "swa_prefill", "swa_prefill_h16",
        "c8_packed_int8_rope0", "c8_packed_int8_value"]


@pytest.mark.parametrize("name", FULL)
def test_full_config_parity(name):
    """Every query row of the workload, at the size the benchmark times."""
    say("[parity] building", name)
    P = synth.make_workload(name)
    say("[parity] gpu run", name)
    res = run_gpu(P)
    say("[parity] oracle", name, "all", P.query_rows, "rows")
    ref = oracle.forward(P)
    n = check_lists(P, res["call"], ref)
    err = check_outputs(P, res, ref)
    say("[parity] %s ok: %d resolved rows bit-exact, max |dO| %.3g" % (name, n, err))


# ---------------------------------------------------------------------------
# small random problems: every family, layout, format and edge case
# ---------------------------------------------------------------------------

TINY = [dict(seed=s) for s in range(40)]
TINY += [dict(seed=100 + s, family="sfa", kv_dtype=["int8_packed", "fp8_e4m3_packed"][s % 2],
              rope_head_dim=[0, 64][(s // 2) % 2], num_heads_q=[1, 16, 20, 128][s % 4])
         for s in range(12)]
TINY += [dict(seed=200 + s, dist="p4", family=["csa", "hca", "swa"][s % 3], num_heads_q=64)
         for s in range(6)]
TINY += [dict(seed=300 + s, family=["csa", "sfa"][s % 2], duplicates=True) for s in range(4)]
TINY += [dict(seed=400 + s, num_heads_q=q) for s, q in enumerate([3, 17, 33, 48, 64, 100, 128])]
# long lists: several splits and a ragged last tile
TINY += [dict(seed=500, family="swa", max_kv=1500, win=(-1, -1), masks=(0, 0), num_heads_q=16),
         dict(seed=501, family="swa", max_kv=1300, win=(1000, 3), masks=(4, 0), num_heads_q=32),
         dict(seed=502, family="sfa", max_kv=3000, topk=1100, num_heads_q=128),
         dict(seed=503, family="csa", max_kv=2500, topk=700, cmp_ratio=2, num_heads_q=64),
         dict(seed=504, family="hca", max_kv=2200, cmp_ratio=1, masks=(0, 3), num_heads_q=16),
         dict(seed=505, family="sfa", max_kv=2100, topk=2048, kv_dtype="int8_packed",
              rope_head_dim=64, num_heads_q=128),
         dict(seed=506, family="sfa", max_kv=2100, topk=1030, kv_dtype="fp8_e4m3_packed",
              rope_head_dim=0, num_heads_q=64),
         dict(seed=507, family="sfa", max_kv=1700, topk=1500, separate_v=True, rope_head_dim=64,
              num_heads_q=128, layout_q="TND", layout_kv="PA_BSND", block_size=64)]
# block-wise TopK entries (sparse_block_size > 1), every layout and format,
# with duplicates, and lists long enough for several splits
TINY += [dict(seed=700 + s, family="sfa", sparse_block_size=[2, 4, 16, 64][s % 4],
              max_kv=300, num_heads_q=[16, 64, 128][s % 3],
              kv_dtype=["bf16", "bf16", "int8_packed", "fp8_e4m3_packed"][(s // 2) % 4],
              duplicates=bool(s % 5 == 4)) for s in range(10)]
# float16 q / kv / output: every family, peaked softmaxes, long lists
TINY += [dict(seed=800 + s, kv_dtype="fp16", family=["swa", "csa", "hca", "sfa"][s % 4],
              dist=["normal", "p4"][(s // 4) % 2], num_heads_q=[16, 64, 128, 5][s % 4])
         for s in range(8)]
TINY += [dict(seed=810, kv_dtype="fp16", family="sfa", max_kv=2600, topk=1300, rope_head_dim=64,
              separate_v=True, num_heads_q=128, layout_q="TND", layout_kv="PA_BSND", block_size=64),
         dict(seed=811, kv_dtype="fp16", family="hca", max_kv=2200, cmp_ratio=1, masks=(0, 3),
              num_heads_q=32)]
TINY += [dict(seed=720, family="sfa", sparse_block_size=16, max_kv=3000, topk=120,
              num_heads_q=128, layout_q="BSND", layout_kv="PA_BSND", block_size=64),
         dict(seed=721, family="sfa", sparse_block_size=8, max_kv=2500, topk=250,
              kv_dtype="int8_packed", rope_head_dim=64, num_heads_q=64)]


@pytest.mark.parametrize("kw", TINY, ids=lambda k: "-".join(str(v) for v in k.values()))
def test_tiny_parity(kw):
    P = synth.random_tiny(**kw)
    ref = oracle.forward(P)
    res = run_gpu(P)
    check_lists(P, res["call"], ref)
    check_outputs(P, res, ref)


def test_all_slots_empty_gives_zero_and_neg_inf():
    P = synth.random_tiny(7, family="csa", sinks=True, num_heads_q=16)
    P.arrays["cmp_sparse_indices"][:] = -1
    P.params["ori_win_left"] = 0
    P.params["ori_win_right"] = 0
    P.params["ori_mask_mode"] = 4
    ref = oracle.forward(P)
    res = run_gpu(P)
    check_lists(P, res["call"], ref)
    check_outputs(P, res, ref)


def test_no_valid_query_rows():
    P = synth.random_tiny(9, family="hca", layout_q="BSND", seqused_q=True, num_heads_q=16,
                          q_lens=[3, 2], ori_lens=[20, 30], batch=2)
    P.arrays["seqused_q"] = np.array([0, 1], np.int32)
    ref = oracle.forward(P)
    res = run_gpu(P)
    assert (res["O"][:3] == 0).all() and np.isneginf(res["lse"][:3]).all()
    check_lists(P, res["call"], ref)
    check_outputs(P, res, ref)


# ---------------------------------------------------------------------------
# properties of the GPU path itself
# ---------------------------------------------------------------------------

def test_deterministic_bitwise():
    import sparse_shared_kv_amd as s
    P = synth.random_tiny(502, family="sfa", max_kv=3000, topk=1100, num_heads_q=128, lse=True)
    call = s.Call(P.params, P.arrays)
    a = [t.clone() for t in call.run()]
    b = [t.clone() for t in call.run()]
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("fmt", ["bf16", "int8_packed"])
def test_head_grouping_invariance_bitwise(fmt):
    """Spreading a row's heads over 1, 2, 4 or 8 head groups (the rest of the
    workgroup's waves only gathering) leaves every output bit unchanged."""
    import sparse_shared_kv_amd as s
    kw = dict(family="sfa", max_kv=2500, topk=1100, num_heads_q=128, lse=True)
    if fmt != "bf16":
        kw.update(kv_dtype=fmt, rope_head_dim=64)
    P = synth.random_tiny(503, **kw)
    outs, status = [], 0
    for bpg in (1, 2, 4, 8):
        # plan and workspace sized for this grouping
        call = s.Call(dict(P.params, head_blocks_per_group=bpg), P.arrays)
        outs.append([None if t is None else t.clone() for t in call.run()])
        torch.cuda.synchronize()
        status |= int(call.status.item())
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0])
        assert (o[1] is None and outs[0][1] is None) or torch.equal(o[1], outs[0][1])
    ref = oracle.forward(P, rows=[0, 1])
    res = dict(O=outs[0][0].float().cpu().numpy(), status=status,
               lse=None if outs[0][1] is None else outs[0][1].cpu().numpy())
    check_outputs(P, res, ref, [0, 1])


@pytest.mark.parametrize("split_rows", [32, 1024, 2048])
@pytest.mark.parametrize("fmt", ["bf16", "int8_packed"])
def test_split_sizes_match_oracle(fmt, split_rows):
    """Lists cut into 32-row splits (many partials to merge) or held whole in
    one workgroup's row table (up to 2048 rows) give the oracle's result."""
    import sparse_shared_kv_amd as s
    kw = dict(family="sfa", max_kv=4000, topk=2100, num_heads_q=64)
    if fmt != "bf16":
        kw.update(kv_dtype=fmt, rope_head_dim=64)
    P = synth.random_tiny(507, **kw)
    call = s.Call(dict(P.params, split_rows=split_rows), P.arrays)
    out = [None if t is None else t.clone() for t in call.run()]
    torch.cuda.synchronize()
    rows = [0, 1, P.params["q_t"] - 1] if "q_t" in P.params else [0, 1]
    rows = sorted(set(r for r in rows if r >= 0))
    ref = oracle.forward(P, rows=rows)
    res = dict(O=out[0].float().cpu().numpy(), status=int(call.status.item()),
               lse=None if out[1] is None else out[1].cpu().numpy())
    check_outputs(P, res, ref, rows)


def test_batch_invariance_bitwise():
    """A sequence alone and inside a batch gives bit-identical rows."""
    L = logical(21, q_lens=[2, 3, 1, 2], ori_lens=[900, 1400, 300, 2000], qn=32, ratio=4,
                cmp_topk=200, win=(127, 0))
    import sparse_shared_kv_amd as s
    full = place(L, "TND", "PA_BSND", bs=16, seed=1)
    out_full = run_gpu(full)["O"]
    per_b = unplace_o(full, out_full, L)
    for b in (1, 3):
        Lb = {k: ([v[b]] if isinstance(v, list) and len(v) == 4 else v) for k, v in L.items()}
        one = place(Lb, "TND", "PA_BSND", bs=16, seed=2)
        got = run_gpu(one)["O"]
        assert np.array_equal(got, per_b[b]), b


def test_batch_invariance_with_long_query_sequences_bitwise():
    """Rows of sequences with many queries keep their list in one split while
    short sequences split theirs; either way a sequence alone and inside a
    batch gives bit-identical rows."""
    L = logical(25, q_lens=[70, 2, 64, 1], ori_lens=[3000, 2600, 1900, 2200], qn=16, ratio=4,
                cmp_topk=600, win=(127, 0))
    full = place(L, "TND", "PA_BSND", bs=16, seed=1)
    res = run_gpu(full)
    rows = [0, 69, 70, 135, 136]
    check_outputs(full, res, oracle.forward(full, rows=rows), rows)
    per_b = unplace_o(full, res["O"], L)
    for b in (0, 1, 2):
        Lb = {k: ([v[b]] if isinstance(v, list) and len(v) == 4 else v) for k, v in L.items()}
        one = place(Lb, "TND", "PA_BSND", bs=16, seed=2)
        got = run_gpu(one)["O"]
        assert np.array_equal(got, per_b[b]), b


def test_split_steps_by_query_count_bitwise():
    """Sequences of 17, 33 and 48 queries take 2, 4 and 6 steps of the split
    length (one per 8 queries), the 2-query one the base length; each
    sequence gives the same bits alone and inside a batch, and matches the
    oracle."""
    L = logical(27, q_lens=[33, 17, 48, 2], ori_lens=[2600, 2200, 3000, 900], qn=32, ratio=2,
                cmp_topk=900, win=(127, 0))
    full = place(L, "TND", "PA_BSND", bs=16, seed=1)
    res = run_gpu(full)
    rows = [0, 32, 33, 49, 50, 97, 98, 99]
    check_outputs(full, res, oracle.forward(full, rows=rows), rows)
    per_b = unplace_o(full, res["O"], L)
    for b in (0, 1, 2):
        Lb = {k: ([v[b]] if isinstance(v, list) and len(v) == 4 else v) for k, v in L.items()}
        one = place(Lb, "TND", "PA_BSND", bs=16, seed=2)
        got = run_gpu(one)["O"]
        assert np.array_equal(got, per_b[b]), b


def test_layout_invariance_bitwise():
    L = logical(23, q_lens=[3, 1, 4], ori_lens=[700, 90, 1500], qn=64, ratio=4, cmp_topk=100)
    outs = []
    for lq, lk, bs in [("BSND", "BSND", 0), ("TND", "TND", 0), ("BSND", "PA_BSND", 16),
                       ("TND", "PA_BSND", 128)]:
        P = place(L, lq, lk, bs=bs or 4, seed=5)
        outs.append(unplace_o(P, run_gpu(P)["O"], L))
    for o in outs[1:]:
        for b in range(3):
            assert np.array_equal(o[b], outs[0][b])


def test_metadata_from_other_params_is_rejected():
    import sparse_shared_kv_amd as s
    P = synth.make_workload("swa_decode")
    call = s.Call(P.params, P.arrays)
    other = dict(P.params)
    other["ori_win_left"] = 63
    call_b = s.Call(other, P.arrays)
    call_b.plan()
    call.metadata.copy_(call_b.metadata)       # plan of different parameters
    call.status.zero_()
    call.forward()
    torch.cuda.synchronize()
    assert torch.isnan(call.out.float()).all()
    assert int(call.status.item()) & 1


@pytest.mark.parametrize("fmt,split_rows,wp", [("bf16", 512, 1), ("bf16", 512, 2),
                                              ("int8_packed", 512, 1), ("int8_packed", 256, 2),
                                              ("bf16", 256, 1)])
def test_forward_reuses_metadata_across_calls_bitwise(fmt, split_rows, wp):
    """One plan, then the forward called again and again on it (as the
    layers of a model step would): the merges leave their arrival counters
    ready for the next call, so every call rewrites the same bits (two
    splits, merged from registers; four splits, merged by the last to
    arrive or by their owners)."""
    import sparse_shared_kv_amd as s
    kw = dict(family="sfa", max_kv=3000, topk=1024, num_heads_q=128, rope_head_dim=64,
              separate_v=False, sinks=True, lse=True)
    if fmt != "bf16":
        kw.update(kv_dtype=fmt)
    P = synth.random_tiny(1210, **kw)
    call = s.Call(dict(P.params, split_rows=split_rows, wave_pairs=wp), P.arrays)
    first = [t.clone() for t in call.run() if t is not None]
    torch.cuda.synchronize()
    assert int(call.status.item()) == 0
    for rep in range(3):
        say(f"forward again {fmt} split_rows={split_rows} wave_pairs={wp} call {rep + 2}")
        for t in (call.out, call.lse):
            t.fill_(float("nan"))
        call.forward()
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
        for e, x in zip(first, (call.out, call.lse)):
            assert torch.equal(e, x), rep
    rows = list(range(P.query_rows))
    res = dict(O=first[0].float().cpu().numpy(), status=0, lse=first[1].cpu().numpy())
    check_outputs(P, res, oracle.forward(P, rows=rows), rows)


@pytest.mark.parametrize("far_sink", [False, True])
def test_combine_entry_point_matches_oracle_merge(far_sink):
    """sfmla_combine (the LSE merge of caller-supplied partials) against the
    oracle's merge; far_sink puts every head's sink 200 above its largest
    part LSE, where O goes to 0 and the LSE must stay finite."""
    import sparse_shared_kv_amd as s
    g = np.random.default_rng(3)
    n_parts, rows, heads, dv = 5, 7, 12, 512
    part_o = g.standard_normal((n_parts, rows, heads, dv)).astype(np.float32)
    part_lse = (g.standard_normal((n_parts, rows, heads)) * 3).astype(np.float32)
    part_lse[1, 2, :] = -np.inf                    # an empty part
    part_lse[:, 4, 3] = -np.inf                    # a fully empty (row, head)
    sinks = g.standard_normal(heads).astype(np.float32)
    if far_sink:
        top = np.where(np.isfinite(part_lse), part_lse, -np.inf).max(axis=(0, 1))
        sinks = (top + 200.0).astype(np.float32)
    dev = torch.device("cuda")
    out = torch.empty((rows, heads, dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows, heads), dtype=torch.float32, device=dev)
    s.sfmla_combine(torch.from_numpy(part_o).to(dev), torch.from_numpy(part_lse).to(dev),
                    torch.from_numpy(sinks).to(dev), out, lse)
    torch.cuda.synchronize()
    for r in range(rows):
        O, L = oracle.combine(part_o[:, r], part_lse[:, r], sinks)
        got = out[r].float().cpu().numpy()
        assert (np.abs(got - O) <= 2e-2 + 2e-2 * np.abs(O)).all()
        gl = lse[r].cpu().numpy()
        fin = np.isfinite(L)
        assert (np.isfinite(gl) == fin).all()
        assert np.abs(gl[fin] - L[fin]).max() <= 1e-3


@pytest.mark.parametrize("fmt", ["int8_packed", "fp8_e4m3_packed"])
def test_rope_free_rows_equal_zero_rope_rows_bitwise(fmt):
    """528-byte rows (no rope) give bit-identical results to 656-byte rows
    whose rope is zero (SparseAttnSharedkv README, 参数说明: the packed row
    width with and without rope)."""
    import copy
    import sparse_shared_kv_amd as s
    P = synth.random_tiny(601, family="sfa", kv_dtype=fmt, rope_head_dim=64, num_heads_q=64,
                          max_kv=700, topk=600, lse=True)
    P656 = copy.deepcopy(P)
    P656.arrays["ori_kv"] = P656.arrays["ori_kv"].copy()
    P656.arrays["ori_kv"][:, 512:640] = 0                      # zero rope
    P528 = copy.deepcopy(P656)
    P528.params["rope_head_dim"] = 0
    P528.arrays["ori_kv"] = np.ascontiguousarray(
        np.concatenate([P656.arrays["ori_kv"][:, :512], P656.arrays["ori_kv"][:, 640:656]], axis=1))
    P528.arrays["q"] = np.ascontiguousarray(P656.arrays["q"][..., :512])
    # the same softmax scale on both sides (not 1/sqrt of each width)
    P528.params["softmax_scale"] = P656.params["softmax_scale"]
    a = run_gpu(P656)
    b = run_gpu(P528)
    assert a["status"] == 0 and b["status"] == 0
    assert np.array_equal(a["O"], b["O"])
    assert np.array_equal(a["lse"], b["lse"])
    ref = oracle.forward(P528, rows=[0, 1])
    check_outputs(P528, b, ref, [0, 1])


GRAPH_CASES = [dict(),                                        # bf16, separate V (staged merge)
               dict(kv_dtype="int8_packed", rope_head_dim=64),
               dict(separate_v=False, rope_head_dim=0),         # V = K nope
               dict(kv_dtype="fp8_e4m3_packed", rope_head_dim=64, separate_v=True)]  # value codes


@pytest.mark.parametrize("kw", GRAPH_CASES, ids=["separate_v", "packed", "shared_v", "packed_value"])
def test_graph_replay_matches_eager(kw):
    """plan + forward captured in one HIP graph: every replay, with other
    eager work and synchronisations in between, reproduces the eager result
    bit for bit (split rows merged in the launch: the arrival counters must
    come back to zero on every replay)."""
    P = synth.random_tiny(602, family="sfa", max_kv=3000, topk=1500, num_heads_q=128, lse=True,
                          **kw)
    _graph_replay(P)


def _graph_replay(P):
    import sparse_shared_kv_amd as s
    other = synth.random_tiny(603, family="csa", num_heads_q=64, max_kv=900)
    call = s.Call(P.params, P.arrays)
    eager = [t.clone() for t in call.run() if t is not None]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call.run()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call.run()
    oc = s.Call(other.params, other.arrays)
    for rep in range(4):
        for t in (call.out, call.lse):
            if t is not None:
                t.fill_(float("nan"))                # the replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        got = [t for t in (call.out, call.lse) if t is not None]
        for e, x in zip(eager, got):
            assert torch.equal(e, x), rep
        oc.run()                                     # unrelated eager work between replays
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0


def test_timing_hook_stamps_the_forward_kernel():
    """sfmla_time_next_forward: the next forward's kernel start and end land
    in the two events (positive duration, result unchanged), and only that
    call is timed."""
    import sparse_shared_kv_amd as s
    P = synth.random_tiny(611, family="sfa", max_kv=3000, topk=1500, num_heads_q=64)
    call = s.Call(P.params, P.arrays)
    ref = [t.clone() for t in call.run() if t is not None]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    call.plan()
    s.sfmla_time_next_forward(e0, e1)
    call.forward()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert 0.0 < ms < 100.0
    call.forward()                                 # not timed: the events keep their stamps
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == ms
    got = [t for t in (call.out, call.lse) if t is not None]
    for x, y in zip(ref, got):
        assert torch.equal(x, y)


@pytest.mark.parametrize("separate_v", [True, False])
def test_topk_rows_long_and_short_sequences_partial_head_block(separate_v):
    """TopK lists in a sequence of 70 queries (one split of up to 2048 rows
    per row, so the first index batch is reloaded, not taken from the
    early loads) next to a short sequence (three 512-row splits merged,
    through LDS staging when V is separate), with 20 heads (the second
    16-head block is partly past q_n)."""
    P = synth.random_tiny(613, family="sfa", layout_q="TND", layout_kv="PA_BSND", q_lens=[70, 3],
                          ori_lens=[3000, 2500], topk=1100, num_heads_q=20, rope_head_dim=64,
                          separate_v=separate_v, block_size=16, win=(-1, -1), masks=(3, 0))
    rows = [0, 35, 69, 70, 72]
    res = run_gpu(P)
    check_outputs(P, res, oracle.forward(P, rows=rows), rows)


# ---------------------------------------------------------------------------
# tensor layouts the boundary accepts: rope stored apart, padded rows
# ---------------------------------------------------------------------------

def _strided(rows_np, width, pad, dev, fill):
    """Device view (rows, width) of a buffer whose rows are width + pad
    elements long; the padding holds `fill` (a NaN pattern for 16-bit
    floats) so that a read of it shows in the output."""
    dt = torch.uint8 if rows_np.dtype == np.uint8 else torch.int16
    src = torch.from_numpy(np.ascontiguousarray(rows_np[:, :width]).view(
        np.uint8 if rows_np.dtype == np.uint8 else np.int16))
    buf = torch.full((rows_np.shape[0], width + pad), fill, dtype=dt, device=dev)
    buf[:, :width] = src.to(dev)
    return buf[:, :width]


def _relayout(P, split_rope, pad):
    """Device arrays of P with the KV rows relaid: the 64 rope values in a
    tensor of their own (SparseFlashAttention page, 参数说明 key_rope:
    the rope part passed apart from the nope part) and / or every row
    stride padded (sparse_flash_mla API page, 约束说明: ori_kv and cmp_kv
    may have padding between rows).  The oracle keeps reading P itself."""
    dev = torch.device("cuda")
    packed = P.params["kv_dtype"] not in ("bf16", "fp16")
    nan16, junk8 = -1, 255                          # 0xFFFF: NaN in bf16 and float16
    arrays = dict(P.arrays)
    rope = P.params["rope_head_dim"]
    for side, pk, pr in (("ori", 8, 8), ("cmp", 24, 0)):
        a = P.arrays.get(side + "_kv")
        if a is None:
            continue
        if packed:
            arrays[side + "_kv"] = _strided(a, a.shape[1], 16 * (pad // 8), dev, junk8)
        elif split_rope and rope:
            arrays[side + "_kv"] = _strided(a, 512, pk if pad else 0, dev, nan16)
            arrays[side + "_rope"] = _strided(a[:, 512:], 64, pr if pad else 0, dev, nan16)
        else:
            arrays[side + "_kv"] = _strided(a, a.shape[1], pk if pad else 0, dev, nan16)
    if P.arrays.get("ori_v") is not None:
        # 16-bit values, or the value codes of packed rows (512 bytes)
        arrays["ori_v"] = _strided(P.arrays["ori_v"], 512, 512 if pad else 0, dev,
                                   junk8 if packed else nan16)
    return arrays


LAYOUT_CASES = [
    # rope stored apart: token-wise TopK (shared and separate V), CSA / HCA
    # with rope on both KV sides, float16
    dict(seed=900, family="sfa", rope_head_dim=64, separate_v=False, split_rope=True),
    dict(seed=901, family="sfa", rope_head_dim=64, separate_v=True, split_rope=True,
         max_kv=1500, topk=700, num_heads_q=128),
    dict(seed=902, family="csa", rope_head_dim=64, split_rope=True, num_heads_q=64),
    dict(seed=903, family="hca", rope_head_dim=64, split_rope=True, num_heads_q=16,
         max_kv=900, cmp_ratio=2),
    dict(seed=904, family="sfa", rope_head_dim=64, kv_dtype="fp16", split_rope=True,
         num_heads_q=32),
    # padded row strides (garbage in the padding), with and without rope apart
    dict(seed=910, family="swa", pad=8, num_heads_q=16, max_kv=600),
    dict(seed=911, family="csa", pad=8, num_heads_q=64),
    dict(seed=912, family="sfa", rope_head_dim=64, separate_v=True, pad=8, num_heads_q=128,
         max_kv=1500, topk=1100),
    dict(seed=913, family="hca", rope_head_dim=64, split_rope=True, pad=8, num_heads_q=32,
         cmp_ratio=4, max_kv=700),
    dict(seed=914, family="sfa", kv_dtype="int8_packed", rope_head_dim=64, pad=8,
         num_heads_q=128, max_kv=900, topk=600),
    dict(seed=915, family="sfa", kv_dtype="fp8_e4m3_packed", rope_head_dim=0, pad=16,
         num_heads_q=16),
    # packed rows with a value tensor of codes, both strides padded (0xFF in
    # the padding: a NaN code in E4M3, -1 in INT8)
    dict(seed=916, family="sfa", kv_dtype="int8_packed", rope_head_dim=64, separate_v=True,
         pad=8, num_heads_q=64, max_kv=900, topk=600),
    dict(seed=917, family="sfa", kv_dtype="fp8_e4m3_packed", rope_head_dim=0, separate_v=True,
         pad=16, num_heads_q=128, max_kv=1300, topk=1100),
]


@pytest.mark.parametrize("kw", LAYOUT_CASES, ids=lambda k: "-".join(str(v) for v in k.values()))
def test_kv_layout_parity(kw):
    """Rope given as its own tensor and / or padded row strides: the oracle on
    the plain rows, the GPU on the relaid device tensors."""
    import sparse_shared_kv_amd as s
    kw = dict(kw)
    split_rope, pad = kw.pop("split_rope", False), kw.pop("pad", 0)
    P = synth.random_tiny(**kw)
    arrays = _relayout(P, split_rope, pad)
    call = s.Call(P.params, arrays)
    if split_rope:
        assert call.tensors.ori_rope and call.tensors.ori_kv_stride == 2 * (512 + (8 if pad else 0))
    ref = oracle.forward(P)
    res = run_gpu(P, call)
    check_lists(P, call, ref)
    check_outputs(P, res, ref)


def test_lse_off_matches_lse_on_bitwise():
    """return_softmax_lse = 0 (no LSE tensor) leaves attention_out bit for
    bit what it is with the LSE returned, over split and unsplit rows."""
    import sparse_shared_kv_amd as s
    for seed, kw in ((920, dict(family="sfa", max_kv=3000, topk=1500, num_heads_q=128,
                                rope_head_dim=64, separate_v=True)),
                     (921, dict(family="csa", num_heads_q=64, max_kv=900, sinks=True)),
                     (922, dict(family="sfa", kv_dtype="int8_packed", rope_head_dim=64,
                                num_heads_q=128, max_kv=2500, topk=1100))):
        P_on = synth.random_tiny(seed, lse=True, **kw)
        P_off = synth.random_tiny(seed, lse=False, **kw)
        on, off = run_gpu(P_on), run_gpu(P_off)
        assert off["lse"] is None and on["lse"] is not None
        assert np.array_equal(on["O"], off["O"]), seed
        check_outputs(P_off, off, oracle.forward(P_off, rows=[0]), [0])


# ---------------------------------------------------------------------------
# the two ways a split row is merged
# ---------------------------------------------------------------------------

MERGE_CASES = [
    # owned merges need every wave of the workgroup to hold heads: 128 heads
    # in one group of 8 head blocks.  4 splits of 512 rows (rope, separate V:
    # the headline's kernel)
    dict(seed=930, family="sfa", max_kv=4000, topk=2048, num_heads_q=128, rope_head_dim=64,
         separate_v=True, layout_q="TND", layout_kv="PA_BSND", block_size=64, q_lens=[2, 1],
         batch=2, head_blocks_per_group=8),
    # 2 and 8 splits with V = K nope (the extra landing buffer)
    dict(seed=931, family="sfa", max_kv=3000, topk=1000, num_heads_q=128, rope_head_dim=0,
         separate_v=False, split_rows=512, head_blocks_per_group=8),
    dict(seed=932, family="sfa", max_kv=3000, topk=2000, num_heads_q=128, rope_head_dim=64,
         separate_v=False, split_rows=256, head_blocks_per_group=8),
    # 3 splits: splits 0 and 1 own too many waves for the landing slots (the
    # last to arrive merges those heads), split 2 owns its two; float16, sinks
    dict(seed=933, family="csa", max_kv=2000, topk=700, num_heads_q=128, cmp_ratio=1,
         kv_dtype="fp16", sinks=True, head_blocks_per_group=8),
    # not owned: 4 head groups of 32 heads; a partial last head block
    dict(seed=934, family="sfa", max_kv=3000, topk=2048, num_heads_q=128, rope_head_dim=64,
         separate_v=True, head_blocks_per_group=2),
    dict(seed=935, family="sfa", max_kv=3000, topk=1000, num_heads_q=100, rope_head_dim=0,
         separate_v=False, split_rows=512, head_blocks_per_group=8),
]


@pytest.mark.parametrize("kw", MERGE_CASES, ids=lambda k: str(k["seed"]))
def test_owned_merge_matches_last_arriver_bitwise(kw):
    """A split row's partials merged by their owning split (the default when
    the launch fits the GPU at once), by the last split to arrive
    (merge_wait_us = -1), and with a 1 us wait bound (owners that time out
    hand the merge over) give the same bits, and the oracle's result."""
    import sparse_shared_kv_amd as s
    kw = dict(kw)
    split_rows = kw.pop("split_rows", 0)
    bpg = kw.pop("head_blocks_per_group", 0)
    P = synth.random_tiny(lse=True, **kw)
    outs = []
    for mw in (0, -1, 1, 0):
        call = s.Call(dict(P.params, split_rows=split_rows, merge_wait_us=mw,
                           head_blocks_per_group=bpg), P.arrays)
        for _ in range(2):
            outs.append([t.clone() for t in call.run()])
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])
    ws = s.sfmla_workspace_size(s.make_params(dict(P.params, split_rows=split_rows,
                                                   head_blocks_per_group=bpg), P.arrays))
    assert ws > 0, "the case must split its rows"
    rows = sorted({0, P.query_rows - 1})
    res = dict(O=outs[0][0].float().cpu().numpy(), lse=outs[0][1].cpu().numpy(), status=0)
    check_outputs(P, res, oracle.forward(P, rows=rows), rows)


# ---------------------------------------------------------------------------
# query tiles: consecutive query rows of a sequence share one gathered list
# ---------------------------------------------------------------------------

def _tiny_tiled(kw):
    kw = dict(kw)
    tq = kw.pop("query_tile")
    P = synth.random_tiny(**kw)
    P.params["query_tile"] = tq
    return P


TILE_CASES = (
    [dict(seed=700 + i, family=["swa", "hca"][i % 2], query_tile=[2, 4, 8][i % 3], max_q=20,
          max_kv=300) for i in range(12)]
    + [dict(seed=720 + i, family=["swa", "hca"][i % 2], query_tile=2, num_heads_q=64, dist="p4",
            max_q=9, max_kv=400) for i in range(2)]
    + [dict(seed=730, family="hca", query_tile=4, num_heads_q=20, max_q=13),
       dict(seed=731, family="swa", query_tile=4, num_heads_q=32, max_q=13, kv_dtype="fp16"),
       dict(seed=732, family="hca", query_tile=8, kv_dtype="fp16", max_q=20),
       dict(seed=733, family="swa", query_tile=2, separate_v=True, rope_head_dim=64,
            num_heads_q=48, max_q=11, max_kv=200),
       dict(seed=734, family="hca", query_tile=8, rope_head_dim=64, max_q=17, max_kv=200),
       dict(seed=735, family="hca", query_tile=4, layout_q="TND", batch=3, q_lens=[5, 0, 9],
            ori_lens=[40, 10, 60]),
       dict(seed=736, family="swa", query_tile=2, layout_q="BSND", batch=2, q_lens=[7, 3],
            ori_lens=[30, 50], seqused_q=True)]
)


@pytest.mark.parametrize("kw", TILE_CASES, ids=lambda k: "-".join(str(v) for v in k.values()))
def test_tiny_tiled_parity(kw):
    """Tiles forced on small problems (every layout, window and mask rule,
    ragged and empty sequences, rows past seqused_q, tiles cut short by the
    sequence's end, 1 to 4 head blocks per row, rope and a separate V,
    float16): every row against the oracle."""
    P = _tiny_tiled(kw)
    say("[tiles] case", kw)
    ref = oracle.forward(P)
    res = run_gpu(P)
    check_lists(P, res["call"], ref)
    check_outputs(P, res, ref)


def _mixed_tile_batch():
    """Sequences by rule (rows with rope: tiles are the rule): 20 queries
    with a short union (tiled), 3 queries (too few: one workgroup per row),
    18 queries whose visible compressed rows exceed one split (rows split
    in 256-row chunks and merged)."""
    return logical(41, q_lens=[20, 3, 18], ori_lens=[600, 900, 9000], qn=16, ratio=4, cmp_topk=0,
                   win=(127, 0), rope=64)


def test_tiled_batch_matches_oracle_and_is_batch_invariant_bitwise():
    L = _mixed_tile_batch()
    full = place(L, "TND", "PA_BSND", bs=16, seed=1)
    say("[tiles] mixed batch: gpu")
    res = run_gpu(full)
    say("[tiles] mixed batch: oracle")
    ref = oracle.forward(full)
    check_lists(full, res["call"], ref)
    check_outputs(full, res, ref)
    per_b = unplace_o(full, res["O"], L)
    for b in range(3):
        Lb = {k: ([v[b]] if isinstance(v, list) and len(v) == 3 else v) for k, v in L.items()}
        one = place(Lb, "TND", "PA_BSND", bs=16, seed=2)
        got = run_gpu(one)["O"]                   # b = 1 alone: no tiles in the launch at all
        assert np.array_equal(got, per_b[b]), b


def test_untiled_rows_of_a_tiled_launch_equal_the_untiled_launch_bitwise():
    """The rows that are not tiled give the same bits with tiles off for the
    whole call; the tiled rows agree with the oracle either way."""
    import sparse_shared_kv_amd as s
    L = _mixed_tile_batch()
    P = place(L, "TND", "PA_BSND", bs=16, seed=1)
    on = run_gpu(P)
    off = run_gpu(P, s.Call(dict(P.params, query_tile=1), P.arrays))
    assert np.array_equal(on["O"][20:], off["O"][20:])
    assert np.array_equal(on["lse"][20:], off["lse"][20:])
    assert not np.array_equal(on["O"][:20], off["O"][:20])   # the tiled rows took another order
    ref = oracle.forward(P, rows=list(range(20)))
    check_outputs(P, off, ref, list(range(20)))


def test_tiled_metadata_from_other_params_is_rejected():
    import sparse_shared_kv_amd as s
    P = synth.make_workload("swa_prefill")
    call = s.Call(dict(P.params, query_tile=2), P.arrays)
    other = dict(P.params, query_tile=2, ori_win_left=63)
    call_b = s.Call(other, P.arrays)
    call_b.plan()
    call.metadata.copy_(call_b.metadata)       # plan of different parameters (same size)
    call.status.zero_()
    call.forward()
    torch.cuda.synchronize()
    assert torch.isnan(call.out.float()).all()
    assert int(call.status.item()) & 1
    # a plan made with tiles off does not serve a call with tiles
    call_c = s.Call(dict(P.params, query_tile=1), P.arrays)
    call_c.plan()
    call.metadata.zero_()
    call.metadata[:call_c.metadata.numel()].copy_(call_c.metadata)
    call.status.zero_()
    call.out.zero_()
    call.forward()
    torch.cuda.synchronize()
    assert torch.isnan(call.out.float()).all()
    assert int(call.status.item()) & 1


def test_tiled_graph_replay_matches_eager():
    L = _mixed_tile_batch()
    _graph_replay(place(L, "TND", "PA_BSND", bs=16, seed=1))


@pytest.mark.parametrize("kw", [
    dict(seed=801, family="sfa", separate_v=True, num_heads_q=128, max_kv=3000, topk=1100),
    dict(seed=802, family="sfa", kv_dtype="int8_packed", num_heads_q=20, max_kv=900),
    dict(seed=803, family="sfa", kv_dtype="fp16", num_heads_q=16, separate_v=False),
    dict(seed=804, family="hca", num_heads_q=32, max_q=20, max_kv=300, query_tile=4),
    dict(seed=805, family="sfa", kv_dtype="int8_packed", num_heads_q=128, max_kv=1500,
         topk=900, head_blocks_per_group=8),
], ids=["bf16_separate_v", "int8_packed", "fp16", "tiles", "int8_packed_eight_waves"])
def test_q_rope_apart_matches_concatenated_bitwise(kw):
    """The query's rope part passed as its own tensor (SparseFlashAttention
    README, 参数说明 query_rope) gives the same bits as one 576-wide q."""
    import sparse_shared_kv_amd as s
    kw = dict(kw, rope_head_dim=64, lse=True)
    tq = kw.pop("query_tile", 0)
    bpg = kw.pop("head_blocks_per_group", 0)
    P = synth.random_tiny(**kw)
    spec = dict(P.params, query_tile=tq, head_blocks_per_group=bpg)
    q = P.arrays["q"]
    split = dict(P.arrays, q=np.ascontiguousarray(q[..., :512]),
                 q_rope=np.ascontiguousarray(q[..., 512:]))
    one = run_gpu(P, s.Call(spec, P.arrays))
    two = run_gpu(P, s.Call(spec, split))
    assert one["status"] == 0 and two["status"] == 0
    assert np.array_equal(one["O"], two["O"])
    assert np.array_equal(one["lse"], two["lse"])
    rows = list(range(min(4, P.query_rows)))
    check_outputs(P, two, oracle.forward(P, rows=rows), rows)


# ---------------------------------------------------------------------------
# wave pairs (16-bit rows, at most 64 heads)
# ---------------------------------------------------------------------------

PAIR_CASES = [
    # rope, separate V, 3 splits (last-arriver merge), sinks
    dict(seed=950, family="sfa", max_kv=3000, topk=1100, num_heads_q=64, rope_head_dim=64,
         separate_v=True, sinks=True, lse=True),
    # V = K nope, 48 heads (three pairs over two head groups), varlen queries
    dict(seed=951, family="swa", max_kv=600, num_heads_q=48, layout_q="TND", lse=True),
    # 32 heads (two pairs, the other four waves only gather), float16, compressed TopK
    dict(seed=952, family="csa", max_kv=2000, topk=700, num_heads_q=32, cmp_ratio=4,
         kv_dtype="fp16", sinks=True, lse=True),
    # a single head, all visible compressed rows, no LSE output
    dict(seed=953, family="hca", max_kv=1500, num_heads_q=1, cmp_ratio=4, lse=False),
    # paged KV, two pairs per head group (two groups), rope in the rows
    dict(seed=954, family="sfa", max_kv=4000, topk=2048, num_heads_q=64, rope_head_dim=64,
         separate_v=False, layout_kv="PA_BSND", block_size=64, head_blocks_per_group=2),
    # float16, separate V without rope, repeated TopK entries
    dict(seed=955, family="sfa", max_kv=2500, topk=900, num_heads_q=16, rope_head_dim=0,
         separate_v=True, kv_dtype="fp16", duplicates=True, lse=True),
    # 128 heads: two head groups of four pairs, rope, separate V, 4 splits
    dict(seed=956, family="sfa", max_kv=4000, topk=2048, num_heads_q=128, rope_head_dim=64,
         separate_v=True, sinks=True, lse=True),
    # packed rows: INT8 with rope (8 splits of the TopK list), FP8 without
    # rope, 20 heads (the second pair of its group half empty)
    dict(seed=957, family="sfa", kv_dtype="int8_packed", max_kv=3000, topk=2048,
         num_heads_q=128, rope_head_dim=64, sinks=True, lse=True),
    dict(seed=958, family="sfa", kv_dtype="fp8_e4m3_packed", max_kv=1500, topk=700, num_heads_q=20,
         rope_head_dim=0, lse=True),
]


@pytest.mark.parametrize("kw", PAIR_CASES, ids=lambda k: str(k["seed"]))
def test_wave_pairs_match_single_waves_bitwise(kw):
    """Two waves sharing 16 heads (each with the scores of half of every KV
    tile and half of the value columns) give the bits of one wave holding
    them, and the oracle's result on every row."""
    import sparse_shared_kv_amd as s
    kw = dict(kw)
    bpg = kw.pop("head_blocks_per_group", 0)
    P = synth.random_tiny(**kw)
    outs = []
    for wp in (1, 2):
        say(f"wave pairs seed {kw['seed']} wave_pairs={wp}")
        call = s.Call(dict(P.params, wave_pairs=wp, head_blocks_per_group=bpg), P.arrays)
        outs.append([None if t is None else t.clone() for t in call.run()])
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
    assert torch.equal(outs[0][0], outs[1][0])
    assert (outs[0][1] is None) == (outs[1][1] is None)
    if outs[0][1] is not None:
        assert torch.equal(outs[0][1], outs[1][1])
    rows = list(range(P.query_rows))
    res = dict(O=outs[1][0].float().cpu().numpy(), status=0,
               lse=None if outs[1][1] is None else outs[1][1].cpu().numpy())
    check_outputs(P, res, oracle.forward(P, rows=rows), rows)


@pytest.mark.parametrize("fmt", ["bf16", "int8_packed"])
def test_merge_rounds_for_every_split_count_bitwise(fmt):
    """A 1024-position TopK list cut into 1 to 16 splits: the merge by the
    last split to arrive loads its partials in rounds whose shape follows the
    split count (and differs between one wave and a wave pair per 16 heads);
    for each split count both kernels give the same bits, and the oracle's
    result on every row."""
    import sparse_shared_kv_amd as s
    kw = dict(family="sfa", max_kv=3000, topk=1024, num_heads_q=128, rope_head_dim=64,
              separate_v=False, sinks=True, lse=True)
    if fmt != "bf16":
        kw.update(kv_dtype=fmt)
    P = synth.random_tiny(1200, **kw)
    rows = list(range(P.query_rows))
    ref = oracle.forward(P, rows=rows)
    for split_rows, nsplit in ((1024, 1), (512, 2), (352, 3), (256, 4), (224, 5), (160, 7),
                               (128, 8), (96, 11), (64, 16)):
        assert -(-1024 // split_rows) == nsplit
        outs = []
        for wp in (1, 2):
            say(f"merge rounds {fmt} split_rows={split_rows} wave_pairs={wp}")
            call = s.Call(dict(P.params, split_rows=split_rows, wave_pairs=wp), P.arrays)
            outs.append([None if t is None else t.clone() for t in call.run()])
            torch.cuda.synchronize()
            assert int(call.status.item()) == 0
        assert torch.equal(outs[0][0], outs[1][0]), split_rows
        assert torch.equal(outs[0][1], outs[1][1]), split_rows
        res = dict(O=outs[1][0].float().cpu().numpy(), status=0, lse=outs[1][1].cpu().numpy())
        check_outputs(P, res, ref, rows)


def test_wave_pairs_on_random_tiny_cases_bitwise():
    """Random small problems of every family and layout (bf16 and float16):
    wave pairs forced on and off give the same bits."""
    import sparse_shared_kv_amd as s
    for seed in range(960, 1000):
        P = synth.random_tiny(seed, kv_dtype="fp16" if seed % 3 == 0 else "bf16", max_kv=800)
        outs = []
        for wp in (1, 2):
            say(f"random tiny seed {seed} wave_pairs={wp}")
            call = s.Call(dict(P.params, wave_pairs=wp), P.arrays)
            outs.append([None if t is None else t.clone() for t in call.run()])
            torch.cuda.synchronize()
            assert int(call.status.item()) == 0, seed
        assert torch.equal(outs[0][0], outs[1][0]), seed
        if outs[0][1] is not None:
            assert torch.equal(outs[0][1], outs[1][1]), seed


def test_wave_pairs_at_full_size_bitwise():
    """The prefill call example's TopK workload (4 x 128 query tokens, 64
    heads) on wave pairs: the same bits as without."""
    import sparse_shared_kv_amd as s
    P = synth.make_workload("csa_prefill")
    outs = []
    for wp in (2, 1):
        say(f"csa_prefill wave_pairs={wp}")
        call = s.Call(dict(P.params, wave_pairs=wp), P.arrays)
        outs.append([None if t is None else t.clone() for t in call.run()])
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
    assert torch.equal(outs[0][0], outs[1][0])


# ---------------------------------------------------------------------------
# four waves, two workgroups per CU (rope-free 16-bit rows, V = K nope)
# ---------------------------------------------------------------------------

W4_CASES = [
    # float16, 48 heads (the fourth wave holds none), 300-row windows in two splits
    dict(seed=990, family="swa", num_heads_q=48, batch=64, max_q=8, max_kv=900, win=(300, 0),
         kv_dtype="fp16", layout_q="TND", lse=True),
    # every visible compressed row, sinks, 64 heads
    dict(seed=991, family="hca", num_heads_q=64, batch=48, max_q=8, max_kv=1200, win=(127, 0),
         cmp_ratio=4, lse=True, sinks=True),
    # TopK compressed rows, 16 heads (one wave holds heads), no LSE output
    dict(seed=992, family="csa", num_heads_q=16, batch=40, max_q=12, max_kv=1500, win=(63, 0),
         cmp_ratio=2, topk=400, lse=False),
]


@pytest.mark.parametrize("kw", W4_CASES, ids=lambda k: str(k["seed"]))
def test_four_wave_kernel_matches_eight_waves_bitwise(kw):
    """Calls of at least 256 (row, split) units with rope-free rows whose V
    is the K nope run on four waves, two workgroups per CU (the workspace
    shows it: 64 heads of partial per row and split instead of 128); split
    rows are merged by the last split to arrive.  Same bits as the
    eight-wave kernel (forced through head_blocks_per_group) and the
    oracle's result on sampled rows."""
    import sparse_shared_kv_amd as s
    P = synth.random_tiny(**kw)
    ws = lambda **o: s.sfmla_workspace_size(s.make_params(dict(P.params, **o), P.arrays))
    assert 0 < ws() < ws(head_blocks_per_group=4)
    outs = []
    for bpg in (0, 4):
        say(f"four waves seed {kw['seed']} head_blocks_per_group={bpg}")
        call = s.Call(dict(P.params, head_blocks_per_group=bpg), P.arrays)
        outs.append([None if t is None else t.clone() for t in call.run()])
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
    assert torch.equal(outs[0][0], outs[1][0])
    if outs[0][1] is not None:
        assert torch.equal(outs[0][1], outs[1][1])
    n = P.query_rows
    rows = sorted({0, 1, n // 3, n // 2, n - 2, n - 1})
    res = dict(O=outs[0][0].float().cpu().numpy(), status=0,
               lse=None if outs[0][1] is None else outs[0][1].cpu().numpy())
    check_outputs(P, res, oracle.forward(P, rows=rows), rows)


# ---------------------------------------------------------------------------
# packed KV with a value tensor of codes (KV quant blog, 参数说明 value: a
# 512-wide NoPE value tensor in the key's format; its tiles take the key
# row's scales)
# ---------------------------------------------------------------------------

PKV_CASES = [
    dict(seed=1100, kv_dtype="int8_packed", rope_head_dim=64, num_heads_q=16),
    dict(seed=1101, kv_dtype="fp8_e4m3_packed", rope_head_dim=0, num_heads_q=1),
    dict(seed=1102, kv_dtype="int8_packed", rope_head_dim=0, num_heads_q=20, duplicates=True),
    dict(seed=1103, kv_dtype="fp8_e4m3_packed", rope_head_dim=64, num_heads_q=128),
    # long lists: several splits and a ragged last tile
    dict(seed=1104, kv_dtype="int8_packed", rope_head_dim=64, num_heads_q=128, max_kv=2100,
         topk=2048, sinks=True, lse=True),
    dict(seed=1105, kv_dtype="fp8_e4m3_packed", rope_head_dim=0, num_heads_q=64, max_kv=1700,
         topk=1030, layout_q="TND", layout_kv="PA_BSND", block_size=64),
]


def _both_kernels(P):
    """Outputs of the eight-wave kernel (wave pairs off) and of wave pairs."""
    import sparse_shared_kv_amd as s
    outs = []
    for wp in (1, 2):
        call = s.Call(dict(P.params, wave_pairs=wp), P.arrays)
        outs.append([None if t is None else t.clone() for t in call.run()])
        torch.cuda.synchronize()
        assert int(call.status.item()) == 0
    return outs


@pytest.mark.parametrize("kw", PKV_CASES, ids=lambda k: str(k["seed"]))
def test_packed_value_tensor_parity(kw):
    """Both packed kernels with a value tensor against the oracle on every
    row, and the same bits from either."""
    P = synth.random_tiny(family="sfa", separate_v=True, **kw)
    say("packed value tensor seed", kw["seed"])
    outs = _both_kernels(P)
    assert torch.equal(outs[0][0], outs[1][0])
    if outs[0][1] is not None:
        assert torch.equal(outs[0][1], outs[1][1])
    rows = list(range(P.query_rows))
    ref = oracle.forward(P, rows=rows)
    for o in outs:
        res = dict(O=o[0].float().cpu().numpy(), status=0,
                   lse=None if o[1] is None else o[1].cpu().numpy())
        check_outputs(P, res, ref, rows)


@pytest.mark.parametrize("fmt,rope", [("int8_packed", 64), ("fp8_e4m3_packed", 0)])
def test_packed_value_tensor_of_the_key_codes_equals_aliased_bitwise(fmt, rope):
    """A value tensor holding the key rows' own codes gives the bits of V
    taken from the packed key rows, on both kernels."""
    P = synth.random_tiny(1110 + rope, family="sfa", kv_dtype=fmt, rope_head_dim=rope,
                          num_heads_q=128, max_kv=1200, topk=1000, separate_v=False)
    V = P.copy()
    V.params["separate_v"] = True
    V.arrays["ori_v"] = np.ascontiguousarray(P.arrays["ori_kv"][:, :512])
    say("packed value tensor = key codes", fmt, rope)
    a, b = _both_kernels(P), _both_kernels(V)
    for x, y in zip(a, b):
        assert torch.equal(x[0], y[0])
        if x[1] is not None:
            assert torch.equal(x[1], y[1])
