"""C ABI checks that need no GPU: the library loads, exports every function
include/sfmla.h declares, and rejects invalid parameters on the host before
anything is launched (API page 约束说明 rules decidable from shapes)."""

import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

s = pytest.importorskip("sparse_shared_kv_amd")


def _declared():
    text = open(os.path.join(ROOT, "include", "sfmla.h")).read()
    return sorted(set(re.findall(r"^\s*(?:sfmla_status|const char\*)\s+(sfmla_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for need in ("sfmla_metadata", "sfmla_forward", "sfmla_combine", "sfmla_metadata_size",
                 "sfmla_workspace_size", "sfmla_debug_resolve", "sfmla_last_error",
                 "sfmla_version"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_shared_kv_amd", "libsfmla.so"))
    for name in _declared():
        assert hasattr(lib, name), name


def test_struct_layout_matches_header(tmp_path):
    """Every field offset of the ctypes mirror equals the C compiler's."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sfmla.h"', "int main(void){"]
    for cname, cls in (("sfmla_params", s.Params), ("sfmla_lengths", s.Lengths),
                       ("sfmla_tensors", s.Tensors)):
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in cls._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0;}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(ln.split() for ln in subprocess.run([str(exe)], capture_output=True, text=True,
                                                   check=True).stdout.splitlines())
    for cname, cls in (("sfmla_params", s.Params), ("sfmla_lengths", s.Lengths),
                       ("sfmla_tensors", s.Tensors)):
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got["%s.%s" % (cname, f)]) == getattr(cls, f).offset, (cname, f)


def _params(**over):
    P = synth.make_workload("swa_decode")
    p = s.make_params(P.params, P.arrays)
    for k, v in over.items():
        setattr(p, k, v)
    return p


BAD = [
    ("head_dim", 576, "head_dim"),
    ("num_heads_kv", 2, "num_heads_kv"),
    ("num_heads_q", 0, "num_heads_q"),
    ("num_heads_q", 129, "num_heads_q"),
    ("rope_head_dim", 32, "rope_head_dim"),
    ("layout_kv", 1, "non-paged"),
    ("q_t", 3, "q_t"),
    ("ori_mask_mode", 2, "ori_mask_mode"),
    ("ori_win_left", -2, "window"),
    ("cmp_topk", 8, "cmp_topk"),
    ("cmp_ratio", 4, "cmp_ratio"),
    ("kv_dtype", 7, "kv_dtype"),
    ("batch_size", 0, "batch_size"),
    ("ori_sparse_block_size", 0, "ori_sparse_block_size"),
    ("ori_sparse_block_size", 3, "ori_sparse_block_size"),
    ("ori_sparse_block_size", 256, "ori_sparse_block_size"),
    ("ori_sparse_block_size", 4, "needs an ori TopK list"),
    ("ori_kv_rows", 2 ** 31 - 1, "ori_kv_rows"),
]


@pytest.mark.parametrize("field,value,msg", BAD, ids=[b[0] + "=" + str(b[1]) for b in BAD])
def test_invalid_params_rejected_on_host(field, value, msg):
    p = _params(**{field: value})
    with pytest.raises(s.SfmlaError) as e:
        s.sfmla_metadata_size(p)
    assert e.value.status == 1 and msg in str(e.value)


def test_packed_value_tensor_needs_the_token_wise_form():
    """A value tensor with packed KV (KV quant blog, 参数说明 value) is taken for
    the token-wise TopK form; with a compressed KV it is refused on the host,
    without it the parameters are valid."""
    P = synth.random_tiny(3, family="sfa", kv_dtype="int8_packed", rope_head_dim=64,
                          separate_v=True)
    p = s.make_params(P.params, P.arrays)
    assert p.has_separate_v == 1
    s.sfmla_metadata_size(p)
    Q = synth.random_tiny(4, family="csa", kv_dtype="int8_packed", rope_head_dim=64)
    q = s.make_params(Q.params, Q.arrays)
    q.has_separate_v = 1
    with pytest.raises(s.SfmlaError, match="token-wise TopK"):
        s.sfmla_metadata_size(q)


def test_paged_needs_block_table_and_seqused():
    P = synth.make_workload("csa_decode_paged")
    p = s.make_params(P.params, P.arrays)
    p.has_seqused_ori_kv = 0
    with pytest.raises(s.SfmlaError, match="seqused_ori_kv"):
        s.sfmla_workspace_size(p)
    p = s.make_params(P.params, P.arrays)
    p.has_cmp_residual_kv = 0
    with pytest.raises(s.SfmlaError, match="cmp_residual_kv"):
        s.sfmla_workspace_size(p)


def test_metadata_rejects_missing_lengths_without_launching():
    P = synth.make_workload("hca_varlen")
    p = s.make_params(P.params, P.arrays)
    lens = s.Lengths()          # TND layouts need cu_seqlens: nothing given
    with pytest.raises(s.SfmlaError, match="cu_seqlens_q"):
        s._abi.check(s._abi.load().sfmla_metadata(ctypes.byref(p), ctypes.byref(lens),
                                                   ctypes.c_void_p(16), 10 ** 6, None))


def test_metadata_buffer_too_small():
    p = _params()
    lens = s.Lengths()
    with pytest.raises(s.SfmlaError) as e:
        s._abi.check(s._abi.load().sfmla_metadata(ctypes.byref(p), ctypes.byref(lens),
                                                   ctypes.c_void_p(16), 4, None))
    assert e.value.status == 3


def test_metadata_buffer_misaligned():
    p = _params()
    lens = s.Lengths()
    with pytest.raises(s.SfmlaError, match="16-byte aligned"):
        s._abi.check(s._abi.load().sfmla_metadata(ctypes.byref(p), ctypes.byref(lens),
                                                   ctypes.c_void_p(20), 10 ** 6, None))


def test_forward_rejects_bad_tensors_without_launching():
    p = _params()
    t = s.Tensors()
    lib = s._abi.load()
    # no q pointer
    st = lib.sfmla_forward(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(16), 10 ** 6,
                           ctypes.c_float(0.1), None, 0, None)
    assert st == 1 and b"q must be" in lib.sfmla_last_error()
    t.q = 4096
    t.ori_kv = 4096
    t.ori_kv_stride = 1000          # shorter than a 512-value bf16 row
    st = lib.sfmla_forward(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(16), 10 ** 6,
                           ctypes.c_float(0.1), None, 0, None)
    assert st == 1 and b"ori_kv_stride" in lib.sfmla_last_error()
    t.ori_kv_stride = 1024
    t.attention_out = 4096
    t.softmax_lse = 8192
    st = lib.sfmla_forward(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(16), 10 ** 6,
                           ctypes.c_float(float("inf")), None, 0, None)
    assert st == 1 and b"finite" in lib.sfmla_last_error()


def test_workspace_sizes():
    for name, expect_split in [("swa_decode", False), ("csa_decode_paged", True),
                               ("sfa_mla_rope", True)]:
        P = synth.make_workload(name) if name != "sfa_mla_rope" else _small_sfa()
        p = s.make_params(P.params, P.arrays)
        ws = s.sfmla_workspace_size(p)
        assert (ws > 0) == expect_split, name


def _expected_workspace(P):
    """The split partials' workspace from the host's documented policy:
    512-row splits for rows of 2 KB or more, 256 otherwise; head groups of
    1/2/4/8 16-head blocks on eight waves, halved while the grid would have
    fewer than 256 workgroups; calls with fewer than 256 (row, split)
    units on wave pairs (groups of 1/2/4 pairs);
    one bf16 partial (1 KB per padded head) and one fp32 LSE per (row,
    split, padded head)."""
    p = P.params
    packed = p["kv_dtype"] not in ("bf16", "fp16")
    rope = p["rope_head_dim"]
    row = 512 + 2 * rope + 16 if packed else 2 * (512 + rope) + (1024 if p["separate_v"] else 0)
    base = 512 if row >= 2048 else 256
    n = p["ori_topk"] * p["sparse_block_size"] + p["cmp_topk"]   # TopK lists here
    parts = -(-n // base)
    srows = -(-(-(-n // parts)) // 32) * 32 if n > base else base   # even splits
    splits = -(-n // srows)
    if splits <= 1:
        return 0
    blocks = -(-p["num_heads_q"] // 16)
    units = p["q_t"] * splits
    if units < 256:
        # wave pairs: groups of up to 4 pairs of 16 heads, eight waves of
        # 16 heads x 256 columns of partial each
        per = min(4, blocks)
        per = 2 if per == 3 else per
        while per > 1 and units * -(-blocks // per) < 256:
            per //= 2
        heads = -(-blocks // per) * 8 * 8
    else:
        wmax = 8
        per = 1
        while per < wmax and per < blocks:
            per *= 2
        while per > 1 and units * -(-blocks // per) < 256:
            per //= 2
        heads = -(-blocks // per) * wmax * 16
    slots = p["q_t"] * splits * heads
    up = lambda x: -(-x // 256) * 256
    return up(slots * 1024) + up(slots * 4)


def test_workspace_size_follows_split_and_group_policy():
    from synth.workloads import sfa_mla_rope
    cases = [_small_sfa(), sfa_mla_rope(batch=32, q_s=2, kv_len=4096, topk=2048),
             synth.make_workload("c8_packed_int8"), sfa_mla_rope(batch=2, q_s=1, kv_len=4096,
                                                                 topk=1100)]
    for P in cases:
        p = s.make_params(P.params, P.arrays)
        assert s.sfmla_workspace_size(p) == _expected_workspace(P), P.name


def _small_sfa():
    from synth.workloads import sfa_mla_rope
    return sfa_mla_rope(batch=2, q_s=2, kv_len=4096, topk=2048)


def test_combine_rejects_bad_dv():
    lib = s._abi.load()
    st = lib.sfmla_combine(2, ctypes.c_void_p(4096), ctypes.c_void_p(4096), None,
                           ctypes.c_void_p(4096), None, 4, 8, 6, None)
    assert st == 1 and b"dv" in lib.sfmla_last_error()


def test_work_split_overrides_are_validated_and_fingerprinted():
    """split_rows / head_blocks_per_group come from the parameters (never the
    environment): out-of-range values are refused, and a different value
    changes the workspace the library asks for."""
    P = _small_sfa()
    p = s.make_params(P.params, P.arrays)
    base = s.sfmla_workspace_size(p)
    for field, bad in (("split_rows", 48), ("split_rows", 4096), ("head_blocks_per_group", 3)):
        q = s.make_params(P.params, P.arrays)
        setattr(q, field, bad)
        with pytest.raises(s.SfmlaError, match=field):
            s.sfmla_workspace_size(q)
    q = s.make_params(dict(P.params, split_rows=256), P.arrays)
    assert s.sfmla_workspace_size(q) == 2 * base          # 2048 rows: 8 splits instead of 4
    q = s.make_params(dict(P.params, head_blocks_per_group=8), P.arrays)
    assert s.sfmla_workspace_size(q) < base               # one group: no padding per group


def test_environment_does_not_change_the_split(monkeypatch):
    P = _small_sfa()
    p = s.make_params(P.params, P.arrays)
    base = s.sfmla_workspace_size(p)
    monkeypatch.setenv("SFMLA_SPLIT_ROWS", "64")
    monkeypatch.setenv("SFMLA_BPG", "1")
    assert s.sfmla_workspace_size(p) == base


def test_binding_rejects_wrong_dtypes_and_layouts():
    """The binding hands q, index lists, tables and sinks over as bare
    pointers: a transposed view or a wrong dtype is refused instead of being
    read with the wrong layout."""
    import torch
    P = synth.random_tiny(31, family="sfa", layout_q="TND", layout_kv="PA_BSND", num_heads_q=4,
                          sinks=True)
    bad = dict(P.arrays)
    bad["ori_sparse_indices"] = P.arrays["ori_sparse_indices"].astype(np.int64)
    with pytest.raises(s.SfmlaError, match="ori_sparse_indices"):
        s.Call(P.params, bad, device="cpu")
    bad = dict(P.arrays)
    bad["sinks"] = P.arrays["sinks"].astype(np.float64)
    with pytest.raises(s.SfmlaError, match="sinks"):
        s.Call(P.params, bad, device="cpu")
    bad = dict(P.arrays)
    q = torch.from_numpy(P.arrays["q"].view(np.int16))
    bad["q"] = q.transpose(0, 1).contiguous().transpose(0, 1)     # same shape, not contiguous
    with pytest.raises(s.SfmlaError, match="q must be contiguous"):
        s.Call(P.params, bad, device="cpu")
    bad = dict(P.arrays)
    kv = torch.from_numpy(P.arrays["ori_kv"].view(np.int16))
    bad["ori_kv"] = kv.t().contiguous().t()                       # rows not contiguous
    with pytest.raises(s.SfmlaError, match="ori_kv"):
        s.Call(P.params, bad, device="cpu")


def test_block_wise_topk_must_divide_the_page():
    P = synth.random_tiny(5, family="sfa", layout_kv="PA_BSND", block_size=16,
                          sparse_block_size=16)
    p = s.make_params(P.params, P.arrays)
    assert s.sfmla_metadata_size(p) > 0
    p.ori_sparse_block_size = 32                    # does not divide the 16-token page
    with pytest.raises(s.SfmlaError, match="divide ori_block_size"):
        s.sfmla_metadata_size(p)


def test_list_longer_than_the_row_table_allows_is_rejected():
    # 4096 splits of at most 2048 rows per query row
    lib = s._abi.load()
    p = _params(ori_mask_mode=0, ori_win_left=-1, ori_win_right=-1,
                max_seqlen_ori_kv=4096 * 2048 + 1, ori_kv_rows=4096 * 2048 + 1)
    n = ctypes.c_size_t()
    assert lib.sfmla_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 1
    assert b"at most 8388608" in lib.sfmla_last_error()
    p = _params(ori_mask_mode=0, ori_win_left=-1, ori_win_right=-1,
                max_seqlen_ori_kv=4096 * 2048, ori_kv_rows=4096 * 2048)
    assert lib.sfmla_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0


def test_partials_of_one_row_beyond_32_bit_offsets_are_rejected():
    # one 16-head block per group (the override) lays 128 heads out as 8
    # groups of 8 waves: 4096 splits x 1024 padded heads x 1 KB = 2^32
    lib = s._abi.load()
    p = _params(num_heads_q=128, ori_mask_mode=0, ori_win_left=-1, ori_win_right=-1,
                max_seqlen_ori_kv=4096 * 256, ori_kv_rows=4096 * 256, head_blocks_per_group=1)
    n = ctypes.c_size_t()
    assert lib.sfmla_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 1
    assert b"2^31" in lib.sfmla_last_error()
    p.head_blocks_per_group = 0
    assert lib.sfmla_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0


# ---------------------------------------------------------------------------
# query tiles: host rule, metadata size and workspace
# ---------------------------------------------------------------------------

def _meta_ints(P, **over):
    return s.sfmla_metadata_size(s.make_params(dict(P.params, **over), P.arrays))


def test_query_tile_rule_sizes_the_tile_descriptors():
    """Tiles by rule need rule lists, 16-bit rows with rope or a separate V
    (rope-free rows whose V is the K nope take the four-wave kernel), at
    most 64 heads and max_seqlen_q >= 16; the plan then holds one (first
    row, row count) pair per possible tile of the fewest rows (2 by rule,
    the forced count otherwise): (q_t + b (tq - 1)) / tq, at most q_t,
    rounded up to a multiple of 8."""
    base_ints = lambda P: 16 + (16 + 64) * P.params["q_t"]
    up8 = lambda n: (n + 7) // 8 * 8
    bound = lambda P, tq: up8(min(P.params["q_t"], (P.params["q_t"] + P.params["batch_size"] *
                                                    (tq - 1)) // tq))
    for name in ("swa_prefill", "hca_prefill", "swa_prefill_h16"):
        P = synth.make_workload(name)
        assert _meta_ints(P) == base_ints(P), name                    # four-wave rows
        assert _meta_ints(P, rope_head_dim=64) == base_ints(P) + 2 * bound(P, 2), name
        assert _meta_ints(P, rope_head_dim=64, query_tile=1) == base_ints(P), name
        assert _meta_ints(P, query_tile=2) == base_ints(P) + 2 * bound(P, 2), name
    P = synth.make_workload("swa_prefill_h16")
    assert _meta_ints(P, query_tile=8) == base_ints(P) + 2 * bound(P, 8)
    # TopK lists (csa), packed rows and 128 heads are never tiled
    for name in ("csa_prefill", "c8_packed_int8_q32", "hca_varlen_q32", "swa_decode"):
        P = synth.make_workload(name)
        assert _meta_ints(P) == base_ints(P), name
    # forced tiles of 4 rows at 16 heads on a decode-sized batch
    P = synth.make_workload("swa_decode")                 # 2 sequences of one query, 16 heads
    assert _meta_ints(P, query_tile=4) == base_ints(P) + 2 * 8


def test_query_tile_override_is_validated_and_fingerprinted():
    P = synth.make_workload("swa_prefill")                # 64 heads: at most 2 rows per tile
    for bad in (3, 16, -1):
        with pytest.raises(s.SfmlaError, match="query_tile"):
            _meta_ints(P, query_tile=bad)
    for bad in (4, 8):                                    # 4 head blocks x 4 rows > 8 waves
        with pytest.raises(s.SfmlaError, match="query_tile"):
            _meta_ints(P, query_tile=bad)
    C = synth.make_workload("csa_prefill")                # TopK compressed rows
    with pytest.raises(s.SfmlaError, match="query_tile"):
        _meta_ints(C, query_tile=2)
    K = synth.make_workload("c8_packed_int8")             # packed rows
    with pytest.raises(s.SfmlaError, match="query_tile"):
        _meta_ints(K, query_tile=2)


def test_tiled_call_lays_out_split_rows_with_every_head_in_one_group():
    """Rows of sequences that are not tiled (too few queries, or a union too
    long for one split) are split as without tiles, with every head in one
    workgroup: the workspace is that of one head group of 8 waves."""
    P = synth.make_workload("hca_prefill")
    q = s.make_params(dict(P.params, max_seqlen_cmp_kv=4096, query_tile=2), P.arrays)
    ws = s.sfmla_workspace_size(q)
    splits = -(-(128 + 4096) // 256)                     # all-visible rows: 256-row splits
    slots = P.params["q_t"] * splits * 128                # 8 waves x 16 heads
    up = lambda n: (n + 255) // 256 * 256
    assert ws == up(slots * 1024) + up(slots * 4)
    # without tiles (the rule for these rope-free rows) the 64 heads take the
    # four-wave kernel: 4 waves x 16 heads per row and split
    q = s.make_params(dict(P.params, max_seqlen_cmp_kv=4096), P.arrays)
    assert s.sfmla_workspace_size(q) == up(slots // 2 * 1024) + up(slots // 2 * 4)


# ---------------------------------------------------------------------------
# wave pairs: host rule and workspace
# ---------------------------------------------------------------------------

def test_wave_pairs_override_is_validated():
    P = synth.make_workload("csa_prefill")                # bf16, 64 heads, TopK lists
    for bad in (3, -1):
        with pytest.raises(s.SfmlaError, match="wave_pairs"):
            _meta_ints(P, wave_pairs=bad)
    assert _meta_ints(P, wave_pairs=2) == _meta_ints(P, wave_pairs=1)
    _meta_ints(synth.make_workload("sfa_mla_rope"), wave_pairs=2)   # 128 heads: two groups
    _meta_ints(synth.make_workload("c8_packed_int8"), wave_pairs=2)  # packed rows
    # refused where pairs do not apply: query tiles
    with pytest.raises(s.SfmlaError, match="wave_pairs"):
        _meta_ints(synth.make_workload("hca_prefill"), query_tile=2, wave_pairs=2)
    _meta_ints(synth.make_workload("hca_prefill"), wave_pairs=2)


def test_wave_pair_workspace_and_rule():
    """With pairs every wave's partial is 16 heads x 256 columns (the bytes of
    8 heads x 512), eight waves per (row, split, head group): 64 heads of
    partial per group, which holds four pairs.  The rule takes pairs where
    the (row, split) units do not fill the GPU (a decode of 4 rows x 3
    splits), not for csa_prefill (512 rows x 3 splits of its 640-row lists),
    whose 64 heads take the four-wave kernel (4 waves x 16 heads of slots);
    the eight-wave kernel (forced through head_blocks_per_group) lays out
    128 heads, four of its waves only gathering."""
    P = synth.make_workload("csa_prefill")
    ws = lambda **o: s.sfmla_workspace_size(s.make_params(dict(P.params, **o), P.arrays))
    up = lambda n: (n + 255) // 256 * 256
    slots = lambda heads: P.params["q_t"] * 3 * heads
    assert ws(wave_pairs=2) == up(slots(64) * 1024) + up(slots(64) * 4)
    assert ws(wave_pairs=1) == up(slots(64) * 1024) + up(slots(64) * 4)
    assert ws(head_blocks_per_group=4) == up(slots(128) * 1024) + up(slots(128) * 4)
    assert ws() == ws(wave_pairs=1)
    D = synth.make_workload("csa_decode_paged")            # 4 rows, 64 heads
    wd = lambda **o: s.sfmla_workspace_size(s.make_params(dict(D.params, **o), D.arrays))
    assert wd() == wd(wave_pairs=2) != wd(wave_pairs=1)


def test_q_rope_apart_is_validated():
    """query_rope stored apart (SparseFlashAttention README, 参数说明):
    only with rope 64; the binding checks both shapes."""
    import torch
    P = synth.random_tiny(41, family="sfa", rope_head_dim=64, num_heads_q=4)
    q = P.arrays["q"]
    split = dict(P.arrays, q=np.ascontiguousarray(q[..., :512]),
                 q_rope=np.ascontiguousarray(q[..., 512:]))
    s.Call(P.params, split, device="cpu")                       # accepted
    with pytest.raises(s.SfmlaError, match="q must have shape"):
        s.Call(P.params, dict(P.arrays, q_rope=split["q_rope"]), device="cpu")
    with pytest.raises(s.SfmlaError, match="q_rope must have shape"):
        s.Call(P.params, dict(split, q_rope=np.ascontiguousarray(q[..., 512:544])), device="cpu")
    # the library refuses q_rope without rope before anything is launched
    lib = s._abi.load()
    P0 = synth.random_tiny(42, family="sfa", rope_head_dim=0, num_heads_q=4)
    p = s.make_params(P0.params, P0.arrays)
    t = s._abi.Tensors()
    t.q = t.ori_kv = t.attention_out = t.q_rope = 4096
    t.ori_kv_stride = 1024
    t.ori_sparse_indices = 4096
    n = ctypes.c_size_t()
    assert lib.sfmla_metadata_size(ctypes.byref(p), ctypes.byref(n)) == 0
    st = lib.sfmla_forward(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(4096), n.value,
                           ctypes.c_float(0.05), None, 0, None)
    assert st == 1 and b"q_rope" in lib.sfmla_last_error()


@pytest.mark.parametrize("topk", [1024, 1280, 1536, 1792, 2048])
def test_head_grouping_stays_within_one_round_of_workgroups(topk):
    """Packed decode of 8 rows, 128 heads: the heads are spread over head
    groups (wave pairs) only as far as one round of 256 workgroups allows.
    Read back from the workspace size: q_t * splits * heads-as-laid-out
    slots of 1 KB of partial O and one LSE each."""
    P = synth.random_tiny(77, family="sfa", kv_dtype="int8_packed", rope_head_dim=64,
                          num_heads_q=128, max_kv=4096, topk=topk, batch=8, q_lens=[1] * 8,
                          ori_lens=[4096] * 8, layout_q="BSND", layout_kv="PA_BSND",
                          block_size=64, separate_v=False)
    splits = -(-topk // 256)                          # 256-row splits of packed rows
    ws = s.sfmla_workspace_size(s.make_params(P.params, P.arrays))
    slots = 8 * splits
    heads = None
    for h in range(1, 1025):                          # the one padded head count that fits
        o = (slots * h * 1024 + 255) // 256 * 256
        lse = (slots * h * 4 + 255) // 256 * 256
        if o + lse == ws:
            heads = h
            break
    assert heads is not None and heads % 64 == 0, (ws, heads)
    groups = heads // 64                              # eight waves of 8 pair-heads each
    assert slots * groups <= 256, (topk, groups)
    # and the heads are spread as far as that allows (pairs of 16 heads: 8 blocks)
    assert slots * min(8, 2 * groups) > 256 or groups == 8, (topk, groups)
