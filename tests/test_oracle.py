"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: the
independent brute-force checker, library routines (scipy logsumexp, torch
SDPA, torch's bf16 / fp8 dtypes), closed forms, invariants the pages imply,
and hand-derived row sets for the pages' example calls (tests/golden).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from oracle import decode as odec
from oracle.bruteforce import brute_force
from synth import Problem
from synth.problem import normal_bf16, pack_rows, bf16_bits

from helpers import logical, place, unplace_o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _close(a, b, tol=1e-10):
    a = np.asarray(a); b = np.asarray(b)
    fa, fb = np.isfinite(a), np.isfinite(b)
    assert (fa == fb).all(), "finite masks differ"
    if fa.any():
        err = np.abs(a[fa] - b[fa]).max()
        assert err <= tol, err


# --------------------------------------------------------------------------
# decoders
# --------------------------------------------------------------------------

def test_fp8_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = odec.fp8_e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # closed forms of the OCP definition
    assert ours[0x38] == 1.0 and ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9
    assert ours[0xFE] == -448.0 and np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_bf16_decoder_matches_torch():
    g = np.random.default_rng(0)
    bits = g.integers(0, 1 << 16, size=100000, dtype=np.uint32).astype(np.uint16)
    ours = odec.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_fp16_decoder_matches_torch_all_codes():
    codes = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.float16).double().numpy()
    got = odec.fp16_to_f64(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert (both_nan | (got == ref)).all()
    assert np.array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


def test_int8_decoder():
    codes = np.arange(256, dtype=np.uint8)
    assert np.array_equal(odec.int8_to_f64(codes),
                          torch.from_numpy(codes).view(torch.int8).double().numpy())


# --------------------------------------------------------------------------
# P1: brute force on tiny inputs, every family / layout / format
# --------------------------------------------------------------------------

CASES = []
for s in range(48):
    CASES.append(dict(seed=s))
for s in range(12):
    CASES.append(dict(seed=100 + s, family="sfa",
                      kv_dtype=["int8_packed", "fp8_e4m3_packed"][s % 2],
                      rope_head_dim=[0, 64][(s // 2) % 2]))
for s in range(6):
    CASES.append(dict(seed=200 + s, dist="p4", family=["csa", "hca", "swa"][s % 3]))
for s in range(4):
    CASES.append(dict(seed=300 + s, family=["csa", "sfa"][s % 2], duplicates=True))
for s in range(8):                                  # float16 q / kv / output
    CASES.append(dict(seed=500 + s, kv_dtype="fp16", family=["swa", "csa", "hca", "sfa"][s % 4],
                      dist=["normal", "p4"][(s // 4) % 2]))
for s in range(9):                                  # block-wise TopK (R18)
    CASES.append(dict(seed=400 + s, family="sfa", sparse_block_size=[2, 4, 16][s % 3],
                      max_kv=90, duplicates=bool(s % 4 == 3)))
for s in range(6):                                  # packed rows with a value tensor (R20)
    CASES.append(dict(seed=600 + s, family="sfa", separate_v=True,
                      kv_dtype=["int8_packed", "fp8_e4m3_packed"][s % 2],
                      rope_head_dim=[0, 64][(s // 2) % 2], duplicates=bool(s == 5)))


@pytest.mark.parametrize("kw", CASES, ids=lambda k: "-".join("%s" % v for v in k.values()))
def test_bruteforce_agrees(kw):
    P = synth.random_tiny(**kw)
    r = oracle.forward(P)
    O, L = brute_force(P)
    _close(r["O"], O, 1e-9)
    _close(r["lse"], L, 1e-9)


# --------------------------------------------------------------------------
# P2: LSE closed form against scipy's logsumexp
# --------------------------------------------------------------------------

def test_lse_against_scipy_logsumexp():
    P = synth.random_tiny(7, family="csa", sinks=True, max_kv=48, num_heads_q=3)
    r = oracle.forward(P)
    q_all = P.arrays["q"]
    for row, phys in r["lists"].items():
        if len(phys) == 0:
            continue
        ori = P.arrays["ori_kv"]; cmp = P.arrays["cmp_kv"]
        rows = [cmp[p & ~int(oracle.CMP_BIT)] if p & int(oracle.CMP_BIT) else ori[p] for p in phys]
        K = torch.from_numpy(np.stack(rows).view(np.int16)).view(torch.bfloat16).double().numpy()
        q = torch.from_numpy(q_all[row].view(np.int16)).view(torch.bfloat16).double().numpy()
        S = P.params["softmax_scale"] * (q @ K.T)
        ref = scipy.special.logsumexp(S, axis=1)
        np.testing.assert_allclose(r["lse"][row], ref, rtol=0, atol=1e-12)
        ref_tot = scipy.special.logsumexp(np.concatenate([S, P.arrays["sinks"].astype(np.float64)[:, None]], 1), axis=1)
        np.testing.assert_allclose(r["lse_total"][row], ref_tot, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P3: uniform attention (q = 0): O = mean of the selected V rows, LSE = log n
# --------------------------------------------------------------------------

def test_uniform_attention_swa_decode_closed_form():
    P = synth.make_workload("swa_decode")
    P.arrays["q"] = np.zeros_like(P.arrays["q"])
    r = oracle.forward(P)
    kv = odec.bf16_to_f64(P.arrays["ori_kv"]).reshape(2, 512, 512)
    for b in range(2):
        # window (127, 0) at position 511 keeps positions 384..511
        mean = kv[b, 384:512].mean(axis=0)
        assert np.abs(r["O"][b] - mean[None, :]).max() < 1e-12
        assert np.abs(r["lse"][b] - math.log(128)).max() < 1e-12


def test_uniform_attention_with_sink():
    P = synth.random_tiny(11, family="hca", sinks=True, num_heads_q=4)
    P.arrays["q"] = np.zeros_like(P.arrays["q"])
    r = oracle.forward(P)
    sig = P.arrays["sinks"].astype(np.float64)
    for row, phys in r["lists"].items():
        n = len(phys)
        if n == 0:
            continue
        _, V = oracle.attention._rows_kv(P, phys)
        mean = V.mean(axis=0)
        expect = mean[None, :] * (n / (n + np.exp(sig)))[:, None]
        assert np.abs(r["O"][row] - expect).max() < 1e-12
        assert np.abs(r["lse"][row] - math.log(n)).max() < 1e-12


# --------------------------------------------------------------------------
# P4: SWA with a window at least as long as the context == dense causal
# attention (torch SDPA, float64, CPU)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["BSND", "TND"])
def test_wide_window_equals_sdpa_causal(layout):
    L = logical(3, q_lens=[24, 17], ori_lens=[24, 17], qn=3, sinks=False, win=(127, 0))
    P = place(L, layout, layout)
    r = oracle.forward(P)
    outs = unplace_o(P, r["O"], L)
    for b in range(2):
        q = torch.from_numpy(L["q"][b].view(np.int16)).view(torch.bfloat16).double()      # (n, h, d)
        k = torch.from_numpy(L["ori"][b].view(np.int16)).view(torch.bfloat16).double()    # (n, d)
        qh = q.permute(1, 0, 2)                                                           # (h, n, d)
        kh = k[None].expand(qh.shape[0], -1, -1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qh, kh, kh, is_causal=True, scale=P.params["softmax_scale"])
        assert np.abs(outs[b] - ref.permute(1, 0, 2).numpy()).max() < 1e-12


# --------------------------------------------------------------------------
# P5: CSA whose TopK lists every visible compressed row == HCA
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ratio", [1, 2, 4])
def test_full_topk_csa_equals_hca(ratio):
    L = logical(5, q_lens=[5, 3, 9], ori_lens=[30, 11, 40], qn=2, ratio=ratio, win=(3, 0))
    hca = place(L, "TND", "TND")
    csa = hca.copy()
    K = 64
    idx = np.full((hca.query_rows, 1, K), -1, np.int32)
    # the CP example's generator: indices 0 .. cmp_end-1 with
    # cmp_end = min(cmp_len, (q_pos + 1) // cmp_ratio), q_pos = ori_len - q_len + row
    row = 0
    for b in range(3):
        for i in range(L["q_lens"][b]):
            q_pos = L["ori_lens"][b] - L["q_lens"][b] + i
            end = min(L["cmp_lens"][b], (q_pos + 1) // ratio)
            idx[row, 0, :end] = np.arange(end)
            row += 1
    csa.arrays["cmp_sparse_indices"] = idx
    csa.params["cmp_topk"] = K
    a, c = oracle.forward(hca), oracle.forward(csa)
    assert np.array_equal(a["O"], c["O"]) and np.array_equal(a["lse"], c["lse"])


# --------------------------------------------------------------------------
# P6 / P7: block-table permutation and layout invariance
# --------------------------------------------------------------------------

@pytest.mark.parametrize("family", ["swa", "hca", "csa", "sfa"])
def test_layout_and_block_permutation_invariance(family):
    kw = dict(q_lens=[3, 1, 4], ori_lens=[37, 9, 50], qn=3)
    if family in ("hca", "csa"):
        kw["ratio"] = 4
    if family == "csa":
        kw["cmp_topk"] = 9
    if family == "sfa":
        kw.update(ori_topk=20, ori_mode=3, win=(-1, -1), rope=64)
    L = logical(9, **kw)
    ref = None
    for lq, lk, bs, seed in [("BSND", "BSND", 0, 0), ("TND", "TND", 0, 0),
                             ("BSND", "PA_BSND", 4, 1), ("BSND", "PA_BSND", 4, 2),
                             ("TND", "PA_BSND", 16, 3), ("TND", "PA_BSND", 1, 4)]:
        P = place(L, lq, lk, bs=bs or 4, seed=seed)
        r = oracle.forward(P)
        per_b = unplace_o(P, r["O"], L)
        lse_b = unplace_o(P, r["lse"], L)
        if ref is None:
            ref = (per_b, lse_b)
        else:
            for b in range(3):
                assert np.array_equal(per_b[b], ref[0][b]), (lq, lk, bs, seed)
                assert np.array_equal(lse_b[b], ref[1][b])


# --------------------------------------------------------------------------
# P8: context-parallel query split (the API page's CP example)
# --------------------------------------------------------------------------

def _cp_problem(q, ori, cmp, q_lens, ori_lens, cmp_lens, res, sinks):
    def cu(x):
        return np.concatenate([[0], np.cumsum(x)]).astype(np.int32)
    K = 8
    rows = sum(q_lens)
    idx = np.full((rows, 1, K), -1, np.int32)
    base = 0
    for ql, ol, cl in zip(q_lens, ori_lens, cmp_lens):
        for r in range(ql):
            q_pos = ol - ql + r
            end = min(cl, (q_pos + 1) // 4)
            idx[base + r, 0, :end] = np.arange(end)
        base += ql
    params = dict(num_heads_q=q.shape[1], num_heads_kv=1, head_dim=512, rope_head_dim=0,
                  batch_size=len(q_lens), layout_q="TND", layout_kv="TND", q_s=0, q_t=rows,
                  ori_kv_s=0, cmp_kv_s=0, ori_block_size=0, cmp_block_size=0,
                  max_seqlen_q=max(q_lens), max_seqlen_ori_kv=max(ori_lens),
                  max_seqlen_cmp_kv=max(cmp_lens), ori_topk=0, cmp_topk=K, cmp_ratio=4,
                  ori_mask_mode=4, cmp_mask_mode=3, ori_win_left=127, ori_win_right=0,
                  has_ori_kv=True, has_cmp_kv=True, kv_dtype="bf16", separate_v=False,
                  softmax_scale=1 / math.sqrt(512), return_softmax_lse=True)
    arrays = dict(q=q, ori_kv=ori, cmp_kv=cmp, cu_seqlens_q=cu(q_lens), cu_seqlens_ori_kv=cu(ori_lens),
                  cu_seqlens_cmp_kv=cu(cmp_lens), cmp_residual_kv=np.asarray(res, np.int32),
                  cmp_sparse_indices=idx, sinks=sinks)
    return Problem("cp", 0, params, arrays)


def test_cp_split_invariance():
    ss = np.random.SeedSequence(77).spawn(4)
    q = normal_bf16(ss[0], (34, 4, 512))
    ori = normal_bf16(ss[1], (34, 512))
    cmp = normal_bf16(ss[2], (8, 512))
    sinks = np.random.default_rng(ss[3]).standard_normal(4).astype(np.float32)
    g = oracle.forward(_cp_problem(q, ori, cmp, [16, 18], [16, 18], [4, 4], [0, 2], sinks))
    r0 = oracle.forward(_cp_problem(np.concatenate([q[0:16], q[16:24]]), np.concatenate([ori[0:16], ori[16:24]]),
                                    np.concatenate([cmp[0:4], cmp[4:6]]), [16, 8], [16, 8], [4, 2], [0, 0], sinks))
    r1 = oracle.forward(_cp_problem(q[24:34], ori[16:34], cmp[4:8], [10], [18], [4], [2], sinks))
    seq1 = np.concatenate([r0["O"][16:24], r1["O"]])
    assert np.array_equal(g["O"][:16], r0["O"][:16])
    assert np.array_equal(g["O"][16:34], seq1)


# --------------------------------------------------------------------------
# P9: sink closed form; P12: split / merge
# --------------------------------------------------------------------------

def test_sink_closed_form():
    P = synth.random_tiny(21, family="csa", sinks=True, num_heads_q=4)
    Pn = P.copy()
    del Pn.arrays["sinks"]
    a, b = oracle.forward(P), oracle.forward(Pn)
    sig = P.arrays["sinks"].astype(np.float64)
    for row in a["lists"]:
        if len(a["lists"][row]) == 0:
            continue
        w = 1.0 / (1.0 + np.exp(sig - b["lse"][row]))     # sigmoid(LSE - sigma)
        assert np.abs(a["O"][row] - b["O"][row] * w[:, None]).max() < 1e-12
        assert np.array_equal(a["lse"][row], b["lse"][row])       # LSE excludes the sink
    Pm = P.copy()
    Pm.arrays["sinks"] = np.full_like(P.arrays["sinks"], -1e30)
    c = oracle.forward(Pm)
    assert np.abs(c["O"] - b["O"]).max() < 1e-15


def test_split_merge_equals_unsplit():
    g = np.random.default_rng(5)
    q = g.standard_normal((5, 512 + 64))
    K = g.standard_normal((300, 576)) * 2
    V = K[:, :512]
    sinks = g.standard_normal(5)
    O, lse, _ = oracle.attend(q, K, V, 0.05, sinks)
    cuts = [0, 7, 8, 150, 151, 300]
    parts = [oracle.attend(q, K[a:b], V[a:b], 0.05, None) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(oracle.attend(q, K[:0], V[:0], 0.05, None))      # an empty part
    Om, lm = oracle.combine([p[0] for p in parts], [p[1] for p in parts], sinks)
    assert np.abs(Om - O).max() < 1e-12 and np.abs(lm - lse).max() < 1e-12


# --------------------------------------------------------------------------
# P11: packed rows == float rows holding the dequantised values
# --------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["int8_packed", "fp8_e4m3_packed"])
@pytest.mark.parametrize("rope", [0, 64])
def test_packed_equals_float_on_dequantised_values(fmt, rope):
    P = synth.random_tiny(31, family="sfa", kv_dtype=fmt, rope_head_dim=rope, num_heads_q=3)
    rows = P.arrays["ori_kv"].copy()
    n = rows.shape[0]
    # power-of-two scales make code * scale exact in bf16
    so = 512 + 2 * rope
    exps = np.random.default_rng(1).integers(-8, 3, size=(n, 4))
    rows[:, so:so + 16] = (2.0 ** exps).astype("<f4").view(np.uint8).reshape(n, 16)
    P.arrays["ori_kv"] = rows
    codes = torch.from_numpy(rows[:, :512].copy())
    x = (codes.view(torch.int8) if fmt == "int8_packed" else codes.view(torch.float8_e4m3fn)).double()
    deq = x * torch.from_numpy(np.repeat(2.0 ** exps, 128, axis=1))
    parts = [deq.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)]
    if rope:
        parts.append(rows[:, 512:512 + 2 * rope].copy().view(np.uint16))
    F = P.copy()
    F.params["kv_dtype"] = "bf16"
    F.arrays["ori_kv"] = np.concatenate(parts, axis=1)
    assert np.array_equal(deq.to(torch.bfloat16).double().numpy(), deq.numpy())  # exact in bf16
    a, b = oracle.forward(P), oracle.forward(F)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])


@pytest.mark.parametrize("fmt", ["int8_packed", "fp8_e4m3_packed"])
@pytest.mark.parametrize("rope", [0, 64])
def test_packed_value_tensor_of_the_key_codes_equals_the_aliased_value(fmt, rope):
    """A value tensor holding the key rows' own 512 codes gives the same
    result, bit for bit, as taking V from the packed key rows (KV quant blog,
    参数说明 value: key and value may be the same packed cache)."""
    P = synth.random_tiny(41, family="sfa", kv_dtype=fmt, rope_head_dim=rope, num_heads_q=3,
                          separate_v=False)
    V = P.copy()
    V.params["separate_v"] = True
    V.arrays["ori_v"] = np.ascontiguousarray(P.arrays["ori_kv"][:, :512])
    a, b = oracle.forward(P), oracle.forward(V)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])
    # a value tensor with other codes changes O but not the scores' LSE
    W = V.copy()
    W.arrays["ori_v"] = np.ascontiguousarray(W.arrays["ori_v"][::-1])
    c = oracle.forward(W)
    assert np.array_equal(a["lse"], c["lse"]) and not np.allclose(a["O"], c["O"])


@pytest.mark.parametrize("fmt", ["int8_packed", "fp8_e4m3_packed"])
@pytest.mark.parametrize("rope", [0, 64])
def test_packed_value_tensor_equals_float_value_on_dequantised_codes(fmt, rope):
    """Value codes scaled by the key row's per-tile scales: with power-of-two
    scales the products are exact in bf16, so the packed problem equals the
    bf16 problem with a separate V of those products (the bf16 separate-V
    path is pinned by brute force and SDPA)."""
    P = synth.random_tiny(43, family="sfa", kv_dtype=fmt, rope_head_dim=rope, num_heads_q=3,
                          separate_v=True)
    rows = P.arrays["ori_kv"].copy()
    n = rows.shape[0]
    so = 512 + 2 * rope
    exps = np.random.default_rng(2).integers(-8, 3, size=(n, 4))
    rows[:, so:so + 16] = (2.0 ** exps).astype("<f4").view(np.uint8).reshape(n, 16)
    P.arrays["ori_kv"] = rows
    dt = torch.int8 if fmt == "int8_packed" else torch.float8_e4m3fn
    scale = torch.from_numpy(np.repeat(2.0 ** exps, 128, axis=1))
    kx = torch.from_numpy(rows[:, :512].copy()).view(dt).double() * scale
    vx = torch.from_numpy(np.ascontiguousarray(P.arrays["ori_v"])).view(dt).double() * scale
    for t in (kx, vx):
        assert np.array_equal(t.to(torch.bfloat16).double().numpy(), t.numpy())   # exact
    parts = [kx.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)]
    if rope:
        parts.append(rows[:, 512:512 + 2 * rope].copy().view(np.uint16))
    F = P.copy()
    F.params["kv_dtype"] = "bf16"
    F.arrays["ori_kv"] = np.concatenate(parts, axis=1)
    F.arrays["ori_v"] = vx.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    a, b = oracle.forward(P), oracle.forward(F)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])


def test_packer_roundtrip_int8():
    g = np.random.default_rng(0)
    v = g.standard_normal((50, 512)).astype(np.float32)
    rows = pack_rows(v, None, "int8")
    _, deq = odec.decode_packed(rows, 0, "int8_packed")
    # per-tile error bound of rounding to the nearest code: scale / 2
    amax = np.abs(v.reshape(50, 4, 128)).max(axis=2)
    bound = np.repeat(amax / 127.0, 128, axis=1) / 2 + 1e-6
    assert (np.abs(deq - v) <= bound).all()


# --------------------------------------------------------------------------
# golden row sets of the API page's example calls
# --------------------------------------------------------------------------

def _golden_problem(case):
    p = dict(num_heads_q=1, num_heads_kv=1, head_dim=512, rope_head_dim=0, batch_size=1,
             layout_q="BSND", layout_kv="BSND", q_s=0, q_t=0, ori_kv_s=0, cmp_kv_s=0,
             ori_block_size=0, cmp_block_size=0, max_seqlen_q=0, max_seqlen_ori_kv=0,
             max_seqlen_cmp_kv=0, ori_topk=0, cmp_topk=0, cmp_ratio=1, ori_mask_mode=4,
             cmp_mask_mode=0, ori_win_left=-1, ori_win_right=-1, has_ori_kv=True,
             has_cmp_kv=False, kv_dtype="bf16", separate_v=False, softmax_scale=1.0,
             return_softmax_lse=True)
    p.update(case["params"])
    a = {}
    src = case["arrays"]
    for k in ("cu_seqlens_q", "cu_seqlens_ori_kv", "cu_seqlens_cmp_kv", "cmp_residual_kv"):
        if k in src:
            a[k] = np.asarray(src[k], np.int32)
    if p["layout_q"] == "BSND":
        rows = p["q_s"]
        n_ori = p["ori_kv_s"]
        n_cmp = p["cmp_kv_s"]
    else:
        rows = int(a["cu_seqlens_q"][-1])
        n_ori = int(a["cu_seqlens_ori_kv"][-1])
        n_cmp = int(a["cu_seqlens_cmp_kv"][-1]) if "cu_seqlens_cmp_kv" in a else 0
    a["q"] = np.zeros((rows, 1, 512), np.uint16)
    a["ori_kv"] = np.zeros((n_ori, 512), np.uint16)
    if p["has_cmp_kv"]:
        a["cmp_kv"] = np.zeros((max(1, n_cmp), 512), np.uint16)
    if p["cmp_topk"]:
        idx = np.full((rows, 1, p["cmp_topk"]), -1, np.int32)
        if "cmp_sparse_indices_first" in src:
            first = np.asarray(src["cmp_sparse_indices_first"])
            idx[:, 0, :first.shape[1]] = first
        else:       # the CP example's make_cmp_sparse_indices
            ql = int(a["cu_seqlens_q"][1]); ol = int(a["cu_seqlens_ori_kv"][1]); cl = int(a["cu_seqlens_cmp_kv"][1])
            for r in range(ql):
                end = min(cl, (ol - ql + r + 1) // p["cmp_ratio"])
                idx[r, 0, :end] = np.arange(end)
        a["cmp_sparse_indices"] = idx
    p["q_t"] = rows
    return Problem(case["name"], 0, p, a), rows


with open(os.path.join(GOLDEN, "page_examples.json")) as _f:
    GOLDEN_CASES = json.load(_f)["cases"]


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=lambda c: c["name"])
def test_golden_row_sets(case):
    P, rows = _golden_problem(case)
    for row, b, i in oracle.query_rows(P):
        ori, cmp, phys = oracle.resolve_rows(P, row, b, i)
        exp_ori, exp_cmp = [], []
        for lo, hi in case["expected"]["ori"]:
            exp_ori += list(range(lo, eval(str(hi), {"min": min}, {"i": i}) + 1))
        for lo, hi in case["expected"]["cmp"]:
            exp_cmp += list(range(lo, eval(str(hi), {"min": min}, {"i": i}) + 1))
        assert ori == exp_ori, (case["name"], i)
        assert cmp == exp_cmp, (case["name"], i)


def test_swa_decode_workload_has_128_rows():
    P = synth.make_workload("swa_decode")
    r = oracle.forward(P)
    for b in range(2):
        assert r["lists"][b].tolist() == list(range(b * 512 + 384, b * 512 + 512))


def test_inconsistent_residual_rejected():
    P = synth.random_tiny(3, family="hca", masks=(4, 3))
    P.arrays["cmp_residual_kv"] = (P.arrays["cmp_residual_kv"] + 1) % max(2, P.params["cmp_ratio"] + 1)
    if P.params["cmp_ratio"] == 1:
        P.arrays["cmp_residual_kv"][:] = 1
    with pytest.raises(ValueError):
        oracle.forward(P)


@pytest.mark.parametrize("fmt", ["int8_packed", "fp8_e4m3_packed"])
def test_rope_free_rows_equal_zero_rope_rows(fmt):
    """A 528-byte row (no rope) and a 656-byte row whose rope is zero are the
    same key and value (SparseAttnSharedkv README, 参数说明: the packed row
    holds the rope between the codes and the scales only when rope is used)."""
    import copy
    P = synth.random_tiny(611, family="sfa", kv_dtype=fmt, rope_head_dim=64, num_heads_q=4,
                          max_kv=60)
    P656 = copy.deepcopy(P)
    P656.arrays["ori_kv"] = P656.arrays["ori_kv"].copy()
    P656.arrays["ori_kv"][:, 512:640] = 0
    P528 = copy.deepcopy(P656)
    P528.params["rope_head_dim"] = 0
    P528.arrays["ori_kv"] = np.ascontiguousarray(
        np.concatenate([P656.arrays["ori_kv"][:, :512], P656.arrays["ori_kv"][:, 640:656]], axis=1))
    P528.arrays["q"] = np.ascontiguousarray(P656.arrays["q"][..., :512])
    a = oracle.forward(P656)
    b = oracle.forward(P528)
    assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["lse"], b["lse"])
    # and the rope does matter when it is not zero
    c = oracle.forward(P)
    assert not np.allclose(c["O"], a["O"])



@pytest.mark.parametrize("sbs", [2, 8])
def test_block_topk_covering_the_prefix_equals_sdpa_causal(sbs):
    """Block-wise TopK (R18) whose entries are every block up to the query's
    block, under the causal mode, is dense causal attention (torch SDPA)."""
    P = synth.random_tiny(431, family="sfa", layout_q="TND", layout_kv="TND", batch=1,
                          q_lens=[5], ori_lens=[37], num_heads_q=3, sparse_block_size=sbs,
                          masks=(3, 0), sinks=False, separate_v=False, rope_head_dim=0)
    K = -(-37 // sbs)
    idx = np.full((5, 1, K), -1, dtype=np.int32)
    rng = np.random.default_rng(5)
    for i in range(5):
        blocks = rng.permutation(np.arange((37 - 5 + i) // sbs + 1))   # any slot order
        idx[i, 0, :len(blocks)] = blocks
    P.arrays["ori_sparse_indices"] = idx
    P.params["ori_topk"] = K
    r = oracle.forward(P)
    q = torch.from_numpy(P.arrays["q"].view(np.int16)).view(torch.bfloat16).double()       # (5, h, d)
    k = torch.from_numpy(P.arrays["ori_kv"].view(np.int16)).view(torch.bfloat16).double()  # (37, d)
    qh = q.permute(1, 0, 2)
    kh = k[None].expand(qh.shape[0], -1, -1).contiguous()
    mask = torch.ones(5, 37, dtype=torch.bool).tril(diagonal=37 - 5)   # right-down causal
    ref = torch.nn.functional.scaled_dot_product_attention(
        qh, kh, kh, attn_mask=mask, scale=P.params["softmax_scale"])
    assert np.abs(r["O"] - ref.permute(1, 0, 2).numpy()).max() < 1e-12
