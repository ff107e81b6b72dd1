"""Test-side helpers: place one logical problem into any q / KV layout."""

from __future__ import annotations

import math

import numpy as np

from synth import Problem
from synth.problem import normal_bf16


def logical(seed, q_lens, ori_lens, qn=4, ratio=None, cmp_topk=0, ori_topk=0,
            rope=0, sinks=True, win=(127, 0), ori_mode=4, cmp_mode=3):
    """Per-batch logical data: q rows, ori rows, cmp rows, index lists."""
    ss = np.random.SeedSequence(seed)
    s_q, s_o, s_c, s_i, s_s = ss.spawn(5)
    g = np.random.default_rng(s_i)
    B = len(q_lens)
    d = 512 + rope
    L = dict(q_lens=list(q_lens), ori_lens=list(ori_lens), qn=qn, rope=rope,
             ratio=ratio, win=win, ori_mode=ori_mode, cmp_mode=cmp_mode,
             cmp_topk=cmp_topk, ori_topk=ori_topk)
    L["q"] = [normal_bf16(s, (q_lens[b], qn, d)) for b, s in enumerate(s_q.spawn(B))]
    L["ori"] = [normal_bf16(s, (max(1, ori_lens[b]), d)) for b, s in enumerate(s_o.spawn(B))]
    if ratio:
        L["cmp_lens"] = [n // ratio for n in ori_lens]
        L["res"] = [n % ratio for n in ori_lens]
        L["cmp"] = [normal_bf16(s, (max(1, L["cmp_lens"][b]), d)) for b, s in enumerate(s_c.spawn(B))]
    if cmp_topk:
        L["cmp_idx"] = []
        for b in range(B):
            rows = np.full((q_lens[b], cmp_topk), -1, np.int32)
            for i in range(q_lens[b]):
                n = L["cmp_lens"][b]
                k = min(n, int(g.integers(0, cmp_topk + 1)))
                rows[i, :k] = g.choice(n, k, replace=False) if k else []
            L["cmp_idx"].append(rows)
    if ori_topk:
        L["ori_idx"] = []
        for b in range(B):
            rows = np.full((q_lens[b], ori_topk), -1, np.int32)
            for i in range(q_lens[b]):
                n = ori_lens[b]
                k = min(n, int(g.integers(1, ori_topk + 1)))
                rows[i, :k] = g.choice(n, k, replace=False)
            L["ori_idx"].append(rows)
    L["sinks"] = np.random.default_rng(s_s).standard_normal(qn).astype(np.float32) if sinks else None
    return L


def place(L, layout_q, layout_kv, bs=4, seed=0):
    """A Problem holding the logical data L in the given layouts."""
    g = np.random.default_rng(seed)
    B = len(L["q_lens"])
    qn, rope = L["qn"], L["rope"]
    d = 512 + rope
    has_cmp = bool(L["ratio"])
    arrays = {}
    params = dict(
        num_heads_q=qn, num_heads_kv=1, head_dim=512, rope_head_dim=rope,
        batch_size=B, layout_q=layout_q, layout_kv=layout_kv, q_s=0, q_t=0,
        ori_kv_s=0, cmp_kv_s=0, ori_block_size=0, cmp_block_size=0,
        max_seqlen_q=max(L["q_lens"]), max_seqlen_ori_kv=max(L["ori_lens"]),
        max_seqlen_cmp_kv=max(L["cmp_lens"]) if has_cmp else 0,
        ori_topk=L["ori_topk"], cmp_topk=L["cmp_topk"],
        cmp_ratio=L["ratio"] or 1, ori_mask_mode=L["ori_mode"],
        cmp_mask_mode=L["cmp_mode"] if has_cmp else 0,
        ori_win_left=L["win"][0], ori_win_right=L["win"][1],
        has_ori_kv=True, has_cmp_kv=has_cmp, kv_dtype="bf16",
        separate_v=False, softmax_scale=1.0 / math.sqrt(d),
        return_softmax_lse=True)

    def q_like(per_batch, width, fill, dtype):
        if layout_q == "BSND":
            qs = max(L["q_lens"])
            out = np.full((B * qs,) + per_batch[0].shape[1:], fill, dtype=dtype)
            for b in range(B):
                out[b * qs:b * qs + L["q_lens"][b]] = per_batch[b]
            return out
        return np.concatenate(per_batch, axis=0).astype(dtype)

    arrays["q"] = q_like(L["q"], None, 0, np.uint16)
    if layout_q == "BSND":
        params["q_s"] = max(L["q_lens"])
        params["q_t"] = B * params["q_s"]
        if any(n != params["q_s"] for n in L["q_lens"]):
            arrays["seqused_q"] = np.asarray(L["q_lens"], np.int32)
    else:
        params["q_t"] = sum(L["q_lens"])
        arrays["cu_seqlens_q"] = np.concatenate([[0], np.cumsum(L["q_lens"])]).astype(np.int32)
    if L.get("cmp_idx") is not None:
        arrays["cmp_sparse_indices"] = q_like([x[:, None, :] for x in L["cmp_idx"]], None, -1, np.int32)
    if L.get("ori_idx") is not None:
        arrays["ori_sparse_indices"] = q_like([x[:, None, :] for x in L["ori_idx"]], None, -1, np.int32)

    def kv(side, rows, lens):
        if layout_kv == "BSND":
            S = max(lens) + 1
            pool = np.zeros((B * S, d), np.uint16)
            for b in range(B):
                pool[b * S:b * S + lens[b]] = rows[b][:lens[b]]
            params[side + "_kv_s"] = S
            arrays["seqused_%s_kv" % side] = np.asarray(lens, np.int32)
        elif layout_kv == "TND":
            pool = np.concatenate([rows[b][:lens[b]] for b in range(B)] + [np.zeros((1, d), np.uint16)])
            arrays["cu_seqlens_%s_kv" % side] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        else:
            need = [max(1, -(-n // bs)) for n in lens]
            total = sum(need) + 2
            perm = g.permutation(total)
            table = np.zeros((B, max(need)), np.int32)
            pool = np.zeros((total * bs, d), np.uint16)
            pos = 0
            for b in range(B):
                for k in range(need[b]):
                    blk = int(perm[pos]); pos += 1
                    table[b, k] = blk
                    lo, hi = k * bs, min(lens[b], (k + 1) * bs)
                    if hi > lo:
                        pool[blk * bs:blk * bs + hi - lo] = rows[b][lo:hi]
            params[side + "_block_size"] = bs
            arrays[side + "_block_table"] = table
            arrays["seqused_%s_kv" % side] = np.asarray(lens, np.int32)
        arrays[side + "_kv"] = pool

    kv("ori", L["ori"], L["ori_lens"])
    if has_cmp:
        kv("cmp", L["cmp"], L["cmp_lens"])
        arrays["cmp_residual_kv"] = np.asarray(L["res"], np.int32)
    if L["sinks"] is not None:
        arrays["sinks"] = L["sinks"]
    return Problem("placed_%s_%s" % (layout_q, layout_kv), seed, params, arrays)


def unplace_o(P, O, L):
    """Per-batch list of the valid query rows of O (any q layout)."""
    out = []
    B = len(L["q_lens"])
    if P.params["layout_q"] == "BSND":
        qs = P.params["q_s"]
        for b in range(B):
            out.append(O[b * qs:b * qs + L["q_lens"][b]])
    else:
        cu = np.concatenate([[0], np.cumsum(L["q_lens"])])
        for b in range(B):
            out.append(O[cu[b]:cu[b + 1]])
    return out
