"""Independent brute-force checker for tiny inputs (test infrastructure).

A second formulation of the same operator, written apart from the oracle
modules and sharing no code with them:

* visibility is evaluated as a weight for *every* logical position of each
  KV side (weight = 1 for a window / all-rows rule, = the number of times the
  position occurs in the TopK list for an index rule), using the pages'
  inequalities written out directly (band: p - j <= win_left and
  j - p <= win_right; compressed causal: j < min(cmp_len, (p + 1) // ratio),
  the CP example's index generator);
* logical -> physical rows come from a table built per batch for all
  positions at once;
* stored values are decoded with torch's own dtypes (bfloat16,
  float8_e4m3fn) rather than bit arithmetic;
* attention is the weighted softmax sum_j w_j e^{s_j} v_j /
  (sum_j w_j e^{s_j} + e^{sigma}), with the sink as one more column of value 0.

Only for tiny problems: Python loops over every position.
"""

from __future__ import annotations

import numpy as np
import torch


def _f16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.float16).to(torch.float64).numpy()


def _elem(P):
    return _f16 if P.params["kv_dtype"] == "fp16" else _bf16


def _bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def _packed(rows, rope, fmt):
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    codes = torch.from_numpy(rows[:, :512].copy())
    if fmt == "int8_packed":
        x = codes.view(torch.int8).to(torch.float64).numpy()
    else:
        x = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc_at = 512 + 2 * rope
    sc = torch.from_numpy(rows[:, sc_at:sc_at + 16].copy()).view(torch.float32)
    sc = sc.to(torch.float64).numpy().reshape(n, 4)
    v = np.concatenate([x[:, t * 128:(t + 1) * 128] * sc[:, t:t + 1] for t in range(4)], axis=1)
    if rope:
        rb = rows[:, 512:512 + 2 * rope].copy().view(np.uint16)
        k = np.concatenate([v, _bf16(rb)], axis=1)
    else:
        k = v
    return k, v


def _phys_table(P, side, b, n):
    p, a = P.params, P.arrays
    lay = p["layout_kv"]
    if lay == "BSND":
        return b * int(p[side + "_kv_s"]) + np.arange(n)
    if lay == "TND":
        return int(a["cu_seqlens_%s_kv" % side][b]) + np.arange(n)
    bs = int(p[side + "_block_size"])
    bt = np.asarray(a[side + "_block_table"])[b].astype(np.int64)
    full = (bt[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
    return full[:n]


def _len(P, side, b):
    p, a = P.params, P.arrays
    if a.get("seqused_%s_kv" % side) is not None:
        return int(a["seqused_%s_kv" % side][b])
    if p["layout_kv"] == "TND":
        cu = a["cu_seqlens_%s_kv" % side]
        return int(cu[b + 1]) - int(cu[b])
    return int(p[side + "_kv_s"])


def _decode(P, side, phys):
    p = P.params
    rope = int(p["rope_head_dim"])
    src = np.asarray(P.arrays[side + "_kv"])[phys]
    if p["kv_dtype"] in ("bf16", "fp16"):
        k = _elem(P)(src[:, :512 + rope])
        if side == "ori" and p.get("separate_v"):
            v = _elem(P)(np.asarray(P.arrays["ori_v"])[phys][:, :512])
        else:
            v = k[:, :512]
        return k, v
    k, v = _packed(src, rope, p["kv_dtype"])
    if side == "ori" and p.get("separate_v"):
        # value codes (dtype of the key's codes), scaled per 128 columns by the
        # key row's scales
        vc = torch.from_numpy(np.ascontiguousarray(np.asarray(P.arrays["ori_v"])[phys][:, :512],
                                                   dtype=np.uint8))
        dt = torch.int8 if p["kv_dtype"] == "int8_packed" else torch.float8_e4m3fn
        x = vc.view(dt).to(torch.float64)
        sc_at = 512 + 2 * rope
        sc = torch.from_numpy(np.ascontiguousarray(src[:, sc_at:sc_at + 16], dtype=np.uint8))
        sc = sc.view(torch.float32).to(torch.float64).reshape(-1, 4)
        v = (x.reshape(-1, 4, 128) * sc[:, :, None]).reshape(-1, 512).numpy()
    return k, v


def brute_force(P):
    """Returns (O (R, q_n, 512), lse (R, q_n)) for every query row."""
    p, a = P.params, P.arrays
    q_all = np.asarray(a["q"])
    R, qn = q_all.shape[:2]
    O = np.zeros((R, qn, 512))
    LSE = np.full((R, qn), -np.inf)
    scale = float(p["softmax_scale"])
    sinks = a.get("sinks")
    B = int(p["batch_size"])
    for b in range(B):
        if p["layout_q"] == "BSND":
            n_rows, base = int(p["q_s"]), b * int(p["q_s"])
        else:
            cu = a["cu_seqlens_q"]
            n_rows, base = int(cu[b + 1]) - int(cu[b]), int(cu[b])
        used = int(a["seqused_q"][b]) if a.get("seqused_q") is not None else n_rows
        n_ori = _len(P, "ori", b)
        n_cmp = _len(P, "cmp", b) if p["has_cmp_kv"] else 0
        for i in range(used):
            row = base + i
            pos = n_ori - used + i
            w_parts, k_parts, v_parts = [], [], []
            # original side
            w = np.zeros(n_ori)
            mode, wl, wr = p["ori_mask_mode"], p["ori_win_left"], p["ori_win_right"]
            for j in range(n_ori):
                if mode == 0:
                    ok = True
                elif mode == 3:
                    ok = not (j > pos)
                else:
                    ok = (wl == -1 or pos - j <= wl) and (wr == -1 or j - pos <= wr)
                if not ok:
                    continue
                if p["ori_topk"] > 0:
                    # entries that select the block holding position j
                    sbs = int(p.get("sparse_block_size", 1))
                    w[j] = np.count_nonzero(np.asarray(a["ori_sparse_indices"])[row, 0] == j // sbs)
                else:
                    w[j] = 1.0
            if n_ori:
                k, v = _decode(P, "ori", _phys_table(P, "ori", b, n_ori))
                w_parts.append(w); k_parts.append(k); v_parts.append(v)
            # compressed side
            if n_cmp:
                r = int(p["cmp_ratio"])
                res = int(a["cmp_residual_kv"][b]) if a.get("cmp_residual_kv") is not None else 0
                pos_c = n_cmp * r + res - used + i
                limit = n_cmp if p["cmp_mask_mode"] == 0 else min(n_cmp, (pos_c + 1) // r)
                w = np.zeros(n_cmp)
                for j in range(n_cmp):
                    if j >= limit:
                        continue
                    if p["cmp_topk"] > 0:
                        w[j] = np.count_nonzero(np.asarray(a["cmp_sparse_indices"])[row, 0] == j)
                    else:
                        w[j] = 1.0
                k, v = _decode(P, "cmp", _phys_table(P, "cmp", b, n_cmp))
                w_parts.append(w); k_parts.append(k); v_parts.append(v)
            if not w_parts:
                continue
            W = np.concatenate(w_parts)
            if not (W > 0).any():
                continue
            Kall = np.concatenate(k_parts)[W > 0]
            Vall = np.concatenate(v_parts)[W > 0]
            Wv = W[W > 0]
            q = _elem(P)(q_all[row])
            for h in range(qn):
                s = scale * (Kall @ q[h])
                top = s.max()
                if sinks is not None:
                    top = max(top, float(sinks[h]))
                e = Wv * np.exp(s - top)
                den = e.sum() + (np.exp(float(sinks[h]) - top) if sinks is not None else 0.0)
                O[row, h] = (e[:, None] * Vall).sum(axis=0) / den
                LSE[row, h] = np.log(e.sum()) + top
    return O, LSE
