"""Dense softmax attention over the resolved rows (oracle; test infrastructure).

Formula and LSE: sparse_flash_mla API page, 功能说明 (O = softmax(Q K~^T
scale) V~, LSE = log sum exp(S - max S) + max S with S = Q K~^T scale).
Sinks: same page, 参数说明 sinks (a learnable per-head virtual offset, fp32,
shape (q_n,)).

Readings (also in the design notes):
  R8   the sink sigma_h is one extra logit in the scaled-score domain whose
       value vector is zero: it enters the softmax normaliser only.  No sink
       tensor means no such logit (a zero sink is not "no sink").
  R9   the returned LSE is the page's formula over S = Q K~^T scale alone, so
       it excludes the sink; lse_total includes it.
  R10  an empty row set gives O = 0 and LSE = -inf.
  R11  merging partial results over disjoint parts of the row set follows
       from the definition: LSE = log sum_i exp(lse_i),
       O = sum_i exp(lse_i) O_i / (sum_i exp(lse_i) + exp(sigma)).
"""

from __future__ import annotations

import numpy as np

from . import decode as _decode
from .decode import bf16_to_f64, decode_packed, decode_packed_value


def elem_to_f64(P):
    """Decoder of the 16-bit q / kv elements: float16 when kv_dtype is
    fp16 (q, kv and the output then share that type), bfloat16 otherwise."""
    return _decode.fp16_to_f64 if P.params["kv_dtype"] == "fp16" else bf16_to_f64
from .resolve import CMP_BIT, query_rows, resolve_rows


def _rows_kv(P, phys: np.ndarray):
    """Decode the gathered rows -> (K (n, d_qk), V (n, 512)) in float64.

    bf16 KV: K is the row's first 512 + rope values; V is the first 512
    (K~ = V~, API page 功能说明) unless the original side carries its own
    value tensor (SparseFlashAttention page, 参数说明 value).  Packed KV:
    decode.decode_packed, or with a value tensor of codes,
    decode.decode_packed_value (KV quant blog, 参数说明 value).
    """
    p = P.params
    rope = int(p["rope_head_dim"])
    d_qk = 512 + rope
    n = phys.shape[0]
    K = np.zeros((n, d_qk))
    V = np.zeros((n, 512))
    is_cmp = (phys & CMP_BIT) != 0
    rid = phys & ~CMP_BIT
    for side, sel in (("ori", ~is_cmp), ("cmp", is_cmp)):
        if not sel.any():
            continue
        src = np.asarray(P.arrays["%s_kv" % side])
        rows = src[rid[sel]]
        if p["kv_dtype"] in ("bf16", "fp16"):
            dec = elem_to_f64(P)
            k = dec(rows[:, :d_qk])
            if side == "ori" and p.get("separate_v"):
                v = dec(np.asarray(P.arrays["ori_v"])[rid[sel]][:, :512])
            else:
                v = k[:, :512]
        else:
            k, v = decode_packed(rows, rope, p["kv_dtype"])
            if side == "ori" and p.get("separate_v"):
                v = decode_packed_value(np.asarray(P.arrays["ori_v"])[rid[sel]], rows, rope,
                                        p["kv_dtype"])
        K[sel] = k
        V[sel] = v
    return K, V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, sinks=None):
    """Softmax attention of every head of one query row over n rows.

    q (q_n, d_qk), K (n, d_qk), V (n, d_v) float64.  Returns (O (q_n, d_v),
    lse (q_n,) without the sink, lse_total (q_n,) with it).
    """
    qn = q.shape[0]
    n = K.shape[0]
    sig = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    if n == 0:                                                  # R10
        lse_tot = np.full(qn, -np.inf) if sig is None else sig.copy()
        return np.zeros((qn, V.shape[1])), np.full(qn, -np.inf), lse_tot
    S = (q @ K.T) * scale
    m_s = S.max(axis=1)
    lse = np.log(np.exp(S - m_s[:, None]).sum(axis=1)) + m_s     # LSE formula
    m = m_s if sig is None else np.maximum(m_s, sig)             # R8
    E = np.exp(S - m[:, None])
    denom = E.sum(axis=1)
    if sig is not None:
        denom = denom + np.exp(sig - m)
    O = (E @ V) / denom[:, None]
    lse_tot = np.log(denom) + m
    return O, lse, lse_tot


def forward(P, rows=None):
    """The whole operator on a Problem (q, KV sources, lengths, indices).

    rows: optional iterable of query-row ids to compute (others stay 0 /
    -inf); all rows by default.  Returns dict with O (R, q_n, 512), lse and
    lse_total (R, q_n), and 'lists' mapping each computed row to its resolved
    physical-id list (canonical order).
    """
    p = P.params
    q_all = np.asarray(P.arrays["q"])
    R, qn = q_all.shape[0], q_all.shape[1]
    sinks = P.arrays.get("sinks")
    O = np.zeros((R, qn, 512))
    lse = np.full((R, qn), -np.inf)
    lse_tot = np.full((R, qn), -np.inf)
    lists = {}
    want = None if rows is None else set(int(r) for r in rows)
    for row, b, i in query_rows(P):
        if want is not None and row not in want:
            continue
        _, _, phys = resolve_rows(P, row, b, i)
        lists[row] = phys
        K, V = _rows_kv(P, phys)
        q = elem_to_f64(P)(q_all[row])
        o, l1, l2 = attend(q, K, V, float(p["softmax_scale"]), sinks)
        O[row], lse[row], lse_tot[row] = o, l1, l2
    return dict(O=O, lse=lse, lse_total=lse_tot, lists=lists)


def combine(part_o: np.ndarray, part_lse: np.ndarray, sinks=None):
    """Merge partial results over disjoint parts of one row set (R11).

    part_o (n_parts, q_n, d) are each part's normalised outputs without the
    sink, part_lse (n_parts, q_n) their LSEs (-inf for an empty part).
    Returns (O (q_n, d), lse (q_n,) without the sink).
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    m = part_lse.max(axis=0)
    sig = None if sinks is None else np.asarray(sinks, dtype=np.float64)
    mm = m if sig is None else np.maximum(m, sig)
    safe = np.where(np.isfinite(mm), mm, 0.0)
    w = np.exp(part_lse - safe[None, :])
    total = w.sum(axis=0)
    denom = total + (0.0 if sig is None else np.exp(sig - safe))
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(total[:, None] > 0,
                     (w[:, :, None] * part_o).sum(axis=0) / denom[:, None], 0.0)
        lse = np.where(total > 0, np.log(total) + safe, -np.inf)
    return O, lse
