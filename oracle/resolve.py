"""Which KV rows each query attends to (oracle; test infrastructure).

Follows the sparse_flash_mla API page (参数说明 and 约束说明 tables, the CP
切分示例 example) for the original / compressed KV, and the
SparseFlashAttention and kv_quant_sparse_flash_attention pages for the
token-wise TopK form over one KV.

Readings of points the pages leave open (each is also listed in the design
notes):
  R1  query positions are right-down aligned: query row i of a batch whose
      valid query count is q_used sits at p = ori_len - q_used + i (the CP
      example derives the q start as ori_prefix_len - q_len).
  R2  window mode 4 keeps [p - win_left, p + win_right], inclusive, clipped to
      [0, ori_len); -1 means unbounded on that side.
  R3  compressed row j is causally visible iff (j + 1) * cmp_ratio <= p_c + 1
      with p_c = cmp_len * cmp_ratio + residual - q_used + i (the CP example's
      cmp_end = min(cmp_len, (q_pos + 1) // cmp_ratio)); consistent inputs
      have p_c == p and the oracle rejects inputs where they differ.
  R4  a TopK index is kept iff it is >= 0 and passes its side's mask
      predicate; -1 and masked entries are dropped; kept indices keep their
      slot order and their multiplicity.
  R5  the token-wise TopK form (one KV, sparse_mode 0/3) is the original-KV
      side with a TopK index list: mode 0 keeps v < kv_len, mode 3 keeps
      v <= p.
  R6  query rows past seqused_q attend to nothing (output 0, LSE -inf).
  R7  block-table entries are >= 0 block ids.
  R18 block-wise TopK (sparse_block_size s > 1, SparseFlashAttention README
      参数说明 sparseBlockSize; kv_quant_sparse_flash_attention blog 参数说明
      sparse_block_size): entry v selects tokens v*s .. v*s + s - 1, which
      share that selection; each of them still passes the side's mask
      predicate on its own.  Entries keep slot order, tokens ascend within
      an entry.
"""

from __future__ import annotations

import numpy as np

# Physical row ids of compressed-KV rows carry this bit in the resolved lists.
CMP_BIT = np.int64(1) << np.int64(62)


def _arr(P, key):
    a = P.arrays.get(key)
    return None if a is None else np.asarray(a)


def batch_lengths(P, b: int) -> dict:
    """Per-batch lengths (API page 参数说明: cu_seqlens_*, seqused_*,
    cmp_residual_kv; 约束说明 SeqLengths and Paged Attention groups).

    q_len: BSND -> q_s; TND -> cu_seqlens_q difference.  q_used: seqused_q if
    given, else q_len.  ori_len: seqused_ori_kv if given (required for PA),
    else the TND difference or the BSND sequence dimension.  cmp_len:
    seqused_cmp_kv if given (it overrides), else the same rule.
    """
    p = P.params
    if p["layout_q"] == "BSND":
        q_len = int(p["q_s"])
    else:
        cu = _arr(P, "cu_seqlens_q")
        q_len = int(cu[b + 1] - cu[b])
    sq = _arr(P, "seqused_q")
    q_used = int(sq[b]) if sq is not None else q_len
    if not 0 <= q_used <= q_len:
        raise ValueError("seqused_q out of range")

    def kv_len(side):
        su = _arr(P, "seqused_%s_kv" % side)
        if su is not None:
            return int(su[b])
        lay = p["layout_kv"]
        if lay == "TND":
            cu = _arr(P, "cu_seqlens_%s_kv" % side)
            return int(cu[b + 1] - cu[b])
        if lay == "BSND":
            return int(p["%s_kv_s" % side])
        raise ValueError("PA layout needs seqused_%s_kv" % side)

    ori_len = kv_len("ori")
    cmp_len = kv_len("cmp") if p["has_cmp_kv"] else 0
    res = _arr(P, "cmp_residual_kv")
    residual = int(res[b]) if res is not None else 0
    return dict(q_len=q_len, q_used=q_used, ori_len=ori_len,
                cmp_len=cmp_len, residual=residual)


def query_rows(P):
    """Every query row as (row, b, i): BSND rows are b*q_s + i, TND rows are
    cu_seqlens_q[b] + i (API page 参数说明: q shapes)."""
    p = P.params
    out = []
    for b in range(int(p["batch_size"])):
        if p["layout_q"] == "BSND":
            for i in range(int(p["q_s"])):
                out.append((b * int(p["q_s"]) + i, b, i))
        else:
            cu = _arr(P, "cu_seqlens_q")
            for i in range(int(cu[b + 1] - cu[b])):
                out.append((int(cu[b]) + i, b, i))
    return out


def ori_visible(mode: int, j: int, p: int, n: int, left: int, right: int) -> bool:
    """Original-KV mask predicate (API page 参数说明 ori_mask_mode,
    ori_win_left / ori_win_right): 0 no mask, 3 right-down causal, 4 band."""
    if not 0 <= j < n:
        return False
    if mode == 0:
        return True
    if mode == 3:
        return j <= p
    if mode == 4:
        lo_ok = left < 0 or j >= p - left
        hi_ok = right < 0 or j <= p + right
        return lo_ok and hi_ok
    raise ValueError("ori_mask_mode %d" % mode)


def cmp_visible(mode: int, j: int, p_c: int, n: int, ratio: int) -> bool:
    """Compressed-KV mask predicate (API page 参数说明 cmp_mask_mode; the CP
    example's index generator): 0 no mask, 3 right-down causal in original
    token units, i.e. row j covers tokens [j*r, (j+1)*r) and is visible once
    all of them are at or before the query."""
    if not 0 <= j < n:
        return False
    if mode == 0:
        return True
    if mode == 3:
        return (j + 1) * ratio <= p_c + 1
    raise ValueError("cmp_mask_mode %d" % mode)


def block_tokens(v: int, sbs: int) -> list:
    """Token positions selected by TopK entry v when entries select blocks of
    sbs consecutive tokens (R18): v*sbs .. v*sbs + sbs - 1."""
    return [v * sbs + u for u in range(sbs)]


def physical_row(P, side: str, b: int, j: int) -> int:
    """Logical position j of batch b -> physical row of the side's KV tensor.

    BSND (b, S, 1, d): b*S + j.  TND (t, 1, d): cu_seqlens[b] + j.  PA_BSND
    (blocks, block_size, 1, d): block_table[b, j // bs] * bs + j % bs (API
    page 参数说明 ori_kv / cmp_kv shapes and the block tables).
    """
    p = P.params
    lay = p["layout_kv"]
    if lay == "BSND":
        return b * int(p["%s_kv_s" % side]) + j
    if lay == "TND":
        return int(_arr(P, "cu_seqlens_%s_kv" % side)[b]) + j
    bs = int(p["%s_block_size" % side])
    table = _arr(P, "%s_block_table" % side)
    return int(table[b, j // bs]) * bs + j % bs


def resolve_rows(P, row: int, b: int, i: int):
    """The resolved KV list of one query row, in canonical order.

    Returns (ori logical positions, cmp logical positions, physical ids) where
    the physical ids are int64, compressed rows tagged with CMP_BIT.  Order:
    the original-KV rows (ascending for window rules, slot order for TopK),
    then the compressed rows (ascending for HCA, slot order for CSA).  The two
    parts are concatenated without removing overlaps: an original token and a
    compressed row covering it are separate KV entries (API page 功能说明:
    K~ is made of the window part of ori_kv and the compressed part of cmp_kv).
    """
    p = P.params
    L = batch_lengths(P, b)
    if i >= L["q_used"]:
        return [], [], np.zeros(0, dtype=np.int64)
    pos = L["ori_len"] - L["q_used"] + i                       # R1
    mode = int(p["ori_mask_mode"])
    left, right = int(p["ori_win_left"]), int(p["ori_win_right"])
    ori = []
    if int(p["ori_topk"]) > 0:                                  # R4, R5
        idx = _arr(P, "ori_sparse_indices")[row, 0]
        sbs = int(p.get("sparse_block_size", 1))                # R18
        for v in idx.tolist():
            if v < 0:
                continue
            for j in block_tokens(v, sbs):
                if ori_visible(mode, j, pos, L["ori_len"], left, right):
                    ori.append(j)
    else:
        for j in range(L["ori_len"]):                           # R2
            if ori_visible(mode, j, pos, L["ori_len"], left, right):
                ori.append(j)
    cmp = []
    if p["has_cmp_kv"]:
        r = int(p["cmp_ratio"])
        cmode = int(p["cmp_mask_mode"])
        pos_c = L["cmp_len"] * r + L["residual"] - L["q_used"] + i
        if cmode == 3 and pos_c != pos:
            raise ValueError("cmp_len*cmp_ratio + residual must equal the original length")
        if int(p["cmp_topk"]) > 0:                              # R4 (CSA)
            idx = _arr(P, "cmp_sparse_indices")[row, 0]
            for v in idx.tolist():
                if v >= 0 and cmp_visible(cmode, v, pos_c, L["cmp_len"], r):
                    cmp.append(v)
        else:                                                   # R3 (HCA)
            for j in range(L["cmp_len"]):
                if cmp_visible(cmode, j, pos_c, L["cmp_len"], r):
                    cmp.append(j)
    phys = [physical_row(P, "ori", b, j) for j in ori]
    phys += [physical_row(P, "cmp", b, j) | int(CMP_BIT) for j in cmp]
    return ori, cmp, np.asarray(phys, dtype=np.int64)
