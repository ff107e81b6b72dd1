"""Workload recipes: the five measured configurations plus small random cases.

Every recipe is seeded; the same (name, seed) always yields the same arrays.
Shapes and distributions follow the workloads the operator pages describe
(sparse_flash_mla examples, the SparseAttnSharedKV example, the QSFA decode
test) at the sizes used for measurement.
"""

from __future__ import annotations

import math

import numpy as np

from .problem import (Problem, banked_rows, bf16_bits, fp16_bits, normal_bf16,
                      packed_rows)


def _seqs(seed, n):
    return np.random.SeedSequence(seed).spawn(n)


def _gen(seq):
    return np.random.Generator(np.random.PCG64(seq))


def _base_params(**kw):
    p = dict(
        num_heads_q=1, num_heads_kv=1, head_dim=512, rope_head_dim=0,
        batch_size=1, layout_q="BSND", layout_kv="BSND", q_s=0, q_t=0,
        ori_kv_s=0, cmp_kv_s=0, ori_block_size=0, cmp_block_size=0,
        max_seqlen_q=0, max_seqlen_ori_kv=0, max_seqlen_cmp_kv=0,
        ori_topk=0, cmp_topk=0, cmp_ratio=1, ori_mask_mode=4,
        cmp_mask_mode=0, ori_win_left=-1, ori_win_right=-1, has_ori_kv=True,
        has_cmp_kv=False, kv_dtype="bf16", separate_v=False,
        softmax_scale=1.0, return_softmax_lse=True, sparse_block_size=1,
    )
    for k, v in kw.items():
        if k not in p:
            raise KeyError(k)
        p[k] = v
    return p


def _prefix(lens):
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


def _paged(g, lens, bs, spare_blocks=1):
    """Random block assignment: returns (block table, number of pool blocks).

    Batch b owns ceil(len_b / bs) blocks drawn from a random permutation of
    the pool; table entries past a batch's own blocks are 0 (never read).
    """
    need = [max(1, -(-int(n) // bs)) for n in lens]
    total = sum(need) + spare_blocks
    perm = g.permutation(total).astype(np.int32)
    width = max(need)
    table = np.zeros((len(lens), width), dtype=np.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb]
        pos += nb
    return table, total


# ---------------------------------------------------------------------------
# The five measured configurations.
# ---------------------------------------------------------------------------

def swa_decode(seed=1):
    """SWA decode: B=2, q_s=1, q_n=16, d=512, BSND; ori_kv length 512,
    window (127, 0); no cmp_kv, no sinks; scale 1/sqrt(512); O and LSE."""
    s_q, s_kv = _seqs(seed, 2)
    B, qs, qn, d, S = 2, 1, 16, 512, 512
    arrays = dict(
        q=normal_bf16(s_q, (B * qs, qn, d)),
        ori_kv=normal_bf16(s_kv, (B * S, d)),
    )
    params = _base_params(
        num_heads_q=qn, batch_size=B, layout_q="BSND", layout_kv="BSND",
        q_s=qs, q_t=B * qs, ori_kv_s=S, max_seqlen_q=qs, max_seqlen_ori_kv=S,
        ori_mask_mode=4, ori_win_left=127, ori_win_right=0, cmp_mask_mode=0,
        cmp_ratio=1, has_cmp_kv=False, softmax_scale=1.0 / math.sqrt(d))
    return Problem("swa_decode", seed, params, arrays,
                   "q, ori_kv ~ N(0,1) bf16; query at position 511")


def _csa_indices(seq, B, C, K):
    g_idx = _gen(seq)
    idx = np.stack([g_idx.choice(C, K, replace=False) for _ in range(B)]).astype(np.int32)
    return idx.reshape(B, 1, K)


def csa_decode_paged(seed=2):
    """CSA decode, paged: B=4, q_n=64, d=512; context 32768, window 128;
    cmp_ratio 4 so 8192 compressed rows; TopK 512 drawn without replacement
    from the 8192 (all visible at position 32767); PA block 128 with random
    permutation block tables; sinks ~ N(0,1)."""
    s_q, s_ori, s_cmp, s_tab, s_idx, s_sink = _seqs(seed, 6)
    B, qn, d, bs, L, C, r, K = 4, 64, 512, 128, 32768, 8192, 4, 512
    g_tab = _gen(s_tab)
    ori_bt = g_tab.permutation(B * L // bs).astype(np.int32).reshape(B, L // bs)
    cmp_blocks = B * L // bs // 4              # pool of 256 blocks
    cmp_bt = g_tab.permutation(cmp_blocks).astype(np.int32).reshape(B, cmp_blocks // B)
    idx = _csa_indices(s_idx, B, C, K)
    arrays = dict(
        q=normal_bf16(s_q, (B, qn, d)),
        ori_kv=banked_rows(s_ori, B * L, lambda s, n: normal_bf16(s, (n, d))),
        cmp_kv=banked_rows(s_cmp, cmp_blocks * bs, lambda s, n: normal_bf16(s, (n, d))),
        ori_block_table=ori_bt, cmp_block_table=cmp_bt,
        seqused_ori_kv=np.full(B, L, np.int32),
        seqused_cmp_kv=np.full(B, C, np.int32),
        cmp_residual_kv=np.zeros(B, np.int32),
        cmp_sparse_indices=idx,
        sinks=_gen(s_sink).standard_normal(qn, dtype=np.float32),
    )
    params = _base_params(
        num_heads_q=qn, batch_size=B, layout_q="BSND", layout_kv="PA_BSND",
        q_s=1, q_t=B, ori_block_size=bs, cmp_block_size=bs, max_seqlen_q=1,
        max_seqlen_ori_kv=L, max_seqlen_cmp_kv=C, cmp_topk=K, cmp_ratio=r,
        ori_mask_mode=4, ori_win_left=127, ori_win_right=0, cmp_mask_mode=3,
        has_cmp_kv=True, softmax_scale=1.0 / math.sqrt(d))
    return Problem("csa_decode_paged", seed, params, arrays,
                   "q, kv ~ N(0,1) bf16; 512 of 8192 compressed rows per query")


def csa_prefill(seed=6):
    """CSA prefill with the shapes of the SparseAttnSharedkv README's call
    example: B=4 sequences of 128 query tokens (TND), q_n=64, d=512, 4096
    cached tokens each in 128-token pages, window (127, 0), cmp_ratio 4 (1024
    compressed rows) with one TopK list of 512 compressed rows drawn from the
    first 1024 - 128 + 1 and shared by every query token, causal cmp mask,
    sinks ~ U(0, 1); q ~ U(-10, 10) and kv ~ U(-5, 10) as in the example."""
    s_q, s_ori, s_cmp, s_tab, s_idx, s_sink = _seqs(seed, 6)
    B, s1, qn, d, bs, L, r, K = 4, 128, 64, 512, 128, 4096, 4, 512
    C = L // r
    g_tab = _gen(s_tab)
    ori_blocks = B * L // bs
    ori_bt = g_tab.permutation(ori_blocks).astype(np.int32).reshape(B, L // bs)
    cmp_blocks = B * ((C + bs - 1) // bs)
    cmp_bt = g_tab.permutation(cmp_blocks).astype(np.int32).reshape(B, cmp_blocks // B)
    one = _gen(s_idx).choice(C - s1 + 1, K, replace=False).astype(np.int32)
    idx = np.broadcast_to(one, (B * s1, 1, K)).copy()
    arrays = dict(
        q=bf16_bits(_gen(s_q).uniform(-10, 10, (B * s1, qn, d)).astype(np.float32)),
        ori_kv=bf16_bits(_gen(s_ori).uniform(-5, 10, (ori_blocks * bs, d)).astype(np.float32)),
        cmp_kv=bf16_bits(_gen(s_cmp).uniform(-5, 10, (cmp_blocks * bs, d)).astype(np.float32)),
        ori_block_table=ori_bt, cmp_block_table=cmp_bt,
        cu_seqlens_q=_prefix([s1] * B),
        seqused_ori_kv=np.full(B, L, np.int32),
        seqused_cmp_kv=np.full(B, C, np.int32),
        cmp_residual_kv=np.zeros(B, np.int32),
        cmp_sparse_indices=idx,
        sinks=_gen(s_sink).uniform(0, 1, qn).astype(np.float32),
    )
    params = _base_params(
        num_heads_q=qn, batch_size=B, layout_q="TND", layout_kv="PA_BSND",
        q_t=B * s1, ori_block_size=bs, cmp_block_size=bs, max_seqlen_q=s1,
        max_seqlen_ori_kv=L, max_seqlen_cmp_kv=C, cmp_topk=K, cmp_ratio=r,
        ori_mask_mode=4, ori_win_left=127, ori_win_right=0, cmp_mask_mode=3,
        has_cmp_kv=True, softmax_scale=1.0 / 24.0)
    return Problem("csa_prefill", seed, params, arrays,
                   "q ~ U(-10,10), kv ~ U(-5,10) bf16; 128 query tokens per sequence")


def rule_prefill(seed=7, family="hca", qn=64):
    """Prefill whose lists are rules, with the shapes of the SparseAttnSharedkv
    README's call example: B=4 sequences of 128 query tokens (TND), d=512,
    4096 cached tokens each in 128-token pages, window (127, 0); "hca" adds
    cmp_ratio 4 (1024 compressed rows) with every causally visible compressed
    row, "swa" has the window only.  q ~ U(-10, 10), kv ~ U(-5, 10), sinks ~
    U(0, 1) as in the example."""
    s_q, s_ori, s_cmp, s_tab, s_sink = _seqs(seed, 5)
    B, s1, d, bs, L, r = 4, 128, 512, 128, 4096, 4
    C = L // r
    g_tab = _gen(s_tab)
    ori_blocks = B * L // bs
    ori_bt = g_tab.permutation(ori_blocks).astype(np.int32).reshape(B, L // bs)
    arrays = dict(
        q=bf16_bits(_gen(s_q).uniform(-10, 10, (B * s1, qn, d)).astype(np.float32)),
        ori_kv=bf16_bits(_gen(s_ori).uniform(-5, 10, (ori_blocks * bs, d)).astype(np.float32)),
        ori_block_table=ori_bt,
        cu_seqlens_q=_prefix([s1] * B),
        seqused_ori_kv=np.full(B, L, np.int32),
        sinks=_gen(s_sink).uniform(0, 1, qn).astype(np.float32),
    )
    hca = family == "hca"
    if hca:
        cmp_blocks = B * ((C + bs - 1) // bs)
        arrays.update(
            cmp_kv=bf16_bits(_gen(s_cmp).uniform(-5, 10, (cmp_blocks * bs, d)).astype(np.float32)),
            cmp_block_table=g_tab.permutation(cmp_blocks).astype(np.int32).reshape(
                B, cmp_blocks // B),
            seqused_cmp_kv=np.full(B, C, np.int32),
            cmp_residual_kv=np.zeros(B, np.int32))
    params = _base_params(
        num_heads_q=qn, batch_size=B, layout_q="TND", layout_kv="PA_BSND",
        q_t=B * s1, ori_block_size=bs, cmp_block_size=bs if hca else 0, max_seqlen_q=s1,
        max_seqlen_ori_kv=L, max_seqlen_cmp_kv=C if hca else 0, cmp_ratio=r if hca else 1,
        ori_mask_mode=4, ori_win_left=127, ori_win_right=0, cmp_mask_mode=3 if hca else 0,
        has_cmp_kv=hca, softmax_scale=1.0 / 24.0)
    name = "%s_prefill" % family + ("" if qn == 64 else "_h%d" % qn)
    return Problem(name, seed, params, arrays,
                   "q ~ U(-10,10), kv ~ U(-5,10) bf16; 128 query tokens per sequence")


def _varlen_lengths(seed):
    (s_len,) = _seqs(seed * 1000 + 7, 1)
    return _gen(s_len).integers(16384, 131072 + 1, size=8).astype(np.int64)


def hca_varlen(seed=3, qps=1):
    """HCA varlen TND: B=8, q_n=128, d=512; contexts ~ U[16384, 131072];
    window 128; cmp_ratio 128 with every causally visible compressed row;
    kv ~ N(0,1), q ~ N(0, 0.5^2); sinks ~ N(0,1); LSE returned.  qps > 1:
    the same contexts with qps query tokens per sequence (the last qps
    positions, each with its own window and compressed-row limit), a
    throughput-mode variant of the decode."""
    s_q, s_ori, s_cmp, s_sink = _seqs(seed, 4)
    B, qn, d, r = 8, 128, 512, 128
    L = _varlen_lengths(seed)
    C = L // r
    arrays = dict(
        q=normal_bf16(s_q, (B * qps, qn, d), std=0.5),
        ori_kv=banked_rows(s_ori, int(L.sum()), lambda s, n: normal_bf16(s, (n, d))),
        cmp_kv=banked_rows(s_cmp, int(C.sum()), lambda s, n: normal_bf16(s, (n, d))),
        cu_seqlens_q=_prefix([qps] * B),
        cu_seqlens_ori_kv=_prefix(L), cu_seqlens_cmp_kv=_prefix(C),
        cmp_residual_kv=(L % r).astype(np.int32),
        sinks=_gen(s_sink).standard_normal(qn, dtype=np.float32),
    )
    params = _base_params(
        num_heads_q=qn, batch_size=B, layout_q="TND", layout_kv="TND", q_t=B * qps,
        max_seqlen_q=qps, max_seqlen_ori_kv=int(L.max()),
        max_seqlen_cmp_kv=int(C.max()), cmp_ratio=r, ori_mask_mode=4,
        ori_win_left=127, ori_win_right=0, cmp_mask_mode=3, has_cmp_kv=True,
        softmax_scale=1.0 / math.sqrt(d))
    name = "hca_varlen" if qps == 1 else "hca_varlen_q%d" % qps
    return Problem(name, seed, params, arrays, "contexts %s" % L.tolist())


def _sfa_indices(seq, batch, q_s, kv_len, topk, sbs=1):
    """Entries drawn without replacement from the causal range of each query;
    with sbs > 1 they are blocks of sbs tokens (the blocks whose first token
    is causal for the query)."""
    g_idx = _gen(seq)
    rows = []
    for _b in range(batch):
        for s in range(q_s):
            # query s of a q_s-token step sits at position kv_len - q_s + s,
            # so positions 0 .. kv_len - q_s + s are its causal range
            rows.append(g_idx.choice((kv_len - q_s + s) // sbs + 1, topk, replace=False))
    return np.stack(rows).astype(np.int32).reshape(batch * q_s, 1, topk)


def sfa_mla_rope(seed=4, batch=32, q_s=2, kv_len=65536, topk=2048, bs=64, fp16=False, sbs=1):
    """Token-wise sparse MLA-absorb with rope: B=32, q_s=2, q_n=128, Q_D=576,
    separate K (576) and V (512) bf16 pools, PA block 64, kv length 65536,
    TopK 2048 drawn uniformly from the causal positions, scale 1/sqrt(576).
    fp16: the same in float16; sbs > 1: topk / sbs entries of sbs-token
    blocks (block-wise TopK, the same 2048 tokens per query)."""
    s_q, s_k, s_v, s_tab, s_idx = _seqs(seed, 5)
    qn, dq = 128, 576
    nblk = batch * kv_len // bs
    g_tab = _gen(s_tab)
    bt = g_tab.permutation(nblk).astype(np.int32).reshape(batch, kv_len // bs)
    idx = _sfa_indices(s_idx, batch, q_s, kv_len, topk // sbs, sbs)
    arrays = dict(
        q=normal_bf16(s_q, (batch * q_s, qn, dq), fp16=fp16),
        ori_kv=banked_rows(s_k, nblk * bs, lambda s, n: normal_bf16(s, (n, dq), fp16=fp16)),
        ori_v=banked_rows(s_v, nblk * bs, lambda s, n: normal_bf16(s, (n, 512), fp16=fp16)),
        ori_block_table=bt,
        seqused_ori_kv=np.full(batch, kv_len, np.int32),
        ori_sparse_indices=idx,
    )
    params = _base_params(
        num_heads_q=qn, rope_head_dim=64, batch_size=batch, layout_q="BSND",
        layout_kv="PA_BSND", q_s=q_s, q_t=batch * q_s, ori_block_size=bs,
        max_seqlen_q=q_s, max_seqlen_ori_kv=kv_len, ori_topk=topk // sbs,
        ori_mask_mode=3, has_cmp_kv=False, separate_v=True, sparse_block_size=sbs,
        kv_dtype="fp16" if fp16 else "bf16", softmax_scale=1.0 / math.sqrt(dq))
    name = "sfa_mla_rope" + ("_fp16" if fp16 else "") + ("_block%d" % sbs if sbs > 1 else "")
    what = ("%d blocks of %d causal tokens" % (topk // sbs, sbs)) if sbs > 1 else (
        "%d of the causal positions" % topk)
    return Problem(name, seed, params, arrays,
                   "q, K, V ~ N(0,1) %s; %s" % ("float16" if fp16 else "bf16", what))


def _c8_indices(seq, L, topk, qps=1):
    """Per query token, TopK entries drawn without replacement from its
    causal range: the token at position p = L - qps + i sees [0, p]."""
    g_idx = _gen(seq)
    idx = np.stack([g_idx.choice(int(n) - qps + 1 + i, topk, replace=False)
                    for n in L for i in range(qps)]).astype(np.int32)
    return idx.reshape(len(L) * qps, 1, topk)


def c8_packed(seed=5, fmt="int8", topk=2048, qps=1, rope=64, value=False):
    """Quantised packed KV: the HCA-varlen shapes (TND, B=8, q_n=128, the same
    context lengths) with Q_D=576 and 656-byte packed rows (512 INT8 or
    FP8-E4M3 codes, 64 bf16 rope values, 4 fp32 per-128-tile scales), V =
    dequantised nope; TopK 2048 over each sequence's positions.  qps > 1:
    qps query tokens per sequence (the last qps positions, each with its own
    causal TopK list), a throughput-mode variant of the decode.  rope 0: the
    528-byte rope-free rows (Q_D = 512).  value: V from a value tensor of 512
    codes per row (an independent quantised draw in the same format), scaled
    by the key rows' tiles."""
    s_q, s_kv, s_idx, s_v = _seqs(seed, 4)
    B, qn, dq = 8, 128, 512 + rope
    L = _varlen_lengths(3)
    idx = _c8_indices(s_idx, L, topk, qps)
    arrays = dict(
        q=normal_bf16(s_q, (B * qps, qn, dq), std=0.5),
        ori_kv=banked_rows(s_kv, int(L.sum()), lambda s, n: packed_rows(s, n, rope, fmt)),
        cu_seqlens_q=_prefix([qps] * B),
        cu_seqlens_ori_kv=_prefix(L),
        ori_sparse_indices=idx,
    )
    if value:
        arrays["ori_v"] = banked_rows(
            s_v, int(L.sum()), lambda s, n: np.ascontiguousarray(packed_rows(s, n, 0, fmt)[:, :512]))
    params = _base_params(
        num_heads_q=qn, rope_head_dim=rope, batch_size=B, layout_q="TND",
        layout_kv="TND", q_t=B * qps, max_seqlen_q=qps,
        max_seqlen_ori_kv=int(L.max()), ori_topk=topk, ori_mask_mode=3,
        has_cmp_kv=False, separate_v=value,
        kv_dtype="int8_packed" if fmt == "int8" else "fp8_e4m3_packed",
        softmax_scale=1.0 / math.sqrt(dq))
    name = ("c8_packed_" + fmt + ("" if rope else "_rope0") + ("_value" if value else "") +
            ("" if qps == 1 else "_q%d" % qps))
    return Problem(name, seed, params, arrays,
                   "packed %s rows, contexts %s" % (fmt, L.tolist()))


WORKLOADS = {
    "swa_decode": swa_decode,
    "csa_decode_paged": csa_decode_paged,
    "csa_prefill": csa_prefill,
    "hca_varlen": hca_varlen,
    "sfa_mla_rope": sfa_mla_rope,
    "sfa_mla_rope_fp16": lambda seed=4: sfa_mla_rope(seed, fp16=True),
    "sfa_mla_rope_block16": lambda seed=4: sfa_mla_rope(seed, sbs=16),
    "c8_packed_int8": lambda seed=5: c8_packed(seed, "int8"),
    "c8_packed_fp8": lambda seed=5: c8_packed(seed, "fp8"),
    "c8_packed_int8_rope0": lambda seed=5: c8_packed(seed, "int8", rope=0),
    "c8_packed_int8_value": lambda seed=5: c8_packed(seed, "int8", value=True),
    "hca_prefill": lambda seed=7: rule_prefill(seed, "hca"),
    "swa_prefill": lambda seed=8: rule_prefill(seed, "swa"),
    "swa_prefill_h16": lambda seed=9: rule_prefill(seed, "swa", qn=16),
    # throughput mode: 32 query tokens per sequence, 256 query rows per call
    "c8_packed_int8_q32": lambda seed=5: c8_packed(seed, "int8", qps=32),
    "hca_varlen_q32": lambda seed=3: hca_varlen(seed, qps=32),
}


def make_workload(name, seed=None, **kw):
    fn = WORKLOADS[name]
    return fn(**kw) if seed is None else fn(seed=seed, **kw)


def index_replicas(P: Problem, n: int):
    """n further TopK index sets drawn by the workload's own index recipe
    (fresh child streams), for rotating through distinct row sets between
    timed calls.  Returns a list of (array name, array)."""
    out = []
    for r in range(n):
        seq = np.random.SeedSequence([P.seed, 7919, r])
        if P.name.startswith("sfa_mla_rope"):
            p = P.params
            out.append(("ori_sparse_indices", _sfa_indices(
                seq, p["batch_size"], p["q_s"], p["max_seqlen_ori_kv"], p["ori_topk"],
                p["sparse_block_size"])))
        elif P.name.startswith("c8_packed"):
            cu = P.arrays["cu_seqlens_ori_kv"]
            out.append(("ori_sparse_indices", _c8_indices(
                seq, np.diff(cu), P.params["ori_topk"], P.params["max_seqlen_q"])))
        elif P.name == "csa_decode_paged":
            p = P.params
            out.append(("cmp_sparse_indices", _csa_indices(
                seq, p["batch_size"], p["max_seqlen_cmp_kv"], p["cmp_topk"])))
        else:
            return []
    return out


# ---------------------------------------------------------------------------
# Small random problems (edge cases, every layout and mode).
# ---------------------------------------------------------------------------

def random_tiny(seed, *, family=None, layout_q=None, layout_kv=None,
                num_heads_q=None, rope_head_dim=None, kv_dtype=None,
                batch=None, max_q=4, max_kv=64, block_size=None,
                cmp_ratio=None, sinks=None, dist="normal", topk=None,
                separate_v=None, q_lens=None, ori_lens=None,
                seqused_q=None, duplicates=False, win=None, masks=None,
                sparse_block_size=1, lse=None):
    """A small random problem.

    family: "swa" (ori window only), "csa" (window + TopK compressed rows),
    "hca" (window + all compressed rows) or "sfa" (TopK over one KV, the
    token-wise sparse MLA-absorb form).  Lengths, windows, mask modes,
    layouts and index tails are drawn at random unless given.  dist "p4" uses
    the SparseAttnSharedKV example's draws (q ~ U(-10,10), kv ~ U(-5,10),
    sinks ~ U(0,1)), which give very peaked softmaxes.  sparse_block_size
    (sfa only) > 1 makes each TopK entry select that many consecutive tokens;
    paged block sizes are then multiples of it.  lse: whether the LSE output
    is asked for (drawn, one case in three without, when not given).
    """
    ss = np.random.SeedSequence(seed)
    s_cfg, s_q, s_ori, s_v, s_cmp, s_idx, s_tab, s_sink = ss.spawn(8)
    (s_lse,) = ss.spawn(1)
    g = _gen(s_cfg)
    family = family or g.choice(["swa", "csa", "hca", "sfa"])
    B = batch or int(g.integers(1, 4))
    layout_q = layout_q or str(g.choice(["BSND", "TND"]))
    if layout_kv is None:
        layout_kv = str(g.choice([layout_q, "PA_BSND"]))
    qn = num_heads_q or int(g.choice([1, 2, 3, 4, 16]))
    rope = rope_head_dim if rope_head_dim is not None else (
        int(g.choice([0, 64])) if family == "sfa" else 0)
    kv_dtype = kv_dtype or "bf16"
    packed = kv_dtype not in ("bf16", "fp16")
    half = kv_dtype == "fp16"                 # q, kv and output in float16
    to_bits = fp16_bits if half else bf16_bits
    if separate_v is None:
        separate_v = bool(family == "sfa" and not packed and g.integers(0, 2))
    bs = block_size or int(g.choice([1, 2, 16]))
    sbs = int(sparse_block_size)
    if sbs > 1 and bs % sbs:
        bs = sbs * (1 + bs // sbs)
    r = cmp_ratio or (1 if family in ("swa", "sfa") else int(g.choice([1, 2, 4])))
    has_cmp = family in ("csa", "hca")

    q_lens = list(q_lens) if q_lens is not None else [int(g.integers(1, max_q + 1)) for _ in range(B)]
    ori_lens = list(ori_lens) if ori_lens is not None else [
        int(g.integers(q_lens[b], max_kv + 1)) for b in range(B)]
    cmp_lens = [n // r for n in ori_lens] if has_cmp else [0] * B
    residual = [n % r for n in ori_lens]

    if win is None:
        win = (int(g.choice([-1, 0, 1, 3, 7, 127])), int(g.choice([-1, 0, 0, 2])))
    if masks is None:
        if family == "sfa":
            masks = (int(g.choice([0, 3])), 0)
        else:
            masks = (int(g.choice([0, 3, 4])), int(g.choice([0, 3])) if has_cmp else 0)
    d_qk = 512 + rope

    # queries
    if layout_q == "BSND":
        q_s = max(q_lens)
        rows = B * q_s
        use_seqused_q = seqused_q if seqused_q is not None else (
            any(n != q_s for n in q_lens) or bool(g.integers(0, 4) == 0))
    else:
        q_s = 0
        rows = sum(q_lens)
        use_seqused_q = False
    if dist == "p4":
        qv = _gen(s_q).uniform(-10, 10, (rows, qn, d_qk)).astype(np.float32)
        q = to_bits(qv)
    else:
        q = normal_bf16(s_q, (rows, qn, d_qk), fp16=half)

    def kv_rows(seq, n, width_elems):
        if packed:
            return packed_rows(seq, n, rope, "int8" if kv_dtype == "int8_packed" else "fp8")
        if dist == "p4":
            return to_bits(_gen(seq).uniform(-5, 10, (n, width_elems)).astype(np.float32))
        return normal_bf16(seq, (n, width_elems), fp16=half)

    g_tab = _gen(s_tab)
    arrays = dict(q=q)
    params = _base_params(
        num_heads_q=qn, rope_head_dim=rope, batch_size=B, layout_q=layout_q,
        layout_kv=layout_kv, q_s=q_s, q_t=rows, max_seqlen_q=max(q_lens),
        max_seqlen_ori_kv=max(ori_lens), max_seqlen_cmp_kv=max(cmp_lens) if has_cmp else 0,
        cmp_ratio=r, ori_mask_mode=masks[0], cmp_mask_mode=masks[1],
        ori_win_left=win[0], ori_win_right=win[1], has_cmp_kv=has_cmp,
        kv_dtype=kv_dtype, separate_v=separate_v,
        softmax_scale=(1.0 / 24.0) if dist == "p4" else 1.0 / math.sqrt(d_qk),
        return_softmax_lse=bool(lse) if lse is not None else bool(_gen(s_lse).integers(0, 3)))
    if layout_q == "TND":
        arrays["cu_seqlens_q"] = _prefix(q_lens)
    elif use_seqused_q:
        arrays["seqused_q"] = np.asarray(q_lens, np.int32)

    def place(name, lens, seq, bs_key, s_key, width):
        if layout_kv == "BSND":
            S = max(1, max(lens) + int(g.integers(0, 3)))
            params[s_key] = S
            arrays[name] = kv_rows(seq, B * S, width)
            return "seqused", None
        if layout_kv == "TND":
            arrays[name] = kv_rows(seq, max(1, int(sum(lens))), width)
            return "cu", None
        table, nblocks = _paged(g_tab, lens, bs)
        params[bs_key] = bs
        arrays[name] = kv_rows(seq, nblocks * bs, width)
        return "pa", table

    kind, table = place("ori_kv", ori_lens, s_ori, "ori_block_size", "ori_kv_s", d_qk)
    if kind == "cu":
        arrays["cu_seqlens_ori_kv"] = _prefix(ori_lens)
    elif kind == "pa":
        arrays["ori_block_table"] = table
        arrays["seqused_ori_kv"] = np.asarray(ori_lens, np.int32)
    elif any(n != params["ori_kv_s"] for n in ori_lens) or g.integers(0, 2):
        arrays["seqused_ori_kv"] = np.asarray(ori_lens, np.int32)
    if separate_v:
        if packed:
            # a value tensor of 512 codes per row in the key's format (codes
            # of an independent quantised draw)
            arrays["ori_v"] = np.ascontiguousarray(
                packed_rows(s_v, arrays["ori_kv"].shape[0], 0,
                            "int8" if kv_dtype == "int8_packed" else "fp8")[:, :512])
        else:
            arrays["ori_v"] = kv_rows(s_v, arrays["ori_kv"].shape[0], 512)

    if has_cmp:
        kind, table = place("cmp_kv", cmp_lens, s_cmp,
                            "cmp_block_size", "cmp_kv_s", d_qk)
        if kind == "cu":
            arrays["cu_seqlens_cmp_kv"] = _prefix(cmp_lens)
        elif kind == "pa":
            arrays["cmp_block_table"] = table
            arrays["seqused_cmp_kv"] = np.asarray(cmp_lens, np.int32)
        else:
            arrays["seqused_cmp_kv"] = np.asarray(cmp_lens, np.int32)
        arrays["cmp_residual_kv"] = np.asarray(residual, np.int32)

    # TopK index lists: draws over the whole sequence (some beyond the causal
    # limit), optional duplicates, and a -1 tail of random length.
    g_idx = _gen(s_idx)

    def index_rows(lens_for_draw, K):
        out = np.full((rows, 1, K), -1, dtype=np.int32)
        for b in range(B):
            n_rows_b = q_s if layout_q == "BSND" else q_lens[b]
            base = b * q_s if layout_q == "BSND" else sum(q_lens[:b])
            for i in range(n_rows_b):
                n = lens_for_draw[b]
                if n <= 0:
                    continue
                k = int(g_idx.integers(0, K + 1))
                if duplicates:
                    vals = g_idx.integers(0, n, size=k)
                else:
                    k = min(k, n)
                    vals = g_idx.choice(n, k, replace=False)
                out[base + i, 0, :k] = vals
        return out

    if family == "sfa":
        nblk = [-(-n // sbs) for n in ori_lens]              # entries index blocks
        K = topk or int(g.integers(1, max(nblk) + 1))
        params["ori_topk"] = K
        params["sparse_block_size"] = sbs
        arrays["ori_sparse_indices"] = index_rows(nblk, K)
    if family == "csa":
        K = topk or int(g.integers(1, 2 * max(1, max(cmp_lens)) + 2))
        params["cmp_topk"] = K
        arrays["cmp_sparse_indices"] = index_rows(cmp_lens, K)

    use_sinks = sinks if sinks is not None else bool(g.integers(0, 2))
    if use_sinks:
        gs = _gen(s_sink)
        arrays["sinks"] = (gs.uniform(0, 1, qn) if dist == "p4"
                           else gs.standard_normal(qn)).astype(np.float32)
    return Problem("tiny_%s_%d" % (family, seed), seed, params, arrays,
                   "random tiny %s" % family)

