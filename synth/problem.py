"""Problem container and low-level seeded fills (no attention arithmetic)."""

from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

# Parameter keys every Problem carries (names follow the operator pages).
PARAM_KEYS = (
    "num_heads_q", "num_heads_kv", "head_dim", "rope_head_dim", "batch_size",
    "layout_q", "layout_kv", "q_s", "q_t", "ori_kv_s", "cmp_kv_s",
    "ori_block_size", "cmp_block_size", "max_seqlen_q", "max_seqlen_ori_kv",
    "max_seqlen_cmp_kv", "ori_topk", "cmp_topk", "cmp_ratio", "ori_mask_mode",
    "cmp_mask_mode", "ori_win_left", "ori_win_right", "has_ori_kv",
    "has_cmp_kv", "kv_dtype", "separate_v", "softmax_scale",
    "return_softmax_lse",
)

# Array keys (all optional except q / ori_kv).  Physical KV arrays are 2-D:
# (physical rows, row width) — BSND (b, s, 1, d) is stored as (b*s, d), TND
# (t, 1, d) as (t, d) and PA_BSND (blocks, block_size, 1, d) as
# (blocks*block_size, d).  bf16 tensors are uint16 bit patterns; packed KV
# rows are uint8.  q is (query rows, q_n, d_qk) with query rows = b*q_s for
# BSND and q_t for TND; index tensors are (query rows, 1, K).
ARRAY_KEYS = (
    "q", "ori_kv", "ori_v", "cmp_kv", "ori_block_table", "cmp_block_table",
    "cu_seqlens_q", "cu_seqlens_ori_kv", "cu_seqlens_cmp_kv", "seqused_q",
    "seqused_ori_kv", "seqused_cmp_kv", "cmp_residual_kv",
    "ori_sparse_indices", "cmp_sparse_indices", "sinks",
)


@dataclasses.dataclass
class Problem:
    name: str
    seed: int
    params: dict
    arrays: dict
    recipe: str = ""

    def get(self, key):
        return self.arrays.get(key)

    def copy(self, name=None, **param_overrides):
        p = dict(self.params)
        p.update(param_overrides)
        return Problem(name or self.name, self.seed, p,
                       {k: v.copy() for k, v in self.arrays.items()},
                       self.recipe)

    @property
    def query_rows(self) -> int:
        return int(self.arrays["q"].shape[0])


def bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (b >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def fp16_bits(x) -> np.ndarray:
    """Round fp32 values to float16 (nearest, ties to even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(seq: np.random.SeedSequence, shape, std=1.0, fp16=False) -> np.ndarray:
    """bf16 bits of N(0, std^2) draws, filled block-parallel.

    Row blocks get their own spawned child stream, so the values do not depend
    on the number of worker threads.
    """
    shape = tuple(int(s) for s in shape)
    n_rows = shape[0]
    width = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((n_rows, width), dtype=np.uint16)
    block = 8192
    n_blocks = (n_rows + block - 1) // block
    children = seq.spawn(n_blocks)

    def work(i):
        r0, r1 = i * block, min(n_rows, (i + 1) * block)
        g = np.random.Generator(np.random.PCG64(children[i]))
        v = g.standard_normal((r1 - r0, width), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[r0:r1] = fp16_bits(v) if fp16 else bf16_bits(v)

    if n_blocks == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_blocks)))
    return out.reshape(shape)


# Pools with more rows than this are filled from a seeded bank of random rows.
BANK_ROWS = 1 << 16
DIRECT_LIMIT = 1 << 17


def banked_rows(seq: np.random.SeedSequence, n_rows: int, make_bank):
    """Fill n_rows KV rows.

    Small pools are drawn directly (make_bank(seq, n_rows)).  Large pools
    (hundreds of MB to GB) are filled from a bank of BANK_ROWS independently
    drawn rows through a seeded uniform row map, so that building a 2.4 GB
    pool takes seconds.  Every row still has the workload's value
    distribution; rows that share a bank entry hold equal values, which the
    attention path treats like any other rows.
    """
    if n_rows <= DIRECT_LIMIT:
        return make_bank(seq, n_rows)
    s_bank, s_map = seq.spawn(2)
    bank = make_bank(s_bank, BANK_ROWS)
    g = np.random.Generator(np.random.PCG64(s_map))
    rmap = g.integers(0, BANK_ROWS, size=n_rows, dtype=np.int64)
    out = np.empty((n_rows,) + bank.shape[1:], dtype=bank.dtype)
    chunk = 1 << 16
    for r0 in range(0, n_rows, chunk):
        np.take(bank, rmap[r0:r0 + chunk], axis=0, out=out[r0:r0 + chunk])
    return out


# ---------------------------------------------------------------------------
# Packed-KV writer (KV-cache side): per-128-tile quantiser and row packer.
# ---------------------------------------------------------------------------

def _e4m3_table():
    """Non-negative finite E4M3FN values by code 0x00..0x7E (writer side)."""
    vals = np.empty(0x7F, dtype=np.float64)
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_table()


def _encode_e4m3(y: np.ndarray) -> np.ndarray:
    """Round |y| <= 448 to the nearest E4M3FN code, ties to the even code."""
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    hi = np.searchsorted(_E4M3_POS, a, side="left")
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(y) & (code != 0)).astype(np.uint8) << 7
    return code | sign


def pack_rows(nope_f32: np.ndarray, rope_bits, fmt: str) -> np.ndarray:
    """Pack rows as [512 codes][rope bf16][4 x fp32 scales] (little-endian).

    nope_f32: (n, 512) fp32 draws; rope_bits: (n, r) uint16 or None.
    fmt: "int8" (scale = absmax/127, code = clamp(rint(v/s), -127, 127)) or
    "fp8" (scale = absmax/448, code = nearest E4M3FN, saturating).  A tile
    with absmax 0 gets scale 1.
    """
    n = nope_f32.shape[0]
    rope_w = 0 if rope_bits is None else rope_bits.shape[1]
    width = 512 + 2 * rope_w + 16
    out = np.zeros((n, width), dtype=np.uint8)
    tiles = nope_f32.reshape(n, 4, 128).astype(np.float32)
    amax = np.abs(tiles).max(axis=2)
    qmax = np.float32(127.0 if fmt == "int8" else 448.0)
    scale = np.where(amax > 0, amax / qmax, np.float32(1.0)).astype(np.float32)
    y = tiles / scale[:, :, None]
    if fmt == "int8":
        codes = np.clip(np.rint(y), -127, 127).astype(np.int8).view(np.uint8)
    elif fmt == "fp8":
        codes = _encode_e4m3(y)
    else:
        raise ValueError(fmt)
    out[:, :512] = codes.reshape(n, 512)
    if rope_w:
        out[:, 512:512 + 2 * rope_w] = np.ascontiguousarray(rope_bits).view(np.uint8).reshape(n, 2 * rope_w)
    out[:, 512 + 2 * rope_w:] = scale.astype("<f4").view(np.uint8).reshape(n, 16)
    return out


def packed_rows(seq: np.random.SeedSequence, n_rows: int, rope_w: int, fmt: str):
    """n_rows packed rows: nope ~N(0,1) quantised per tile, rope ~N(0,1) bf16."""
    s_nope, s_rope = seq.spawn(2)
    out = []
    block = 16384
    g = np.random.Generator(np.random.PCG64(s_nope))
    rope = normal_bf16(s_rope, (n_rows, rope_w)) if rope_w else None
    for r0 in range(0, n_rows, block):
        r1 = min(n_rows, r0 + block)
        v = g.standard_normal((r1 - r0, 512), dtype=np.float32)
        out.append(pack_rows(v, None if rope is None else rope[r0:r1], fmt))
    return np.concatenate(out, axis=0)
