"""Exact decoders for the stored KV formats (oracle; test infrastructure).

* bf16: a 16-bit pattern is the upper half of an IEEE binary32 value.
* INT8 packed rows (kv_quant_sparse_flash_attention blog, 参数说明 key / the
  A2/A3 C8 NoPE table): 512 signed 8-bit codes, then rope_dim bf16 values, then
  four little-endian fp32 scales, one per 128 nope values; the dequantised
  value is code * scale of its tile (计算公式: Dequant(K^INT8, Scale_K)).
* FP8 E4M3FN (same blog, Ascend 950 INT8/FP8 section) decoded from the OCP
  8-bit floating point definition: 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; the
  format has no infinities, so its largest magnitude is 1.75 * 2^8 = 448.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE 754 binary16 bits -> float64, from the format's definition: sign,
    5-bit exponent with bias 15, 10-bit fraction; exponent 0 is subnormal
    (f / 2^10 * 2^-14), exponent 31 is infinity (f = 0) or NaN.  float16 is
    the other q / kv type the pages allow (sparse_flash_mla API page and
    SparseFlashAttention README, 参数说明 data types)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    subnormal = (f / 1024.0) * 2.0 ** -14
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def int8_to_f64(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.uint8).view(np.int8).astype(np.float64)


def fp8_e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def packed_layout(rope_dim: int):
    """Byte offsets of a packed row: (rope offset, scale offset, row bytes).

    512 code bytes, 2*rope_dim rope bytes, 16 scale bytes: 656 bytes with the
    scales at 640 for rope 64, 528 bytes with the scales at 512 for rope 0
    (blog, A2/A3 C8 NoPE table; the width formula printed beside it is read as
    512 + 2*rope + 4*4).
    """
    rope_off = 512
    scale_off = 512 + 2 * rope_dim
    return rope_off, scale_off, scale_off + 16


def decode_packed(rows_u8: np.ndarray, rope_dim: int, fmt: str):
    """Decode packed rows -> (K (n, 512+rope), V (n, 512)) in float64.

    K = [dequantised nope || rope], V = dequantised nope (blog, 参数说明 value:
    the effective V is the dequantised 512-dim NoPE part of key).
    """
    rows_u8 = np.asarray(rows_u8, dtype=np.uint8)
    n = rows_u8.shape[0]
    rope_off, scale_off, width = packed_layout(rope_dim)
    if rows_u8.shape[1] < width:
        raise ValueError("packed row narrower than %d bytes" % width)
    codes = rows_u8[:, :512]
    if fmt == "int8_packed":
        x = int8_to_f64(codes)
    elif fmt == "fp8_e4m3_packed":
        x = fp8_e4m3fn_to_f64(codes)
    else:
        raise ValueError(fmt)
    scales = np.ascontiguousarray(rows_u8[:, scale_off:scale_off + 16]).view("<f4")
    scales = scales.astype(np.float64).reshape(n, 4)
    nope = x * np.repeat(scales, 128, axis=1)
    if rope_dim:
        rope_bits = np.ascontiguousarray(rows_u8[:, rope_off:rope_off + 2 * rope_dim]).view("<u2")
        rope = bf16_to_f64(rope_bits.reshape(n, rope_dim))
        k = np.concatenate([nope, rope], axis=1)
    else:
        k = nope
    return k, nope


def decode_packed_value(value_u8: np.ndarray, key_rows_u8: np.ndarray, rope_dim: int, fmt: str):
    """V rows from a value tensor of 512 codes per row (same format as the key's
    codes), each 128-column tile scaled by the matching key row's fp32 scale.

    Reading: the blog's value parameter may be a 512-wide NoPE tensor instead
    of the packed key cache itself; its dtype follows the key, its quant mode
    is per-tile and its own dequant-scale input is reserved, while the
    effective V is stated to be the key's dequantised NoPE, so the scales are
    the key row's.  With the key's own codes in it, V equals decode_packed's.
    """
    value_u8 = np.asarray(value_u8, dtype=np.uint8)
    key_rows_u8 = np.asarray(key_rows_u8, dtype=np.uint8)
    n = value_u8.shape[0]
    if value_u8.shape[1] < 512:
        raise ValueError("value rows narrower than 512 bytes")
    codes = value_u8[:, :512]
    if fmt == "int8_packed":
        x = int8_to_f64(codes)
    elif fmt == "fp8_e4m3_packed":
        x = fp8_e4m3fn_to_f64(codes)
    else:
        raise ValueError(fmt)
    _, scale_off, _ = packed_layout(rope_dim)
    scales = np.ascontiguousarray(key_rows_u8[:, scale_off:scale_off + 16]).view("<f4")
    scales = scales.astype(np.float64).reshape(n, 4)
    return x * np.repeat(scales, 128, axis=1)
