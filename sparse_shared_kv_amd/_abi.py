"""ctypes mirror of include/sfmla.h and loader of libsfmla.so.

Argument marshalling only: every step of the attention path runs in the
library's HIP kernels.  If the library is missing this module raises instead
of falling back to anything else.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SFMLA_LIB") or os.path.join(HERE, "libsfmla.so")

LAYOUTS = {"BSND": 0, "TND": 1, "PA_BSND": 2, "PA_BBND": 2, "PA_ND": 2}
KV_DTYPES = {"bf16": 0, "int8_packed": 1, "fp8_e4m3_packed": 2, "fp16": 3}
STATUS = {0: "SFMLA_OK", 1: "SFMLA_ERR_INVALID_ARGUMENT", 2: "SFMLA_ERR_UNSUPPORTED",
          3: "SFMLA_ERR_BUFFER_TOO_SMALL", 4: "SFMLA_ERR_LAUNCH", 5: "SFMLA_ERR_METADATA"}
STATUS_METADATA_MISMATCH = 1
STATUS_ROW_OUT_OF_RANGE = 2

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p


class Params(ctypes.Structure):
    _fields_ = [
        ("num_heads_q", _i32), ("num_heads_kv", _i32), ("head_dim", _i32),
        ("rope_head_dim", _i32), ("batch_size", _i32), ("layout_q", _i32),
        ("layout_kv", _i32), ("q_s", _i32), ("q_t", _i32), ("ori_kv_s", _i32),
        ("cmp_kv_s", _i32), ("ori_block_size", _i32), ("cmp_block_size", _i32),
        ("ori_block_table_cols", _i32), ("cmp_block_table_cols", _i32),
        ("ori_kv_rows", _i64), ("cmp_kv_rows", _i64),
        ("max_seqlen_q", _i32), ("max_seqlen_ori_kv", _i32), ("max_seqlen_cmp_kv", _i32),
        ("ori_topk", _i32), ("cmp_topk", _i32), ("ori_sparse_block_size", _i32),
        ("cmp_ratio", _i32),
        ("ori_mask_mode", _i32), ("cmp_mask_mode", _i32), ("ori_win_left", _i32),
        ("ori_win_right", _i32), ("has_ori_kv", _i32), ("has_cmp_kv", _i32),
        ("kv_dtype", _i32), ("has_separate_v", _i32), ("has_sinks", _i32),
        ("return_softmax_lse", _i32), ("has_seqused_q", _i32),
        ("has_seqused_ori_kv", _i32), ("has_seqused_cmp_kv", _i32),
        ("has_cmp_residual_kv", _i32), ("split_rows", _i32),
        ("head_blocks_per_group", _i32), ("merge_wait_us", _i32), ("query_tile", _i32),
        ("wave_pairs", _i32),
    ]


class Lengths(ctypes.Structure):
    _fields_ = [(n, _vp) for n in (
        "cu_seqlens_q", "cu_seqlens_ori_kv", "cu_seqlens_cmp_kv", "seqused_q",
        "seqused_ori_kv", "seqused_cmp_kv", "cmp_residual_kv")]


class Tensors(ctypes.Structure):
    _fields_ = [
        ("q", _vp),
        ("ori_kv", _vp), ("ori_kv_stride", _i64),
        ("ori_rope", _vp), ("ori_rope_stride", _i64),
        ("ori_v", _vp), ("ori_v_stride", _i64),
        ("cmp_kv", _vp), ("cmp_kv_stride", _i64),
        ("cmp_rope", _vp), ("cmp_rope_stride", _i64),
        ("ori_block_table", _vp), ("cmp_block_table", _vp),
        ("ori_sparse_indices", _vp), ("cmp_sparse_indices", _vp),
        ("sinks", _vp), ("attention_out", _vp), ("softmax_lse", _vp), ("status", _vp),
        ("q_rope", _vp),
    ]


SYMBOLS = ("sfmla_metadata_size", "sfmla_metadata", "sfmla_workspace_size",
           "sfmla_forward", "sfmla_forward_static_workspace", "sfmla_combine",
           "sfmla_debug_resolve", "sfmla_time_next_forward", "sfmla_last_error",
           "sfmla_version")

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsfmla.so (built by sparse_shared_kv_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libsfmla.so not found at %s; build it with "
                          "`python -m sparse_shared_kv_amd.build`" % path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    sz = ctypes.c_size_t
    lib.sfmla_metadata_size.argtypes = [P(Params), P(sz)]
    lib.sfmla_metadata.argtypes = [P(Params), P(Lengths), _vp, sz, _vp]
    lib.sfmla_workspace_size.argtypes = [P(Params), P(sz)]
    lib.sfmla_forward.argtypes = [P(Params), P(Tensors), _vp, sz, ctypes.c_float, _vp, sz, _vp]
    lib.sfmla_forward_static_workspace.argtypes = [P(Params), P(Tensors), _vp, sz,
                                                   ctypes.c_float, _vp]
    lib.sfmla_combine.argtypes = [_i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp]
    lib.sfmla_debug_resolve.argtypes = [P(Params), P(Tensors), _vp, sz, _vp, _i32, _vp, _vp]
    lib.sfmla_time_next_forward.argtypes = [_vp, _vp]
    for name in SYMBOLS[:8]:
        getattr(lib, name).restype = ctypes.c_int
    lib.sfmla_last_error.restype = ctypes.c_char_p
    lib.sfmla_last_error.argtypes = []
    lib.sfmla_version.restype = ctypes.c_char_p
    lib.sfmla_version.argtypes = []
    _lib = lib
    return lib


class SfmlaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


def check(status: int):
    if status != 0:
        raise SfmlaError(status, load().sfmla_last_error().decode())
