"""Shared-KV sparse flash MLA attention on MI355X (gfx950).

Python binding of libsfmla.so (include/sfmla.h).  The functions below keep
the C entry points' names and only marshal arguments; torch supplies device
memory and the current HIP stream.  `Call` bundles one problem's device
tensors, plan and workspace for repeated calls.

There is no fallback: if libsfmla.so is missing, importing the binding
functions raises ImportError.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import _abi
from ._abi import KV_DTYPES, LAYOUTS, Lengths, Params, SfmlaError, Tensors

__all__ = ["sfmla_metadata_size", "sfmla_metadata", "sfmla_workspace_size", "sfmla_forward",
           "sfmla_forward_static_workspace", "sfmla_combine", "sfmla_debug_resolve", "sfmla_time_next_forward",
           "sfmla_version", "Params", "Lengths",
           "Tensors", "SfmlaError", "Call", "make_params", "CMP_BIT"]

CMP_BIT = 1 << 62


def _lib():
    return _abi.load()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype, shape=None):
    """A tensor handed to the library as a bare pointer: contiguous, of the
    given dtype (and shape).  None passes (an absent optional tensor)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise SfmlaError(1, "%s must be %s (got %s)" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise SfmlaError(1, "%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise SfmlaError(1, "%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))


def _require_rows(t, name, dtypes):
    """A KV pool: 2-D (physical rows, row elements), each row contiguous;
    consecutive rows may be further apart (row stride >= row, padding
    allowed, a multiple of 16 bytes)."""
    if t is None:
        return
    if t.dtype not in dtypes:
        raise SfmlaError(1, "%s must be one of %s (got %s)" % (name, dtypes, t.dtype))
    if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
        raise SfmlaError(1, "%s must be 2-D with contiguous rows (stride(1) == 1, "
                            "stride(0) >= row width)" % name)


def sfmla_version() -> str:
    return _lib().sfmla_version().decode()


def sfmla_metadata_size(params: Params) -> int:
    n = ctypes.c_size_t()
    _abi.check(_lib().sfmla_metadata_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def sfmla_workspace_size(params: Params) -> int:
    n = ctypes.c_size_t()
    _abi.check(_lib().sfmla_workspace_size(ctypes.byref(params), ctypes.byref(n)))
    return n.value


def sfmla_metadata(params: Params, lengths: Lengths, metadata: torch.Tensor, stream=None):
    _abi.check(_lib().sfmla_metadata(ctypes.byref(params), ctypes.byref(lengths),
                                     _ptr(metadata), metadata.numel(), _stream(stream)))


def sfmla_forward(params: Params, tensors: Tensors, metadata: torch.Tensor, softmax_scale: float,
                  workspace: torch.Tensor | None = None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _abi.check(_lib().sfmla_forward(ctypes.byref(params), ctypes.byref(tensors), _ptr(metadata),
                                    metadata.numel(), ctypes.c_float(softmax_scale),
                                    _ptr(workspace), ws_bytes, _stream(stream)))


def sfmla_forward_static_workspace(params: Params, tensors: Tensors, metadata: torch.Tensor,
                                   softmax_scale: float, stream=None):
    """sfmla_forward with the split workspace held by the library (one static
    device buffer per GPU; allocates nothing)."""
    _abi.check(_lib().sfmla_forward_static_workspace(
        ctypes.byref(params), ctypes.byref(tensors), _ptr(metadata), metadata.numel(),
        ctypes.c_float(softmax_scale), _stream(stream)))


def sfmla_combine(part_o: torch.Tensor, part_lse: torch.Tensor, sinks, out: torch.Tensor,
                  lse_out=None, stream=None):
    """LSE merge of caller-supplied partials: part_o fp32 (n_parts, rows, heads,
    dv), part_lse fp32 (n_parts, rows, heads), sinks fp32 (heads) or None,
    out bf16 (rows, heads, dv), lse_out fp32 (rows, heads) or None."""
    n_parts, rows, heads, dv = part_o.shape
    _require(part_o, "part_o", torch.float32, (n_parts, rows, heads, dv))
    _require(part_lse, "part_lse", torch.float32, (n_parts, rows, heads))
    _require(sinks, "sinks", torch.float32, (heads,))
    _require(out, "out", torch.bfloat16, (rows, heads, dv))
    _require(lse_out, "lse_out", torch.float32, (rows, heads))
    _abi.check(_lib().sfmla_combine(n_parts, _ptr(part_o), _ptr(part_lse), _ptr(sinks),
                                    _ptr(out), _ptr(lse_out), rows, heads, dv, _stream(stream)))


def sfmla_debug_resolve(params: Params, tensors: Tensors, metadata: torch.Tensor,
                        rows_out: torch.Tensor, counts_out: torch.Tensor, stream=None):
    _abi.check(_lib().sfmla_debug_resolve(ctypes.byref(params), ctypes.byref(tensors),
                                          _ptr(metadata), metadata.numel(), _ptr(rows_out),
                                          rows_out.shape[1], _ptr(counts_out), _stream(stream)))


def sfmla_time_next_forward(start: torch.cuda.Event, stop: torch.cuda.Event):
    """The next sfmla_forward on this thread has its kernel's start and end
    stamped into these events by the dispatch (no event packets around it).
    The events must already exist: record each once beforehand."""
    for e in (start, stop):
        if not e.cuda_event:
            raise ValueError("record the event once before passing it")
    _abi.check(_lib().sfmla_time_next_forward(ctypes.c_void_p(start.cuda_event),
                                              ctypes.c_void_p(stop.cuda_event)))


# ---------------------------------------------------------------------------
# convenience: one problem's device tensors, plan and workspace
# ---------------------------------------------------------------------------

def make_params(spec: dict, arrays: dict) -> Params:
    """sfmla_params from the pages' parameter names plus the arrays present."""
    p = Params()
    g = spec.get
    p.num_heads_q = int(g("num_heads_q"))
    p.num_heads_kv = int(g("num_heads_kv", 1))
    p.head_dim = int(g("head_dim", 512))
    p.rope_head_dim = int(g("rope_head_dim", 0))
    p.batch_size = int(g("batch_size"))
    p.layout_q = LAYOUTS[g("layout_q")]
    p.layout_kv = LAYOUTS[g("layout_kv")]
    p.q_s = int(g("q_s", 0)) if g("layout_q") == "BSND" else 0
    p.q_t = int(arrays["q"].shape[0])
    p.ori_kv_s = int(g("ori_kv_s", 0))
    p.cmp_kv_s = int(g("cmp_kv_s", 0))
    p.ori_block_size = int(g("ori_block_size", 0))
    p.cmp_block_size = int(g("cmp_block_size", 0))
    bt = arrays.get("ori_block_table")
    p.ori_block_table_cols = int(bt.shape[1]) if bt is not None else 0
    bt = arrays.get("cmp_block_table")
    p.cmp_block_table_cols = int(bt.shape[1]) if bt is not None else 0
    p.ori_kv_rows = int(arrays["ori_kv"].shape[0])
    p.cmp_kv_rows = int(arrays["cmp_kv"].shape[0]) if arrays.get("cmp_kv") is not None else 0
    p.max_seqlen_q = int(g("max_seqlen_q"))
    p.max_seqlen_ori_kv = int(g("max_seqlen_ori_kv"))
    p.max_seqlen_cmp_kv = int(g("max_seqlen_cmp_kv", 0))
    p.ori_topk = int(g("ori_topk", 0))
    p.cmp_topk = int(g("cmp_topk", 0))
    p.ori_sparse_block_size = int(g("sparse_block_size", 1))
    p.cmp_ratio = int(g("cmp_ratio", 1))
    p.ori_mask_mode = int(g("ori_mask_mode"))
    p.cmp_mask_mode = int(g("cmp_mask_mode", 0))
    p.ori_win_left = int(g("ori_win_left", -1))
    p.ori_win_right = int(g("ori_win_right", -1))
    p.has_ori_kv = 1
    p.has_cmp_kv = int(bool(g("has_cmp_kv", False)))
    p.kv_dtype = KV_DTYPES[g("kv_dtype", "bf16")]
    p.has_separate_v = int(arrays.get("ori_v") is not None)
    p.has_sinks = int(arrays.get("sinks") is not None)
    p.return_softmax_lse = int(bool(g("return_softmax_lse", True)))
    p.has_seqused_q = int(arrays.get("seqused_q") is not None)
    p.has_seqused_ori_kv = int(arrays.get("seqused_ori_kv") is not None)
    p.has_seqused_cmp_kv = int(arrays.get("seqused_cmp_kv") is not None)
    p.has_cmp_residual_kv = int(arrays.get("cmp_residual_kv") is not None)
    p.split_rows = int(g("split_rows", 0))
    p.head_blocks_per_group = int(g("head_blocks_per_group", 0))
    p.merge_wait_us = int(g("merge_wait_us", 0))
    p.query_tile = int(g("query_tile", 0))
    p.wave_pairs = int(g("wave_pairs", 0))
    return p


def _to_device(a, device):
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.to(device)
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class Call:
    """Device state of one problem: inputs, outputs, plan and workspace.

    spec: the pages' parameter names (a dict); arrays: numpy or torch arrays
    named as in the pages (q, ori_kv, ori_v, cmp_kv, block tables, cu_seqlens_*,
    seqused_*, cmp_residual_kv, *_sparse_indices, sinks).  bf16 data may be
    given as uint16 bit patterns.
    """

    def __init__(self, spec: dict, arrays: dict, device="cuda"):
        self.spec = dict(spec)
        self.device = torch.device(device)
        self.d = {k: _to_device(v, self.device) for k, v in arrays.items() if v is not None}
        self.params = make_params(self.spec, self.d)
        self.scale = float(self.spec["softmax_scale"])
        qn = self.params.num_heads_q
        odt = torch.float16 if self.spec.get("kv_dtype") == "fp16" else torch.bfloat16
        self.out = torch.empty((self.params.q_t, qn, 512), dtype=odt, device=self.device)
        self.lse = (torch.empty((self.params.q_t, qn), dtype=torch.float32, device=self.device)
                    if self.params.return_softmax_lse else None)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)
        self.lengths = Lengths()
        for name, _ in Lengths._fields_:
            t = self.d.get(name)
            setattr(self.lengths, name, None if t is None else t.data_ptr())
        self.metadata = torch.zeros(sfmla_metadata_size(self.params), dtype=torch.int32,
                                    device=self.device)
        ws = sfmla_workspace_size(self.params)
        self.workspace = (torch.empty(ws // 4 + 64, dtype=torch.float32, device=self.device)
                          if ws else None)
        self.tensors = self._tensors()

    def _check(self):
        """dtype and layout of every tensor the library reads through a bare
        pointer: q, index lists, block tables, length tensors and sinks
        contiguous with their pages' dtypes; KV pools with contiguous rows."""
        d = self.d
        half = torch.float16 if self.spec.get("kv_dtype") == "fp16" else torch.bfloat16
        rope = int(self.params.rope_head_dim)
        q_rope = d.get("q_rope")
        q_t, qn = int(self.params.q_t), int(self.params.num_heads_q)
        for name in ("q", "q_rope"):
            if d.get(name) is None:
                continue
            if d[name].dtype not in (half, torch.int16):
                raise SfmlaError(1, "%s must be %s (or its int16 bits)" % (name, half))
            if not d[name].is_contiguous():
                raise SfmlaError(1, "%s must be contiguous" % name)
        want = (q_t, qn, 512 if q_rope is not None else 512 + rope)
        if tuple(d["q"].shape) != want:
            raise SfmlaError(1, "q must have shape %s, got %s" % (want, tuple(d["q"].shape)))
        if q_rope is not None and tuple(q_rope.shape) != (q_t, qn, rope):
            raise SfmlaError(1, "q_rope must have shape %s" % ((q_t, qn, rope),))
        for name in ("ori_block_table", "cmp_block_table", "ori_sparse_indices",
                     "cmp_sparse_indices") + tuple(n for n, _ in Lengths._fields_):
            _require(d.get(name), name, torch.int32)
        _require(d.get("sinks"), "sinks", torch.float32)
        packed = self.spec.get("kv_dtype") in ("int8_packed", "fp8_e4m3_packed")
        kv_types = (torch.uint8,) if packed else (half, torch.int16)
        for name in ("ori_kv", "cmp_kv"):
            _require_rows(d.get(name), name, kv_types)
        _require_rows(d.get("ori_v"), "ori_v", kv_types)   # packed: value codes
        for name in ("ori_rope", "cmp_rope"):
            _require_rows(d.get(name), name, (half, torch.int16))

    def _tensors(self) -> Tensors:
        d = self.d
        self._check()
        t = Tensors()

        def row_bytes(x):
            return x.stride(0) * x.element_size() if x is not None else 0

        t.q = d["q"].data_ptr()
        if d.get("q_rope") is not None:
            t.q_rope = d["q_rope"].data_ptr()
        t.ori_kv = d["ori_kv"].data_ptr()
        t.ori_kv_stride = row_bytes(d["ori_kv"])
        if d.get("ori_v") is not None:
            t.ori_v = d["ori_v"].data_ptr()
            t.ori_v_stride = row_bytes(d["ori_v"])
        if d.get("ori_rope") is not None:
            t.ori_rope = d["ori_rope"].data_ptr()
            t.ori_rope_stride = row_bytes(d["ori_rope"])
        if d.get("cmp_kv") is not None:
            t.cmp_kv = d["cmp_kv"].data_ptr()
            t.cmp_kv_stride = row_bytes(d["cmp_kv"])
        if d.get("cmp_rope") is not None:
            t.cmp_rope = d["cmp_rope"].data_ptr()
            t.cmp_rope_stride = row_bytes(d["cmp_rope"])
        for name in ("ori_block_table", "cmp_block_table", "ori_sparse_indices",
                     "cmp_sparse_indices", "sinks"):
            if d.get(name) is not None:
                setattr(t, name, d[name].data_ptr())
        t.attention_out = self.out.data_ptr()
        t.softmax_lse = None if self.lse is None else self.lse.data_ptr()
        t.status = self.status.data_ptr()
        return t

    def plan(self, stream=None):
        sfmla_metadata(self.params, self.lengths, self.metadata, stream)

    def forward(self, stream=None):
        sfmla_forward(self.params, self.tensors, self.metadata, self.scale, self.workspace, stream)

    def run(self, stream=None):
        """One pass of the whole path: plan, then the forward (which merges
        the KV splits it plans)."""
        self.plan(stream)
        self.forward(stream)
        return self.out, self.lse

    def resolve(self, max_rows, stream=None):
        rows = torch.empty((self.params.q_t, max_rows), dtype=torch.int64, device=self.device)
        counts = torch.empty(self.params.q_t, dtype=torch.int32, device=self.device)
        sfmla_debug_resolve(self.params, self.tensors, self.metadata, rows, counts, stream)
        return rows, counts


def default_scale(spec: dict) -> float:
    return 1.0 / math.sqrt(512 + int(spec.get("rope_head_dim", 0)))
