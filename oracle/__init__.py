"""CPU oracle for shared-KV sparse flash MLA attention — TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The GPU library never calls it, links it or
falls back to it.

What it computes is the plain definition the operator pages give: resolve the
set of KV rows each query attends to (sliding window over the original KV,
TopK-selected or all causally visible compressed rows, or TopK tokens of one
KV), gather and decode those rows, and take dense softmax attention with an
optional per-head sink:

    O = softmax(Q . K~^T . softmax_scale) . K~     with  K~ = V~
    LSE = log sum exp(S - max S) + max S,          S = Q . K~^T . softmax_scale

(sparse_flash_mla API page, 功能说明 / Function; SparseAttnSharedKV README,
功能说明; kv_quant_sparse_flash_attention blog, 计算公式 for the dequantised
form.)  Arithmetic is float64 throughout; bf16, INT8 and FP8-E4M3 inputs are
decoded exactly.

Modules:
    decode      exact decoders for bf16 bits, INT8 codes, FP8-E4M3FN codes and
                packed 656/528-byte rows
    resolve     lengths, query positions, visible row sets, physical rows
    attention   dense softmax attention with sink, forward(), combine()
    bruteforce  an independent checker for tiny inputs (explicit visibility
                weights over every position, decoders from torch dtypes)

Every function states the page passage it follows.  Readings of points the
pages leave open are listed in each function's docstring.
"""

from .attention import attend, combine, forward  # noqa: F401
from .resolve import (batch_lengths, query_rows, resolve_rows,  # noqa: F401
                      CMP_BIT)
