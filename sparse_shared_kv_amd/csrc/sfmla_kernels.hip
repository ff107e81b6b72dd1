// gfx950 kernels of shared-KV sparse flash MLA attention.
//
//   plan_kernel        one thread per query row: lengths, position, extents of
//                      the window / list rules, split count (the metadata
//                      step of the sparse_flash_mla API page).
//   fwd_kernel         one workgroup per (split, query row, head group):
//                      resolve the split's list positions to physical rows,
//                      gather them into LDS (packed INT8 / FP8 rows are then
//                      decoded exactly to bf16), S^T = K Q^T on bf16 MFMA,
//                      online softmax, O^T += V^T P^T on bf16 MFMA, then the
//                      final output, or a partial that the last split of the
//                      row to finish merges.
//   combine_kernel     LSE merge of caller-supplied fp32 partials (sfmla_combine),
//                      sink applied once.
//   resolve_kernel     debug dump of the resolved rows in canonical order.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Lane l holds A[m = l%16][k = 8(l/16)+i],
// B[k = 8(l/16)+i][n = l%16] (i < 8) and D[m = 4(l/16)+i][n = l%16] (i < 4).
// Scores are computed transposed (M = KV rows, N = heads) so that each lane's
// accumulators belong to a single head; the P tile then is directly the B
// operand of the PV product with the row index permuted consistently on both
// operands, and V^T is read from the row-major LDS tile with ds_read_tr16_b64
// (within a 16-lane group, lane t gets column t of a 4 x 16 block whose row r
// is addressed by lanes 4r..4r+3).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "sfmla_internal.h"

namespace sfmla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// The resolution of one list position is split into its memory steps so
// that a workgroup can issue every position's index load, then every
// position's block-table load, with the loads of all positions in flight.
// The row's plan record is read once, into uniform registers.
struct RowInfo {
  int b, p, ori_lo, ori_cnt, ori_len, cmp_limit, ori_base, cmp_base;
};

__device__ __forceinline__ RowInfo row_info(const int32_t* rec) {
  RowInfo r;
  r.b = __builtin_amdgcn_readfirstlane(rec[R_B]);
  r.p = __builtin_amdgcn_readfirstlane(rec[R_P]);
  r.ori_lo = __builtin_amdgcn_readfirstlane(rec[R_ORI_LO]);
  r.ori_cnt = __builtin_amdgcn_readfirstlane(rec[R_ORI_CNT]);
  r.ori_len = __builtin_amdgcn_readfirstlane(rec[R_ORI_LEN]);
  r.cmp_limit = __builtin_amdgcn_readfirstlane(rec[R_CMP_LIMIT]);
  r.ori_base = __builtin_amdgcn_readfirstlane(rec[R_ORI_BASE]);
  r.cmp_base = __builtin_amdgcn_readfirstlane(rec[R_CMP_BASE]);
  return r;
}

// List position k of query row `row` -> the index-list entry it reads, or
// nullptr where the position follows a window or all-visible rule.
__device__ __forceinline__ const int32_t* slot_entry(const FwdArgs& a, const RowInfo& ri, int row,
                                                     int k) {
  if (k < ri.ori_cnt)
    return a.ori_topk > 0 ? a.ori_idx + (int64_t)row * a.ori_topk + (k >> a.ori_sbs_log2) : nullptr;
  return a.cmp_topk > 0 ? a.cmp_idx + (int64_t)row * a.cmp_topk + (k - ri.ori_cnt) : nullptr;
}

// List position k (entry value v where it has one) -> logical row j of its
// KV (-1: empty or masked slot); *is_cmp tells which KV.
__device__ __forceinline__ int slot_row(const FwdArgs& a, const RowInfo& ri, int k, int v,
                                        int* is_cmp) {
  if (k < ri.ori_cnt) {
    *is_cmp = 0;
    if (a.ori_topk <= 0) return ri.ori_lo + k;
    if (v < 0) return -1;
    // block-wise entries select tokens v*s .. v*s+s-1 (s = 1: token-wise);
    // each passes the mask on its own
    const int64_t j = ((int64_t)v << a.ori_sbs_log2) + (k & ((1 << a.ori_sbs_log2) - 1));
    if (j >= ri.ori_len) return -1;
    if (a.ori_mode == SFMLA_MASK_CAUSAL && j > ri.p) return -1;
    if (a.ori_mode == SFMLA_MASK_BAND &&
        ((a.win_l >= 0 && j < ri.p - a.win_l) || (a.win_r >= 0 && j > ri.p + a.win_r)))
      return -1;
    return (int)j;
  }
  *is_cmp = 1;
  if (a.cmp_topk <= 0) return k - ri.ori_cnt;
  if (v < 0 || v >= ri.cmp_limit) return -1;
  return v;
}

// PA layout: the block-table entry logical row j lies in (nullptr when the
// layout is not paged, j < 0, or j is past the table: the last is reported).
__device__ __forceinline__ const int32_t* table_entry(const FwdArgs& a, const RowInfo& ri, int j,
                                                      int is_cmp) {
  if (a.layout_kv != SFMLA_LAYOUT_PA_BSND || j < 0) return nullptr;
  const int bs = is_cmp ? a.cmp_bs : a.ori_bs;
  const int cols = is_cmp ? a.cmp_bt_cols : a.ori_bt_cols;
  const int blk = j / bs;
  if (blk >= cols) {
    if (a.status) atomicOr(a.status, SFMLA_STATUS_ROW_OUT_OF_RANGE);
    return nullptr;
  }
  return (is_cmp ? a.cmp_bt : a.ori_bt) + (int64_t)ri.b * cols + blk;
}

// Logical row j (table entry value e for PA) -> physical row, or -1 when the
// slot is empty or the row lies outside its pool (reported).
__device__ __forceinline__ int64_t phys_row(const FwdArgs& a, const RowInfo& ri, int j, int is_cmp,
                                            bool has_entry, int e) {
  if (j < 0) return -1;
  int64_t phys;
  if (a.layout_kv == SFMLA_LAYOUT_PA_BSND) {
    if (!has_entry) return -1;                                   // past the table
    const int bs = is_cmp ? a.cmp_bs : a.ori_bs;
    phys = (int64_t)e * bs + (j - (j / bs) * bs);
  } else {
    phys = (int64_t)(is_cmp ? ri.cmp_base : ri.ori_base) + j;
  }
  if (phys < 0 || phys >= (is_cmp ? a.cmp_rows : a.ori_rows)) {
    if (a.status) atomicOr(a.status, SFMLA_STATUS_ROW_OUT_OF_RANGE);
    return -1;
  }
  return phys;
}

// One list position, all steps in order (debug dump).
__device__ __forceinline__ int64_t resolve_pos(const FwdArgs& a, const int32_t* rec, int row,
                                               int k, int* is_cmp) {
  const RowInfo ri = row_info(rec);
  const int32_t* ep = slot_entry(a, ri, row, k);
  const int j = slot_row(a, ri, k, ep ? *ep : 0, is_cmp);
  const int32_t* tp = table_entry(a, ri, j, *is_cmp);
  return phys_row(a, ri, j, *is_cmp, tp != nullptr, tp ? *tp : 0);
}

// ---------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 128;

// Lengths of sequence b, read from the length tensors.
struct SeqLens {
  int q_len, q_used, ori_len, ori_base, cmp_len, cmp_base, res;
};
__device__ __forceinline__ SeqLens seq_lens(const PlanArgs& a, int b) {
  const sfmla_params& p = a.p;
  SeqLens s;
  s.q_len = p.layout_q == SFMLA_LAYOUT_BSND ? p.q_s
                                            : a.len.cu_seqlens_q[b + 1] - a.len.cu_seqlens_q[b];
  const int qu = a.len.seqused_q ? a.len.seqused_q[b] : s.q_len;
  s.q_used = qu < 0 ? 0 : (qu > s.q_len ? s.q_len : qu);
  s.ori_base = 0;
  if (a.len.seqused_ori_kv) s.ori_len = a.len.seqused_ori_kv[b];
  else if (p.layout_kv == SFMLA_LAYOUT_TND)
    s.ori_len = a.len.cu_seqlens_ori_kv[b + 1] - a.len.cu_seqlens_ori_kv[b];
  else s.ori_len = p.ori_kv_s;
  if (p.layout_kv == SFMLA_LAYOUT_TND) s.ori_base = a.len.cu_seqlens_ori_kv[b];
  else if (p.layout_kv == SFMLA_LAYOUT_BSND) s.ori_base = b * p.ori_kv_s;
  s.cmp_len = 0, s.cmp_base = 0, s.res = 0;
  if (p.has_cmp_kv) {
    if (a.len.seqused_cmp_kv) s.cmp_len = a.len.seqused_cmp_kv[b];
    else if (p.layout_kv == SFMLA_LAYOUT_TND)
      s.cmp_len = a.len.cu_seqlens_cmp_kv[b + 1] - a.len.cu_seqlens_cmp_kv[b];
    else s.cmp_len = p.cmp_kv_s;
    if (p.layout_kv == SFMLA_LAYOUT_TND) s.cmp_base = a.len.cu_seqlens_cmp_kv[b];
    else if (p.layout_kv == SFMLA_LAYOUT_BSND) s.cmp_base = b * p.cmp_kv_s;
    if (a.len.cmp_residual_kv) s.res = a.len.cmp_residual_kv[b];
  }
  return s;
}

// Query rows per tile of a sequence (0: its rows are not tiled): a decision
// from the sequence's own lengths, so a sequence is tiled the same way in any
// batch, taken where tiles are possible at all (a.tq > 1).  It needs enough
// valid queries and a bound on the union of a tile's lists within one split:
// the union of tq consecutive rows' windows spans at most win_left +
// win_right + tq positions (each row's window is its predecessor's moved by
// one), every rule list lies within the sequence's ori rows, and the visible
// compressed rows of any row lie within the sequence's compressed rows.  By
// rule (a.tile_auto) the tile grows from 2 rows up to a.tq while the
// sequence still has 128 valid queries per 2 rows of tile (about 64 tiles
// per sequence, so that short prefills still fill the chip); otherwise every
// tiled sequence takes a.tq.
__device__ __forceinline__ int seq_tile_rows(const PlanArgs& a, const SeqLens& s) {
  const sfmla_params& p = a.p;
  if (a.tq < 2 || s.q_used < a.tile_min_queries) return 0;
  int tq = a.tq;
  if (a.tile_auto) {
    tq = 2;
    while (tq < a.tq && tq * 2 * 64 <= s.q_used) tq *= 2;
  }
  int64_t n = max(s.ori_len, 0);
  if (p.ori_mask_mode == SFMLA_MASK_BAND && p.ori_win_left >= 0 && p.ori_win_right >= 0)
    n = min(n, (int64_t)p.ori_win_left + p.ori_win_right + tq);
  if (p.has_cmp_kv) n += max(s.cmp_len, 0);
  return n <= kMaxSplitRows ? tq : 0;
}

// Query tiles of consecutive rows of the tiled sequences, numbered
// sequence by sequence with no gaps, so that the workgroups of the tiled
// launch that find no tile all come after the real ones.  One workgroup:
// sequences go in chunks of kPlanThreads, an LDS scan of their tile counts
// gives each chunk's numbers, then every thread writes descriptors (first
// row, row count), finding a tile's sequence by binary search over the
// chunk's scan.  Descriptors past the last tile read (-1, 0).  Only rows
// < q_t belong to a sequence's tiles.
__device__ void plan_tiles(const PlanArgs& a) {
  const sfmla_params& p = a.p;
  __shared__ int32_t s_scan[kPlanThreads], s_first[kPlanThreads], s_row0[kPlanThreads],
      s_len[kPlanThreads], s_tq[kPlanThreads];
  const int tid = threadIdx.x;
  int32_t* desc = a.meta + a.tile_off;
  int64_t base = 0;                              // tiles of the chunks before
  for (int b0 = 0; b0 < p.batch_size; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int r0 = 0, len = 0, tq = 1;
    if (b < p.batch_size) {
      const SeqLens sl = seq_lens(a, b);
      r0 = p.layout_q == SFMLA_LAYOUT_BSND ? b * p.q_s : a.len.cu_seqlens_q[b];
      tq = seq_tile_rows(a, sl);
      len = tq > 0 ? sl.q_len : 0;
      tq = max(tq, 1);
      if (r0 < 0 || r0 >= p.q_t) len = 0;
      len = max(0, min(len, p.q_t - max(r0, 0)));
    }
    const int cnt = (len + tq - 1) / tq;
    int v = cnt;                                  // inclusive scan over the chunk
    s_scan[tid] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      v += add;
      s_scan[tid] = v;
      __syncthreads();
    }
    s_first[tid] = v - cnt;
    s_row0[tid] = r0;
    s_len[tid] = len;
    s_tq[tid] = tq;
    __syncthreads();
    const int total = s_scan[kPlanThreads - 1];
    const int last = min(kPlanThreads, p.batch_size - b0) - 1;
    for (int u = tid; u < total; u += kPlanThreads) {
      // the last sequence whose first tile is <= u holds tile u
      int lo = 0, hi = last;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_first[mid] <= u) lo = mid; else hi = mid - 1;
      }
      const int k = u - s_first[lo], tq = s_tq[lo];
      const int64_t gu = base + u;
      if (gu < a.tile_bound)
        *(int2*)(desc + kTileDescInts * gu) =
            make_int2(s_row0[lo] + tq * k, min(tq, s_len[lo] - tq * k));
    }
    base += total;
    __syncthreads();                              // before the next chunk reuses LDS
  }
  for (int64_t u = base + tid; u < a.tile_bound; u += kPlanThreads)
    *(int2*)(desc + kTileDescInts * u) = make_int2(-1, 0);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  const sfmla_params& p = a.p;
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (a.tq > 1 && blockIdx.x == 0) plan_tiles(a);
  if (row == 0) {
    a.meta[0] = kMagic;
    a.meta[1] = (int32_t)a.fingerprint;
    a.meta[2] = p.q_t;
    a.meta[3] = a.max_splits;
    for (int i = 4; i < kHeaderInts; ++i) a.meta[i] = 0;
  }
  {
    // arrival counters of every row, zeroed by all threads with coalesced
    // 16-byte stores (q_t * kCounterInts ints, a multiple of 4)
    uint4* cnt = (uint4*)(a.meta + kHeaderInts + (int64_t)p.q_t * kRecInts);
    const int64_t n4 = (int64_t)p.q_t * (kCounterInts / 4);
    for (int64_t k = row; k < n4; k += (int64_t)gridDim.x * blockDim.x) cnt[k] = make_uint4(0, 0, 0, 0);
  }
  if (row >= p.q_t) return;
  int b, i;
  if (p.layout_q == SFMLA_LAYOUT_BSND) {
    b = row / p.q_s;
    i = row - b * p.q_s;
  } else {
    int lo = 0, hi = p.batch_size - 1;  // last b with cu[b] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.len.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    b = lo;
    i = row - a.len.cu_seqlens_q[b];
  }
  const SeqLens sl = seq_lens(a, b);
  const int q_used = sl.q_used, ori_len = sl.ori_len, ori_base = sl.ori_base;
  const int cmp_len = sl.cmp_len, cmp_base = sl.cmp_base, res = sl.res;
  const int tiled = seq_tile_rows(a, sl) > 0;

  const int valid = i < q_used;
  const int pos = ori_len - q_used + i;
  const int pos_c = cmp_len * p.cmp_ratio + res - q_used + i;

  int ori_lo = 0, ori_cnt = 0;
  if (p.ori_topk > 0) {
    ori_cnt = p.ori_topk * p.ori_sparse_block_size;   // list positions (tokens)
  } else {
  int lo = 0, hi = ori_len - 1;
    if (p.ori_mask_mode == SFMLA_MASK_CAUSAL) {
      hi = pos < hi ? pos : hi;
    } else if (p.ori_mask_mode == SFMLA_MASK_BAND) {
      if (p.ori_win_left >= 0 && pos - p.ori_win_left > lo) lo = pos - p.ori_win_left;
      if (p.ori_win_right >= 0 && pos + p.ori_win_right < hi) hi = pos + p.ori_win_right;
    }
    ori_lo = lo;
    ori_cnt = hi >= lo ? hi - lo + 1 : 0;
  }
  int cmp_limit = 0, cmp_cnt = 0;
  if (p.has_cmp_kv) {
    cmp_limit = cmp_len;
    if (p.cmp_mask_mode == SFMLA_MASK_CAUSAL) {
      const int vis = pos_c + 1 >= 0 ? (pos_c + 1) / p.cmp_ratio : 0;
      cmp_limit = vis < cmp_len ? vis : cmp_len;
    }
    cmp_cnt = p.cmp_topk > 0 ? p.cmp_topk : cmp_limit;
  }
  if (!valid) { ori_cnt = 0; cmp_cnt = 0; }
  const int n = ori_cnt + cmp_cnt;
  // A sequence with many queries already gives the launch many rows: its
  // rows take longer splits, one more split_rows per kQueriesPerStep
  // queries, up to what the row table holds (fewer partials to write, read
  // back and merge).  Depends on the row's own sequence only, so a sequence
  // splits the same way in any batch.
  const int steps = q_used / kQueriesPerStep;
  const int srows = min(a.split_rows_long, a.split_rows * (steps > 1 ? steps : 1));
  int nsplit = n > 0 ? (n + srows - 1) / srows : 1;
  int chunk = srows;
  if (nsplit > a.max_splits) {
    nsplit = a.max_splits;
    chunk = (n + nsplit - 1) / nsplit;
    chunk = (chunk + kTile - 1) / kTile * kTile;
  }
  int32_t* r = a.meta + kHeaderInts + (int64_t)row * kRecInts;
  r[R_B] = b; r[R_I] = i; r[R_VALID] = valid | (tiled << 1); r[R_P] = pos; r[R_PC] = pos_c;
  r[R_ORI_LO] = ori_lo; r[R_ORI_CNT] = ori_cnt; r[R_CMP_CNT] = cmp_cnt;
  r[R_ORI_BASE] = ori_base; r[R_CMP_BASE] = cmp_base; r[R_ORI_LEN] = ori_len;
  r[R_CMP_LEN] = cmp_len; r[R_NSPLIT] = nsplit; r[R_CHUNK] = chunk;
  r[R_CMP_LIMIT] = cmp_limit; r[R_NTOTAL] = n;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

// h: the plan header, read as one 16-byte value (no chain of dependent reads)
__device__ __forceinline__ bool plan_matches(const FwdArgs& a, int4 h) {
  return (h.x == kMagic) & ((uint32_t)h.y == a.fingerprint) & (h.z == a.q_t) &
         (h.w == a.max_splits);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// The 16-bit element type of q, bf16 / fp16 kv, P and the outputs: bfloat16,
// or IEEE float16 when the kv format is SFMLA_KV_FP16 (q, kv and the output
// then share that type).  Vectors of 8 elements travel as bf16x8 bit
// patterns either way.
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
template <bool HALF>
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (HALF)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <bool HALF>
__device__ __forceinline__ uint16_t to16(float f) {
  if constexpr (HALF) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return f2bf(f);
}
template <bool HALF>
__device__ __forceinline__ __bf16 elem16(float f) {
  if constexpr (HALF) return __builtin_bit_cast(__bf16, (_Float16)f);
  else return (__bf16)f;
}
// element 0 / 1 of a pair packed in 32 bits
template <bool HALF>
__device__ __forceinline__ float lo16(uint32_t u) {
  if constexpr (HALF) return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu));
  else return __builtin_bit_cast(float, u << 16);
}
template <bool HALF>
__device__ __forceinline__ float hi16(uint32_t u) {
  if constexpr (HALF) return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
  else return __builtin_bit_cast(float, u & 0xffff0000u);
}

// 16 stored codes -> 16 bf16 values (exact: INT8 and E4M3 values fit bf16).
template <int FMT>
__device__ __forceinline__ void codes_to_bf16(uint4 c, uint4& lo, uint4& hi) {
  uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float f[4];
    if (FMT == SFMLA_KV_INT8_PACKED) {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = (float)(int8_t)((w[q] >> (8 * e)) & 0xff);
    } else {
      typedef __attribute__((ext_vector_type(2))) float f32x2;
      const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
      const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
      f[0] = a.x;
      f[1] = a.y;
      f[2] = b.x;
      f[3] = b.y;
    }
    // pairs to bf16 (round to nearest even: exact, as every code's value
    // has at most 8 significant bits)
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    o[2 * q] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)f[0], (__bf16)f[1]});
    o[2 * q + 1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)f[2], (__bf16)f[3]});
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// ---------------------------------------------------------------------------
// forward: pipelined gather with direct global -> LDS loads
// ---------------------------------------------------------------------------
//
// The split's list positions are resolved once into LDS.  KV tiles of 32 rows
// are then double-buffered: while tile t is multiplied, tile t+1 streams in
// through global_load_lds_dwordx4 (each wave instruction moves 1 KB straight
// into LDS, lane i landing at byte 16*i of the destination).  Every stage
// lives in its own LDS array so that the compiler can tell the in-flight
// loads apart from the reads of the other stage and keeps the explicit
// partial vmcnt waits; the block barrier is a bare s_barrier for the same
// reason.  Empty / masked slots load a zero row so no stale LDS bytes (which
// could hold NaN patterns) ever meet a zero probability.

__device__ __align__(16) const uint4 g_zero_row[72] = {};

// Wait until at most N vector-memory ops of this wave are outstanding (the
// counter has 6 bits: larger N waits for slightly more than needed).
template <int N0>
__device__ __forceinline__ void wait_vmcnt() {
  constexpr int N = N0 > 63 ? 63 : N0;
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void;

// One global_load_lds_dwordx4: every lane moves 16 bytes from `g` to LDS at
// lds_wave_base + 16 * lane (the LDS base is taken from M0).  Issued through
// inline asm so that the compiler's wait insertion neither tracks these loads
// (it cannot tell the in-flight stage apart from the stage being read and
// would wait for all of them) nor reorders LDS reads across them ("memory"
// clobber).  Every wait on this data is explicit (wait_vmcnt +
// block_barrier).  Untracked vector-memory ops only make the compiler's own
// in-order vmcnt waits stricter, never insufficient.  M0 is an input operand
// ("{m0}"): the compiler writes it and knows its value is read here, so no
// register it holds is clobbered behind its back; s_nop 0 gives the one wait
// state an LDS DMA needs after an M0 write.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "{m0}"(lds_addr)
               : "memory");
}

// The same with a uniform row address in an SGPR pair (lane offset in a
// VGPR).  s_nop 4 gives the five wait states a VMEM instruction needs after a
// VALU write (v_readlane) of an SGPR it reads, which also covers the M0 write.
__device__ __forceinline__ void dma16_s(uint64_t base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "{m0}"(lds_addr)
               : "memory");
}

// The same with the agent-scope cache policy (sc1): data another workgroup
// stored with sc1 stores (split partials).
__device__ __forceinline__ void dma16_sc1(const void* g, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1"
               :
               : "v"(g), "{m0}"(lds_addr)
               : "memory");
}

// 64-bit value held by lane j, as a uniform (SGPR) value.
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, j);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}

// After an explicit full vmcnt wait: make an empty asm the last writer of
// the loaded registers, so the compiler's wait tracking cannot attribute a
// pending memory load to them inside the tile loop.
template <int A, int B>
__device__ __forceinline__ void settle(bf16x8 (&r)[A][B]) {
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int j = 0; j < B; ++j) asm volatile("" : "+v"(r[i][j]));
}

// Cross-workgroup exchange of split partials.  The partials and their LSEs
// are written and read with agent-scope accesses (sc1 cache policy: the code
// the gfx950 memory model uses for relaxed agent-scope atomic loads and
// stores, coherent per location across all XCDs) without the whole-L2
// write-back / invalidate that an agent-scope fence costs.  Ordering against
// the arrival counter comes from waiting for every store of the wave to
// complete (vmcnt 0) before the counter update; the merging workgroup issues
// its loads only after it has read the counter.  Partials move as 16-byte
// buffer accesses (one full 16-byte chunk per lane), so no line is written
// or fetched twice.
constexpr int kSc1 = 16;                 // cache-policy bit sc1 of buffer ops
constexpr int kBufWord3 = 0x00020000;    // raw buffer descriptor, 32-bit data format
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, kBufWord3);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load((float*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every vector-memory op of this wave (stores included) has completed
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS byte address of a __shared__ object.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)p;
}
// 16 bytes at an LDS byte address
__device__ __forceinline__ uint4 lds_ld16(uint32_t addr) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = *(const __attribute__((address_space(3))) v4u*)(uintptr_t)addr;
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int NW, int DQK, int VMODE>
struct Pipe {
  static constexpr int T = kTile;
  static constexpr int RSTR = 1024 + 32;      // LDS row stride: conflict-free K and V^T reads
  static constexpr bool ROPE = DQK == 576;
  static constexpr int NR = T / NW;           // rows each wave gathers per tile
  static constexpr int ROPE_INSTR = ROPE ? (NR >= 8 ? NR / 8 : 1) : 0;
  static constexpr int NK = NR + ROPE_INSTR;  // K-side loads per wave per tile
  static constexpr int NV = VMODE ? NR : 0;   // V-side loads per wave per tile
  static constexpr int KBYTES = T * RSTR + (ROPE ? T * 128 : 0);
};

// A resolved list position, as kept in LDS: the physical row id, with bit 31
// set for the compressed KV; kNoRow for an empty or masked slot, which reads
// the zero row.  Row ids stay below 2^31 - 1 (checked on the host).
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
constexpr uint32_t kCmpBit = 0x80000000u;

__device__ __forceinline__ const char* row_at(const char* base, uint32_t phys, uint32_t stride) {
  return base + (uint64_t)phys * stride;
}
// (the host gives every side a V and a rope base: the K row itself and the
// bytes after its nope when they are not stored apart)
__device__ __forceinline__ const char* k_addr(const FwdArgs& a, uint32_t e) {
  if (e == kNoRow) return (const char*)g_zero_row;
  const bool c = e & kCmpBit;
  return row_at(c ? a.cmp_kv : a.ori_kv, e & ~kCmpBit, c ? a.cmp_stride : a.ori_stride);
}
__device__ __forceinline__ const char* v_addr(const FwdArgs& a, uint32_t e) {
  if (e == kNoRow) return (const char*)g_zero_row;
  const bool c = e & kCmpBit;
  return row_at(c ? a.cmp_kv : a.ori_v, e & ~kCmpBit, c ? a.cmp_stride : a.ori_v_stride);
}
__device__ __forceinline__ const char* rope_addr(const FwdArgs& a, uint32_t e) {
  if (e == kNoRow) return (const char*)g_zero_row;
  const bool c = e & kCmpBit;
  return row_at(c ? a.cmp_rope : a.ori_rope, e & ~kCmpBit,
                c ? a.cmp_rope_stride : a.ori_rope_stride);
}

// K side of one tile: 512 nope values per row (1 KB per wave instruction) and,
// with rope, 8 rows of 64 rope values per instruction (row r's 16-byte chunk c
// lands at position c ^ ((r >> 1) & 7) of its 128-byte LDS row, which keeps
// the 16-row reads conflict-free).  The wave's row entries are read from LDS
// once (lane j holds row j) before the first load is issued (the loads'
// "memory" clobber would otherwise serialise one LDS round trip per load);
// each row's addresses are then computed in SGPRs from its entry, handed out
// with v_readlane, and a rope lane picks its row's address from them.
template <int NW, int DQK, int VMODE>
__device__ __forceinline__ void issue_k(const FwdArgs& a, const uint32_t* sRow, int tbase,
                                        uint32_t ldsK, int w, int l) {
  using C = Pipe<NW, DQK, VMODE>;
  const uint32_t wk = __builtin_amdgcn_readfirstlane(ldsK + w * C::NR * C::RSTR);
  const uint32_t mine = sRow[tbase + w * C::NR + (l < C::NR ? l : 0)];
  const char* rsrc[C::ROPE ? C::ROPE_INSTR : 1];
#pragma unroll
  for (int j = 0; j < C::NR; ++j) {
    const uint32_t e = __builtin_amdgcn_readlane(mine, j);
    dma16_s((uint64_t)k_addr(a, e), l * 16, wk + j * C::RSTR);
    if constexpr (C::ROPE) {
      // rope instruction j / 8, lanes 8 (j % 8) .. 8 (j % 8) + 7 (row 0's
      // address also fills the lanes of rows past NR, which issue nothing)
      const char* ra = rope_addr(a, e);
      if (j % 8 == 0 || (l >> 3) == j % 8) rsrc[j / 8] = ra;
    }
  }
  if constexpr (C::ROPE) {
    const uint32_t wr = __builtin_amdgcn_readfirstlane(ldsK + kTile * C::RSTR + w * C::NR * 128);
#pragma unroll
    for (int q = 0; q < C::ROPE_INSTR; ++q) {
      const int rr = w * C::NR + 8 * q + ((l >> 3) < C::NR ? (l >> 3) : 0);
      const int chunk = (l & 7) ^ ((rr >> 1) & 7);
      if (C::NR >= 8 || (l >> 3) < C::NR) dma16(rsrc[q] + chunk * 16, wr + q * 1024);
    }
  }
}

template <int NW, int DQK, int VMODE>
__device__ __forceinline__ void issue_v(const FwdArgs& a, const uint32_t* sRow, int tbase,
                                        uint32_t ldsV, int w, int l) {
  using C = Pipe<NW, DQK, VMODE>;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(ldsV + w * C::NR * C::RSTR);
  const uint32_t mine = sRow[tbase + w * C::NR + (l < C::NR ? l : 0)];
#pragma unroll
  for (int j = 0; j < C::NR; ++j) {
    const uint32_t e = __builtin_amdgcn_readlane(mine, j);
    dma16_s((uint64_t)v_addr(a, e), l * 16, wv + j * C::RSTR);
  }
}

// Packed rows (512 INT8 / FP8-E4M3 codes, the bf16 rope, four fp32 scales of
// 128 columns each) are gathered as raw bytes: tile rows lie back to back in
// the LDS stage (row stride = the packed row size), each wave instruction
// moving 64 consecutive 16-byte chunks, which may span several rows.  Padding
// lanes (past the tile) read the zero row into the stage's tail so that every
// wave issues the same number of loads.
// A lane value the compiler cannot prove loop-invariant (an empty asm that
// takes it and gives it back, in a register): per-lane addresses derived
// from it are recomputed where they are used instead of being hoisted out
// of the tile loop and held in registers (on the eight-wave packed kernel
// they were spilled to scratch and reloaded every tile; the four-wave one
// has the registers and keeps them).
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int NW, int DQK, int VC = 0>
struct PackedPipe {
  static constexpr int ROPE = DQK - 512;                     // rope values per row
  static constexpr int KC = (512 + 2 * ROPE + 16) / 16;       // 16-byte chunks of a key row
  // chunks per row in the stage: the key row, then (VC) the row's 512 value
  // codes from the value tensor
  static constexpr int CPR = KC + (VC ? 32 : 0);
  static constexpr int NI = (kTile * CPR + 63) / 64;          // instructions per tile
  static constexpr int PER = (NI + NW - 1) / NW;              // per wave
  static constexpr int RAWB = PER * NW * 1024;                // LDS bytes per stage
};

template <int NW, int DQK, int VC = 0>
__device__ __forceinline__ void issue_raw(const FwdArgs& a, const uint32_t* sRow, int tbase,
                                          uint32_t ldsRaw, int w, int l) {
  using P = PackedPipe<NW, DQK, VC>;
  if constexpr (NW == 8) l = fresh(l);   // two waves per SIMD: no room for hoisted addresses
  const uint32_t base = __builtin_amdgcn_readfirstlane(ldsRaw + w * P::PER * 1024);
  // every row entry first (one LDS round trip for all), then branch-free
  // addresses: a slot without a row, and chunks past the tile (the last
  // wave's tail), read the zero row
  uint32_t e[P::PER];
#pragma unroll
  for (int q = 0; q < P::PER; ++q) {
    const int c = (w * P::PER + q) * 64 + l;                  // chunk index in the tile
    e[q] = sRow[tbase + min(c / P::CPR, kTile - 1)];
  }
#pragma unroll
  for (int q = 0; q < P::PER; ++q) {
    const int c = (w * P::PER + q) * 64 + l;
    const int r = c / P::CPR;
    const int j = c - r * P::CPR;                             // chunk within the row
    const char* rowp;
    if constexpr (VC) {
      // chunks past the key row: the value tensor's row, chunk j - KC of its
      // 512 code bytes (only original-KV rows: the host refuses a value
      // tensor with a compressed KV)
      const bool vc = j >= P::KC;
      rowp = row_at(vc ? a.ori_v : a.ori_kv, e[q], vc ? a.ori_v_stride : a.ori_stride) +
             16 * (vc ? j - P::KC : j);
    } else {
      const bool cmp = e[q] & kCmpBit;
      rowp = row_at(cmp ? a.cmp_kv : a.ori_kv, e[q] & ~kCmpBit,
                    cmp ? a.cmp_stride : a.ori_stride) + 16 * j;
    }
    const bool zero = e[q] == kNoRow || c >= kTile * P::CPR;
    dma16(zero ? (const char*)g_zero_row : rowp, base + q * 1024);
  }
}

// Lane exchanges within a wave on the VALU (gfx950 v_permlane16_swap /
// v_permlane32_swap, no LDS round trip).  Given the same value twice, the
// 16-lane swap returns (x of lane l & ~16, x of lane l | 16) and the 32-lane
// swap (x of lane l & ~32, x of lane l | 32), so every lane of a pair gets
// the same operands in the same order.
__device__ __forceinline__ void pair16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void pair32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one head's 32
// rows of a tile in the score layout)
__device__ __forceinline__ float max4(float x) {
  float a, b;
  pair16(x, a, b);
  pair32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum4(float x) {
  float a, b;
  pair16(x, a, b);
  pair32(a + b, a, b);
  return a + b;
}

// Raw packed tile -> the bf16 K tile the MFMA path reads (codes decoded
// exactly; rope copied into its swizzled region) and the tile's scales,
// stored scale-tile major: sScale[32 * j + row] for columns [128 j, 128 j + 128).
template <int NW, int DQK, int FMT, int VC = 0>
__device__ __forceinline__ void decode_tile(const char* raw, char* kbf, float* sScale, int tid) {
  using P = PackedPipe<NW, DQK, VC>;
  constexpr int NTHR = NW * 64;
  constexpr int RB = P::CPR * 16;
  constexpr int RS = 1024 + 32;
  constexpr int NIT = kTile * 32 / NTHR;          // 16-code chunks per thread
  constexpr int U = NIT < 4 ? NIT : 4;            // chunks read before any is converted
  static_assert(kTile * 32 % NTHR == 0 && NIT % U == 0, "decode split");
  if constexpr (NW == 8) tid = fresh(tid);
#pragma unroll
  for (int i0 = 0; i0 < NIT; i0 += U) {
    uint4 c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = tid + (i0 + u) * NTHR;
      c[u] = *(const uint4*)(raw + (i >> 5) * RB + 16 * (i & 31));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = tid + (i0 + u) * NTHR;
      uint4 lo, hi;
      codes_to_bf16<FMT>(c[u], lo, hi);
      *(uint4*)(kbf + (i >> 5) * RS + 32 * (i & 31)) = lo;
      *(uint4*)(kbf + (i >> 5) * RS + 32 * (i & 31) + 16) = hi;
    }
  }
  if constexpr (P::ROPE > 0) {
    for (int i = tid; i < kTile * 8; i += NTHR) {
      const int r = i >> 3, c = i & 7;
      *(uint4*)(kbf + kTile * RS + r * 128 + 16 * (c ^ ((r >> 1) & 7))) =
          *(const uint4*)(raw + r * RB + 512 + 16 * c);
    }
  }
  for (int i = tid; i < kTile; i += NTHR) {
    const float4 sc = *(const float4*)(raw + i * RB + 512 + 2 * P::ROPE);
    sScale[i] = sc.x;
    sScale[kTile + i] = sc.y;
    sScale[2 * kTile + i] = sc.z;
    sScale[3 * kTile + i] = sc.w;
  }
}

// The value tensor's codes of a raw tile (stored after each key row in the
// stage) -> the nope columns of the bf16 tile, where the key's codes were;
// the rope columns and the row scales (the key row's) stay.
template <int NW, int DQK, int FMT>
__device__ __forceinline__ void decode_value(const char* raw, char* kbf, int tid) {
  using P = PackedPipe<NW, DQK, 1>;
  constexpr int NTHR = NW * 64;
  constexpr int RB = P::CPR * 16;
  constexpr int RS = 1024 + 32;
  constexpr int NIT = kTile * 32 / NTHR;          // 16-code chunks per thread
  constexpr int U = NIT < 4 ? NIT : 4;
  static_assert(kTile * 32 % NTHR == 0 && NIT % U == 0, "decode split");
  if constexpr (NW == 8) tid = fresh(tid);
#pragma unroll
  for (int i0 = 0; i0 < NIT; i0 += U) {
    uint4 c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = tid + (i0 + u) * NTHR;
      c[u] = *(const uint4*)(raw + (i >> 5) * RB + 16 * P::KC + 16 * (i & 31));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = tid + (i0 + u) * NTHR;
      uint4 lo, hi;
      codes_to_bf16<FMT>(c[u], lo, hi);
      *(uint4*)(kbf + (i >> 5) * RS + 32 * (i & 31)) = lo;
      *(uint4*)(kbf + (i >> 5) * RS + 32 * (i & 31) + 16) = hi;
    }
  }
}

// Running-max growth (log2 units) below which the accumulators are not
// rescaled: probabilities then stay below 2^8 and the normaliser uses the
// same (stale) max, so the result is unchanged while the accumulators are
// touched only when the max jumps.
constexpr float kRescaleThreshold = 8.0f;
constexpr int kMergeSplits = 4;       // splits whose partials one merge round loads (8 waves)
constexpr int kMaxOwnerSplits = 8;    // splits of a row whose partials an owning wave merges
template <int N>
struct IntC {                         // a compile-time int passed as an argument
  static constexpr int value = N;
};

// Position of slot u of a resolve batch starting at i0 (PPT slots per thread).
// bf16 rows: wave w resolves exactly the rows it gathers (row w*NR + l%NR of
// tile l/NR, then the next 64/NR tiles for u = 1).  Packed rows (gathered in
// 16-byte chunks across rows): one position per thread in order.
template <int NW, int DQK, int VMODE, bool PK, int PPT>
__device__ __forceinline__ int posn_of(int i0, int u, int tid, int w, int l) {
  if constexpr (PK) {
    return i0 + tid + u * NW * 64;
  } else {
    constexpr int NR = Pipe<NW, DQK, VMODE>::NR, TPB = 64 / NR;
    static_assert(PPT * TPB * kTile == PPT * NW * 64, "a batch covers PPT*NTHR positions");
    return i0 + (u * TPB + l / NR) * kTile + w * NR + (l % NR);
  }
}

// HB head blocks of 16 heads per wave; FMT is the KV storage format.
// TILED: the launch starts with a.tile_units workgroups, one per query tile
// (a.tq consecutive rows of a sequence, a.nb head blocks each): the tile's
// union list is resolved and gathered once, wave w computes row w / a.nb's
// head block w % a.nb and masks the union positions its row's list does not
// hold.  The rows of sequences that are not tiled follow, one workgroup per
// (split, row) with every head (one head group), as without tiles.
// PAIR: two waves share 16 heads.  Each computes the scores of one 16-row
// half of every tile, the pair swaps its raw scores through LDS, both run the
// same softmax over all 32 rows, and each accumulates half of the value
// columns (16 heads x 256 columns of accumulators): a row of at most 64
// heads keeps all eight waves, two per SIMD, in the products.  Every MFMA
// and every softmax step is the one a single wave holding those heads would
// take, so the results are the same bits.
// Four waves with 16-bit rows (d_qk 512, V = K nope): a two-stage K ring
// and no owned merge keep the workgroup within half the LDS and its waves
// within 256 registers, so two workgroups share a CU and every SIMD has two
// waves in the products.
template <int NW, int FMT>
constexpr bool kTwoPerCu = NW == 4 && (FMT == SFMLA_KV_BF16 || FMT == SFMLA_KV_FP16);

template <int NW, int HB, int DQK, int VMODE, int FMT, bool TILED = false, bool PAIR = false>
__global__ __launch_bounds__(NW * 64, (kTwoPerCu<NW, FMT> ? 2 : 1)) void fwd_kernel(FwdArgs a) {
  using C = Pipe<NW, DQK, VMODE>;
  constexpr bool HALF = FMT == SFMLA_KV_FP16;     // float16 q / kv / P / output
  constexpr bool PK = FMT != SFMLA_KV_BF16 && !HALF;   // packed rows (V = decoded nope)
  // packed KV with VMODE: the value codes come from their own tensor
  constexpr bool PKV = PK && VMODE;
  using PP = PackedPipe<NW, DQK, PKV ? 1 : 0>;
  static_assert(!TILED || (!PK && NW == 8 && HB == 1), "query tiles: 16-bit rows, 8 waves");
  static_assert(!PAIR || (!TILED && NW == 8 && HB == 1), "wave pairs: 8 waves");
  constexpr bool W4 = kTwoPerCu<NW, FMT>;
  static_assert(!W4 || (VMODE == 0 && DQK == 512 && !TILED && !PAIR && HB == 1),
                "four-wave 16-bit rows: d_qk 512, V = K nope");
  static_assert(FMT == SFMLA_KV_BF16 || FMT == SFMLA_KV_INT8_PACKED ||
                FMT == SFMLA_KV_FP8_E4M3_PACKED || FMT == SFMLA_KV_FP16, "KV format");
  constexpr int T = C::T;
  constexpr int NKS = DQK / 32;
  constexpr int NTHR = NW * 64;
  constexpr int HPW = 16 * HB;                     // heads per wave (per pair)
  constexpr int NMB = PAIR ? 16 : 32;              // 16-column blocks of O per wave
  constexpr int NPW = PAIR ? NW / 2 : NW;          // head-holding units (waves or pairs)
  constexpr int RS = C::RSTR;
  // bf16, separate V: two K stages and two V stages; bf16, aliased V: three K
  // stages; packed: three raw stages and one decoded K tile (sK0)
  __shared__ __align__(16) char sK0[C::KBYTES];
  __shared__ __align__(16) char sK1[PK ? 16 : C::KBYTES];
  __shared__ __align__(16) char sK2[(VMODE || PK || W4) ? 16 : C::KBYTES];
  __shared__ __align__(16) char sV0[(VMODE && !PK) ? T * RS : 16];
  __shared__ __align__(16) char sV1[(VMODE && !PK) ? T * RS : 16];
  __shared__ __align__(16) char sW0[PK ? PP::RAWB : 16];
  __shared__ __align__(16) char sW1[PK ? PP::RAWB : 16];
  __shared__ __align__(16) char sW2[(PK && !PKV) ? PP::RAWB : 16];
  __shared__ __align__(16) float sScale[PK ? 4 * T : 4];
  __shared__ uint32_t sRow[kMaxSplitRows + T];      // resolved positions of the split
  // bf16 / fp16 with a separate V: a merging wave stages its output in the
  // K / V stage buffers (two waves per buffer) once every wave of the
  // workgroup is done with them (sOut counts the waves out); owning waves
  // (below) land the other splits' partials there
  constexpr bool STAGE = VMODE && !PK && !PAIR;
  constexpr bool OUTCNT = !PK;
  constexpr int kStgRow = 1040;                      // staged output row (one head), padded
  static_assert(!STAGE || (NW == 8 && 2 * 16 * kStgRow <= T * RS && T * RS <= C::KBYTES),
                "output staging: two waves' 16 heads per stage buffer");
  __shared__ int32_t sOut;
  // V = K nope: two more landing slots for the owned merge (the separate-V
  // kernel has its V stages for them; the tiled kernel merges splits of its
  // untiled rows with the last split to arrive)
  __shared__ __align__(16) char sM[(VMODE || PK || TILED || PAIR || W4) ? 16 : 32768];
  // owned merge: per owning wave, every split's weight and the normaliser
  // per head, and a flag (1: landed and weighted, 2: handed off)
  __shared__ float sWs[(PK || TILED || PAIR || W4) ? 1 : NW][(PK || TILED || PAIR || W4) ? 1 : kMaxOwnerSplits][16];
  __shared__ float sInv[(PK || TILED || PAIR || W4) ? 1 : NW][16];
  // wave pairs: each wave's raw scores of its 16 tile rows, per head block
  __shared__ __align__(16) f32x4 sSx[PAIR ? NW : 1][PAIR ? HB : 1][64];
  __shared__ int32_t sReady[NW];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 4, t = l & 15;
  const int hf = PAIR ? (w & 1) : 0;                // wave pairs: this wave's half
  const int wp = PAIR ? (w >> 1) : w;               // head-holding unit
  // NaN outputs of query row r for this wave's heads (a plan that does not
  // match, or a list longer than the parameters allow)
  auto fail_row = [&](int r, int hfirst, bool on) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = hfirst + 16 * hb + t;
      if (!on || h >= a.qn) continue;
      uint16_t* op = a.out + ((int64_t)r * a.qn + h) * 512;
      for (int c = g; c < 512; c += 4) op[c] = to16<HALF>(__builtin_nanf(""));
      if (a.lse && g == 0) a.lse[(int64_t)r * a.qn + h] = __builtin_nanf("");
    }
  };
  int row;            // the query row whose plan record gives the list's sequence
  int orow;           // the query row this wave computes
  int split, hg, h0, nsplit, n, chunk;
  bool wave_on;
  const int32_t* rec;
  RowInfo ri;
  constexpr int PPT = (512 + T + NTHR - 1) / NTHR;   // positions per thread and batch
  int vspec[PPT];
  // tiles: the union positions this wave's row holds are [m_a0, m_a0 + m_cnt)
  // (original KV) and [m_ucnt, m_ucnt + m_cc) (compressed KV); a row's own
  // list holds every position
  int m_a0 = 0, m_cnt = 0x7fffffff, m_ucnt = 0, m_cc = 0;
  if (TILED && (int)blockIdx.x < a.tile_units) {
    // Tiles are numbered without gaps (descriptor: first row, row count), so
    // the workgroups past the last tile, which exit at once, all come after
    // the real ones.  Tile u is dealt to XCD u mod 8.
    const int unit = blockIdx.x;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    const int tau = wu / a.nb;                      // this wave's row in the tile
    split = 0;
    hg = 0;
    h0 = (wu - tau * a.nb) * HPW;
    const int4 hdr = *(const int4*)a.meta;
    const int2 ud = *(const int2*)(a.meta + a.tile_off + (int64_t)kTileDescInts * unit);
    // a plan of other parameters: the rows' workgroups that follow the tiles
    // (split 0 of every row) write the NaN outputs and the status
    if (!plan_matches(a, hdr)) return;
    const int ntok = ud.y;
    if (ud.x < 0 || ntok < 1 || ntok > a.tq || ud.x > a.q_t - ntok) return;   // no tile
    row = ud.x;
    orow = row + min(tau, ntok - 1);
    wave_on = tau < ntok && h0 < a.qn;
    rec = a.meta + kHeaderInts + (int64_t)row * kRecInts;
    ri = row_info(rec);
    // every row's list extents: lane j reads row min(j, ntok - 1) of the tile
    const int32_t* rj = a.meta + kHeaderInts + (int64_t)(row + min(l & 7, ntok - 1)) * kRecInts;
    const int olo = rj[R_ORI_LO], ocnt = rj[R_ORI_CNT], occ = rj[R_CMP_CNT];
    // union: the window rows from the first row's start to the last row's end
    // (consecutive rows' windows overlap or touch, and a position of the
    // union outside a row's own window is masked for it anyway), and the
    // visible compressed rows of the row that sees the most
    int ulo = 0x7fffffff, uhi = -0x7fffffff - 1, ucc = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = __builtin_amdgcn_readlane(ocnt, j), lo = __builtin_amdgcn_readlane(olo, j);
      if (c > 0) {
        ulo = min(ulo, lo);
        uhi = max(uhi, lo + c);
      }
      ucc = max(ucc, __builtin_amdgcn_readlane(occ, j));
    }
    const int ucnt = uhi > ulo ? uhi - ulo : 0;
    if (ucnt == 0) ulo = 0;
    const int me = min(tau, ntok - 1);
    const int my_cnt = __builtin_amdgcn_readlane(ocnt, me);
    m_a0 = my_cnt > 0 ? __builtin_amdgcn_readlane(olo, me) - ulo : 0;
    m_cnt = my_cnt;
    m_ucnt = ucnt;
    m_cc = __builtin_amdgcn_readlane(occ, me);
    ri.ori_lo = ulo;
    ri.ori_cnt = ucnt;
    ri.cmp_limit = ucc;
    n = ucnt + ucc;
    nsplit = 1;
    chunk = n;
  } else {
    // 1-D grid: workgroups are dealt to the 8 XCDs round-robin, so XCD x = bid
    // mod 8 takes the query rows 8k + x, and within it slot bid / 8 runs over
    // (split, k, head group), split slowest: every split and head group of a
    // row is on one XCD, so the groups' repeated gathers and the merger's reads
    // of the other splits' partials stay within that XCD's L2.  Split-major
    // order puts the workgroups of splits a row does not have (its list is
    // shorter than the longest) after all the real ones; interleaved between
    // them they were measured to slow a one-split launch by a third.
    const int G = a.groups;
    const int K8 = (a.q_t + 7) >> 3;
    const int bid = (int)blockIdx.x - (TILED ? a.tile_units : 0);   // a multiple of 8
    const int slot = bid >> 3;
    hg = slot % G;
    split = slot / G / K8;
    row = ((slot / G) % K8) * 8 + (bid & 7);
    if (row >= a.q_t) return;
    orow = row;
    // a head group holds a.bpg 16-head blocks; waves past them only gather
    h0 = (hg * a.bpg + wp) * HPW;                   // first head of this wave
    wave_on = wp < a.bpg && h0 < a.qn;

    // The row's plan record is read together with the plan header (the buffer
    // always holds both; its size is checked on the host), so the two reads
    // cost one round trip; the record is only used once the header matches.
    const int4 hdr = *(const int4*)a.meta;
    rec = a.meta + kHeaderInts + (int64_t)row * kRecInts;
    nsplit = rec[R_NSPLIT];
    n = rec[R_NTOTAL];
    chunk = rec[R_CHUNK];
    ri = row_info(rec);
    // Index loads of the first resolve batch, issued in the same round trip:
    // where the original-KV list is a TopK list its length is fixed by the
    // parameters, so a position's entry does not depend on the plan record
    // unless the row is empty or split in other chunks (a long-query row);
    // the resolve below reloads in those cases.  Every load is in bounds
    // (positions past the lists read the plan header instead).
    const int spec_cnt0 = a.ori_topk << a.ori_sbs_log2;
    const int spec_cap = a.ori_topk > 0 ? spec_cnt0 + (a.cmp_topk > 0 ? a.cmp_topk : 0) : 0;
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int i = posn_of<NW, DQK, VMODE, PK, PPT>(0, u, tid, w, l);
      const int k = split * a.split_rows + i;
      const int32_t* ep = (const int32_t*)a.meta;
      if (i < a.split_rows && k < spec_cap)
        ep = k < spec_cnt0 ? a.ori_idx + (int64_t)row * a.ori_topk + (k >> a.ori_sbs_log2)
                           : a.cmp_idx + (int64_t)row * a.cmp_topk + (k - spec_cnt0);
      vspec[u] = *ep;
    }
    if (!plan_matches(a, hdr)) {
      if (split == 0) {
        fail_row(row, h0, wave_on);
        if (a.status && tid == 0) atomicOr(a.status, SFMLA_STATUS_METADATA_MISMATCH);
      }
      return;
    }
    if (split >= nsplit) return;
    if (TILED && (rec[R_VALID] & 2)) return;        // the row is in a tile
  }
  if (chunk > kMaxSplitRows) {
    // a list longer than the parameters' maxima allow: refuse the row
    if (split == 0) {
      fail_row(orow, h0, wave_on);
      if (a.status && tid == 0) atomicOr(a.status, SFMLA_STATUS_LIST_TOO_LONG);
    }
    return;
  }
  const int spec_cnt = a.ori_topk << a.ori_sbs_log2;
  // bf16 rows: each wave resolves the rows it gathers, so it can issue its
  // share of the first tiles as soon as its own entries are in, with no
  // workgroup barrier
  auto posn = [&](int i0, int u) -> int { return posn_of<NW, DQK, VMODE, PK, PPT>(i0, u, tid, w, l); };
  const int k0 = split * chunk;
  const int k1 = min(n, k0 + chunk);
  const int nt = (k1 - k0 + T - 1) / T;

  // Q slices (B operand: k = d, n = head).  They are loaded right after the
  // table loads of the resolve below: loads complete in order, so waiting
  // for the table entries does not wait for Q, which travels while the
  // entries go to LDS.  Every load here is an ordinary one the compiler
  // tracks: it places the waits for its results itself.
  // Q slices held in registers: every k-step, except on the eight-wave packed
  // kernel with rope, whose two waves per SIMD keep the two rope k-steps in
  // LDS (16 KB; loaded two MFMA steps ahead of their use)
  constexpr int NQR = (PK && NW == 8 && C::ROPE) ? 16 : NKS;
  __shared__ __align__(16) bf16x8 sQr[NQR < NKS ? NW : 1][NQR < NKS ? NKS - NQR : 1][64];
  bf16x8 qreg[HB][NQR];
  bf16x8 qrt[NQR < NKS ? NKS - NQR : 1];
  // ---- resolve every list position of this split once, into physical row
  //      entries in LDS (empty or masked slots: kNoRow).  Positions go in
  //      batches of PPT per thread: the index loads of a batch, then its
  //      table loads, are all in flight together; the first batch covers a
  //      512-row split, the Q loads follow its table loads.
  {
    const int ntT = nt * T;
    const bool spec = !TILED && a.ori_topk > 0 && chunk == a.split_rows && ri.ori_cnt == spec_cnt;
    auto batch = [&](int i0, bool use_spec, auto&& between) {
      int vv[PPT], jj[PPT], sd[PPT], ee[PPT];
      bool he[PPT];
      if (use_spec) {
#pragma unroll
        for (int u = 0; u < PPT; ++u) vv[u] = vspec[u];
      } else {
        // loads are unconditional (a position without an entry reads its own
        // plan record), and waited for inside this branch, so that no branch
        // join waits for them
#pragma unroll
        for (int u = 0; u < PPT; ++u) {
          const int i = posn(i0, u);
          const int k = k0 + i;
          const int32_t* ep = (i < ntT && k < k1) ? slot_entry(a, ri, row, k) : nullptr;
          vv[u] = *(ep ? ep : rec);
        }
#pragma unroll
        for (int u = 0; u < PPT; ++u) asm volatile("" ::"v"(vv[u]));
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int i = posn(i0, u);
        const int k = k0 + i;
        sd[u] = 0;
        jj[u] = (i < ntT && k < k1) ? slot_row(a, ri, k, vv[u], &sd[u]) : -1;
      }
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int32_t* tp = table_entry(a, ri, jj[u], sd[u]);
        he[u] = tp != nullptr;
        ee[u] = *(tp ? tp : rec);
      }
      __builtin_amdgcn_sched_barrier(0);            // every table load before the Q loads
      between();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < PPT; ++u) {
        const int i = posn(i0, u);
        if (i >= ntT) continue;
        const int64_t phys = phys_row(a, ri, jj[u], sd[u], he[u], ee[u]);
        sRow[i] = phys >= 0 ? (uint32_t)phys | (sd[u] ? kCmpBit : 0u) : kNoRow;
      }
    };
    batch(0, spec, [&] {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        // unconditional loads (a branch join would wait for them): lanes of
        // heads past q_n read head 0; their scores stay in their own lanes
        // and their outputs are never written
        // (row * q_n + head < 2^31, checked on the host; a 32-bit index
        // here also keeps it from being held until the epilogue)
        const int h = h0 + 16 * hb + t;
        const int qi = orow * a.qn + (h < a.qn ? h : 0);
        const uint16_t* qp = a.q + (uint32_t)qi * (uint64_t)a.q_stride + 8 * g;
        // the rope k-steps (16, 17) read q_rope when it is stored apart
        const uint16_t* qr = a.q_rope ? a.q_rope + (uint32_t)qi * (uint64_t)64 + 8 * g - 512 : qp;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 v = __builtin_bit_cast(bf16x8, *(const uint4*)((ks < 16 ? qp : qr) + 32 * ks));
          if (ks < NQR) qreg[hb][ks < NQR ? ks : 0] = v;
          else qrt[ks - NQR] = v;
        }
      }
    });
    for (int i0 = PPT * NTHR; i0 < ntT; i0 += PPT * NTHR) batch(i0, false, [] {});
  }
  // one more tile of empty entries after the resolved positions: a read of
  // the row table past them finds the zero row, never stale LDS
  if (tid < T) sRow[nt * T + tid] = kNoRow;
  if (OUTCNT && tid == 0) sOut = 0;
  if (OUTCNT && tid < NW) sReady[tid] = 0;
  if constexpr (PK) {
    wait_lgkm0();
    block_barrier();
  }

  f32x4 o[HB][NMB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) o[hb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[HB], l_run[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) { m_run[hb] = kNegInf; l_run[hb] = 0.f; }
  bf16x8 pb[HB];
  // packed rows: the probabilities in fp32 (this lane's 8 rows), scaled by
  // each 128-column tile's row scales just before that tile's PV products
  float pj32[PK ? HB : 1][8];

  // ---- S^T = K Q^T, online softmax -> pb (M = 16 rows, N = 16 heads per MFMA).
  // The operands of the next PF k-steps are in flight while step ks
  // multiplies; sched_barrier fences pin that order.
  auto qk_softmax = [&](const char* sK, int tbase) {
    const char* sR = sK + T * RS;
    // The tile rows that take part for this wave, one bit per row: a KV row
    // behind the position (lanes l and l + 32 read row l mod 32), and with
    // tiles the position in this wave's row's own list (two intervals of the
    // union, intersected in scalar registers).  A full tile takes no
    // per-element selects.
    uint32_t vm = (uint32_t)__ballot(sRow[tbase + (l & 31)] != kNoRow);
    if constexpr (TILED) {
      auto span = [&](int lo, int cnt) -> uint32_t {
        const int a0 = max(lo - tbase, 0), a1 = min(lo - tbase + cnt, 32);
        return a1 > a0 ? (uint32_t)((((uint64_t)1 << a1) - 1) & ~(((uint64_t)1 << a0) - 1)) : 0u;
      };
      vm &= span(m_a0, m_cnt) | span(m_ucnt, m_cc);
    }
    const bool full = vm == 0xffffffffu;
    // this lane's rows {4g + i, 16 + 4g + i}: bit j of nib <-> x[j] below
    const uint32_t nib = ((vm >> (4 * g)) & 0xfu) | (((vm >> (16 + 4 * g)) & 0xfu) << 4);
    f32x4 s[HB][2];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) s[hb][0] = s[hb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // wave pairs: this wave's 16-row half of the scores (the partner's comes
    // through LDS below)
    f32x4 sm[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) sm[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (PK) {
      // Packed rows: exact scaling, one partial product per 128-column scale
      // tile, taken one 16-row half of the tile at a time (the partial sums,
      // K operands and row scales of one half are live at once).
      auto pk_half = [&](int half, auto&& acc) __attribute__((always_inline)) {
        const char* kp = sK + (16 * half + t) * RS + 16 * g;
        auto kload = [&](int ks) -> bf16x8 {
          if (!C::ROPE || ks < 16) return *(const bf16x8*)(kp + 64 * ks);
          const int c = 4 * (ks - 16) + g, r = 16 * half + t;
          return *(const bf16x8*)(sR + r * 128 + 16 * (c ^ ((r >> 1) & 7)));
        };
        constexpr int PF = NW * HB >= 8 ? 2 : 4;
        bf16x8 kb[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kb[i] = kload(i);
        // The partial product of scale tile j lives in sp[j & 1]; it is scaled
        // into acc one k-step after its last MFMA (after the first MFMA of
        // tile j + 1 is issued), so that the VALU does not wait on the MFMA
        // that just wrote it.  The additions into acc keep their order.
        f32x4 sp[2][HB], scq;
        bf16x8 qlds[NQR < NKS ? NKS - NQR : 1];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (NQR < NKS) {
            if (ks + 2 >= NQR && ks + 2 < NKS) qlds[ks + 2 - NQR] = sQr[w][ks + 2 - NQR][l];
          }
          const bf16x8 kv = kb[ks % PF];
          const int jt = ks / 4;                       // scale tile of this k-step
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            if (ks < 16) {
              const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
              sp[jt & 1][hb] = mfma16<HALF>(kv, qreg[hb][ks < NQR ? ks : 0], ks % 4 ? sp[jt & 1][hb] : z);
              if (ks % 4 == 0 && ks > 0) acc(hb) += sp[(jt - 1) & 1][hb] * scq;   // tile jt - 1
            } else {
              if (ks == 16) acc(hb) += sp[1][hb] * scq;                              // tile 3
              const bf16x8 qv = ks < NQR ? qreg[hb][ks < NQR ? ks : 0] : qlds[ks >= NQR ? ks - NQR : 0];
              acc(hb) = mfma16<HALF>(kv, qv, acc(hb));
            }
          }
          if (ks < 16 && ks % 4 == 0)   // this lane's rows' scales of tile jt (read after tile jt - 1 used them)
            scq = *(const f32x4*)(sScale + jt * T + 16 * half + 4 * g);
          if (ks + PF < NKS) kb[ks % PF] = kload(ks + PF);
        }
        if constexpr (NKS == 16) {      // no rope k-steps: tile 3 is scaled here
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) acc(hb) += sp[1][hb] * scq;
        }
      };
      if constexpr (PAIR) {
        if (wave_on) pk_half(hf, [&](int hb) -> f32x4& { return sm[hb]; });
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half)
          pk_half(half, [&](int hb) -> f32x4& { return s[hb][half]; });
      }
    } else if constexpr (PAIR) {
      // this wave's 16 rows of the tile
      if (wave_on) {
        const int r = 16 * hf + t;
        const char* kp = sK + r * RS + 16 * g;
        auto kload = [&](int ks) -> bf16x8 {
          if (!C::ROPE || ks < 16) return *(const bf16x8*)(kp + 64 * ks);
          const int c = 4 * (ks - 16) + g;
          return *(const bf16x8*)(sR + r * 128 + 16 * (c ^ ((r >> 1) & 7)));
        };
        constexpr int PF = 4;
        bf16x8 kb[PF];
#pragma unroll
        for (int i = 0; i < PF; ++i) kb[i] = kload(i);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 kv = kb[ks % PF];
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) sm[hb] = mfma16<HALF>(kv, qreg[hb][ks], sm[hb]);
          if (ks + PF < NKS) kb[ks % PF] = kload(ks + PF);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      const char* kp0 = sK + t * RS + 16 * g;
      const char* kp1 = kp0 + 16 * RS;
      auto kload = [&](int ks, bf16x8& k0v, bf16x8& k1v) {
        if (!C::ROPE || ks < 16) {
          k0v = *(const bf16x8*)(kp0 + 64 * ks);
          k1v = *(const bf16x8*)(kp1 + 64 * ks);
        } else {
          const int c = 4 * (ks - 16) + g;
          k0v = *(const bf16x8*)(sR + t * 128 + 16 * (c ^ ((t >> 1) & 7)));
          k1v = *(const bf16x8*)(sR + (16 + t) * 128 + 16 * (c ^ (((16 + t) >> 1) & 7)));
        }
      };
      constexpr int PF = (NW * HB >= 8 || W4) ? (C::ROPE ? 1 : 2) : 4;   // 2 waves/SIMD: fewer registers
      bf16x8 kb[PF][2];
#pragma unroll
      for (int i = 0; i < PF; ++i) kload(i, kb[i][0], kb[i][1]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 k0v = kb[ks % PF][0], k1v = kb[ks % PF][1];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          s[hb][0] = mfma16<HALF>(k0v, qreg[hb][ks < NQR ? ks : 0], s[hb][0]);
          s[hb][1] = mfma16<HALF>(k1v, qreg[hb][ks < NQR ? ks : 0], s[hb][1]);
        }
        if (ks + PF < NKS) kload(ks + PF, kb[ks % PF][0], kb[ks % PF][1]);
      }
    }
    if constexpr (PAIR) {
      // swap the halves' raw scores within the pair
      if (wave_on) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) sSx[w][hb][l] = sm[hb];
      }
      wait_lgkm0();
      block_barrier();                              // both halves' scores are in
      if (wave_on) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const f32x4 so = sSx[w ^ 1][hb][l];
          s[hb][0] = hf ? so : sm[hb];
          s[hb][1] = hf ? sm[hb] : so;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // lane holds head t of each block and rows {4g+i, 16+4g+i}
    bool any_grow = false;
    float alpha[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s[hb][j >> 2][j & 3] * a.scale_log2;
      if (!full) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = (nib >> j) & 1u ? x[j] : kNegInf;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) mx = fmaxf(mx, x[j]);
      mx = max4(mx);
      const bool grow = mx > m_run[hb] + kRescaleThreshold;
      alpha[hb] = grow ? __builtin_amdgcn_exp2f(m_run[hb] - mx) : 1.f;
      if (grow) m_run[hb] = mx;
      any_grow |= grow;
      const float m_use = m_run[hb] == kNegInf ? 0.f : m_run[hb];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pj = __builtin_amdgcn_exp2f(x[j] - m_use);
        psum += pj;
        if constexpr (PK) pj32[PK ? hb : 0][j] = pj;
        else pb[hb][j] = elem16<HALF>(pj);
      }
      l_run[hb] = l_run[hb] * alpha[hb] + psum;
    }
    if (__any(any_grow)) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) o[hb][mb] *= alpha[hb];
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- O^T += V^T P^T (M = 16 value columns, N = 16 heads, K = 32 rows with
  //      k = 8g+i <-> row (i < 4 ? 4g+i : 16+4g+i-4), the S^T lane layout)
  auto pv = [&](const char* sV) {
    // (wave pairs: this wave's 256 value columns)
    const char* vp = sV + (4 * g + (t >> 2)) * RS + 8 * (t & 3) + 512 * hf;
    constexpr int PV = 4;
    s16x4 vb[PV][2];
    auto vload = [&](int mb, s16x4& lo, s16x4& hi) {
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 32 * mb));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 16 * RS + 32 * mb));
    };
#pragma unroll
    for (int i = 0; i < PV; ++i) vload(i, vb[i][0], vb[i][1]);
    bf16x8 pbt[HB];                // packed: P times the rows' scales of tile mb / 8
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (PK && mb % 8 == 0) {
        const int grp = mb / 8 + (PAIR ? 2 * hf : 0);   // 128-column scale tile
        const f32x4 c0 = *(const f32x4*)(sScale + grp * T + 4 * g);
        const f32x4 c1 = *(const f32x4*)(sScale + grp * T + 16 + 4 * g);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            pbt[hb][j] = elem16<HALF>(pj32[PK ? hb : 0][j] * (j < 4 ? c0[j] : c1[j - 4]));
      }
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8 va = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(vb[mb % PV][0], vb[mb % PV][1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        o[hb][mb] = mfma16<HALF>(va, PK ? pbt[hb] : pb[hb], o[hb][mb]);
      if (mb + PV < NMB) vload(mb + PV, vb[mb % PV][0], vb[mb % PV][1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if constexpr (PKV) {
    // Packed rows with a value tensor: each raw stage holds a tile's key rows
    // and its value codes (W0, W1: the next tile streams in while this one is
    // used).  Per tile: the key codes are decoded into sK0 for the scores,
    // then the value codes overwrite its nope columns for the values (the
    // key row's scales apply to both), and only then is the stage refilled
    // with the tile two ahead.  Every wave takes the same four barriers per
    // tile (the wave pairs' score exchange adds one inside the scores).
    auto step = [&](int tt, char* sWc) {
      if (tt + 1 < nt) wait_vmcnt<PP::PER>(); else wait_vmcnt<0>();   // raw(tt) landed
      wait_lgkm0();
      block_barrier();                          // ... and the values of tile tt-1 are consumed
      decode_tile<NW, DQK, FMT, 1>(sWc, sK0, sScale, tid);
      wait_lgkm0();
      block_barrier();                          // K(tt) decoded
      if constexpr (PAIR) {
        qk_softmax(sK0, tt * T);                // (a barrier inside)
      } else if (wave_on) {
        qk_softmax(sK0, tt * T);
      }
      wait_lgkm0();
      block_barrier();                          // every wave is done with K(tt)
      decode_value<NW, DQK, FMT>(sWc, sK0, tid);
      wait_lgkm0();
      block_barrier();                          // V(tt) decoded; stage sWc is free
      if (tt + 2 < nt) issue_raw<NW, DQK, 1>(a, sRow, (tt + 2) * T, lds_addr(sWc), w, l);
      if (wave_on) pv(sK0);
    };
    if (nt > 0) issue_raw<NW, DQK, 1>(a, sRow, 0, lds_addr(sW0), w, l);
    wait_vmcnt<0>();                            // raw(0) and the Q slices
    settle(qreg);
    if constexpr (NQR < NKS) {                  // the rope slices to this wave's LDS rows
#pragma unroll
      for (int i = 0; i < NKS - NQR; ++i) sQr[w][i][l] = qrt[i];
    }
    if (nt > 1) issue_raw<NW, DQK, 1>(a, sRow, T, lds_addr(sW1), w, l);
    for (int tt = 0; tt < nt; tt += 2) {
      step(tt, sW0);
      if (tt + 1 < nt) step(tt + 1, sW1);
    }
  } else if constexpr (PK) {
    // raw stages W0..W2 (two tiles in flight); the decoded tile lives in sK0
    auto step = [&](int tt, char* sWc, char* sWn2) {
      if (tt + 1 < nt) wait_vmcnt<PP::PER>(); else wait_vmcnt<0>();   // raw(tt) landed
      wait_lgkm0();
      block_barrier();                          // ... and tile tt-1 is consumed
      if (tt + 2 < nt) issue_raw<NW, DQK>(a, sRow, (tt + 2) * T, lds_addr(sWn2), w, l);
      decode_tile<NW, DQK, FMT>(sWc, sK0, sScale, tid);
      wait_lgkm0();
      block_barrier();                          // decoded tile complete
      if constexpr (PAIR) {
        qk_softmax(sK0, tt * T);                // (a barrier inside)
        if (wave_on) pv(sK0);
      } else if (wave_on) {
        qk_softmax(sK0, tt * T);
        pv(sK0);
      }
    };
    if (nt > 0) issue_raw<NW, DQK>(a, sRow, 0, lds_addr(sW0), w, l);
    wait_vmcnt<0>();                            // raw(0) and the Q slices
    settle(qreg);
    if constexpr (NQR < NKS) {                  // the rope slices to this wave's LDS rows
#pragma unroll
      for (int i = 0; i < NKS - NQR; ++i) sQr[w][i][l] = qrt[i];
    }
    if (nt > 1) issue_raw<NW, DQK>(a, sRow, T, lds_addr(sW1), w, l);
    for (int tt = 0; tt < nt; tt += 3) {
      step(tt, sW0, sW2);
      if (tt + 1 < nt) step(tt + 1, sW1, sW0);
      if (tt + 2 < nt) step(tt + 2, sW2, sW1);
    }
  } else if constexpr (VMODE) {
    // K(t+2) streams in from the end of QK(t); V(t+1) from the start of QK(t).
    auto step = [&](int tt, char* sKc, char* sVc, char* sVn) {
      if (tt + 1 < nt) wait_vmcnt<C::NV + C::NK>(); else wait_vmcnt<C::NV>();   // K(tt) landed
      wait_lgkm0();
      block_barrier();                                    // ... and V(tt-1) reads are done
      if (tt + 1 < nt) issue_v<NW, DQK, VMODE>(a, sRow, (tt + 1) * T, lds_addr(sVn), w, l);
      if (PAIR || wave_on) qk_softmax(sKc, tt * T);   // (pairs: a barrier inside)
      if (tt + 1 < nt) wait_vmcnt<C::NK + C::NV>(); else wait_vmcnt<0>();        // V(tt) landed
      wait_lgkm0();
      block_barrier();                                    // ... and K(tt) reads are done
      if (tt + 2 < nt) issue_k<NW, DQK, VMODE>(a, sRow, (tt + 2) * T, lds_addr(sKc), w, l);
      if (wave_on) pv(sVc);
    };
    // Q lands before the first tiles go out: the compiler waits for the Q
    // loads at their first use, which is here (settle), so that no wait it
    // places inside the loop covers a gather in flight.  K(0), V(0) and K(1)
    // then go out together; every wave issues the rows whose entries it
    // resolved itself.
    settle(qreg);
    if (nt > 0) {
      issue_k<NW, DQK, VMODE>(a, sRow, 0, lds_addr(sK0), w, l);
      issue_v<NW, DQK, VMODE>(a, sRow, 0, lds_addr(sV0), w, l);
      if (nt > 1) issue_k<NW, DQK, VMODE>(a, sRow, T, lds_addr(sK1), w, l);
    }
    for (int tt = 0; tt < nt; tt += 2) {
      step(tt, sK0, sV0, sV1);
      if (tt + 1 < nt) step(tt + 1, sK1, sV1, sV0);
    }
  } else {
    // V aliases K: a ring of three K stages, two tiles in flight.  Where at
    // most four waves hold heads, waves 4..7 issue every row of the tiles
    // from K(2) on (8 rows each, as a four-wave workgroup would), so that the
    // head waves go from the barrier straight to their products; K(0) and
    // K(1) go out before the loop from the waves that resolved their rows.
    // (Not with rope: its extra addresses push that kernel's registers
    // past the limit of two waves per SIMD; not with wave pairs, whose small
    // launches were measured faster with every wave issuing a share.)
    using C4 = Pipe<4, DQK, VMODE>;
    constexpr bool LD = !TILED && !PAIR && NW == 8 && !C::ROPE;
    const bool loaders = LD && a.bpg <= 4;
    auto step = [&](int tt, char* sKc, char* sKn2) {
      if (!LD || !loaders) {
        if (tt + 1 < nt) wait_vmcnt<C::NK>(); else wait_vmcnt<0>();   // K(tt) landed
      } else if (w >= 4) {
        if (tt + 1 >= nt) wait_vmcnt<0>();
        else if (tt == 0) wait_vmcnt<C::NK>();          // K(1): this wave's own rows
        else wait_vmcnt<C4::NK>();
      } else {
        if (tt == 0 && nt > 1) wait_vmcnt<C::NK>(); else wait_vmcnt<0>();
      }
      wait_lgkm0();
      block_barrier();                                    // ... and tile tt-1 is consumed
      if (tt + 2 < nt) {
        if (!LD || !loaders) issue_k<NW, DQK, VMODE>(a, sRow, (tt + 2) * T, lds_addr(sKn2), w, l);
        else if (LD && w >= 4) issue_k<4, DQK, VMODE>(a, sRow, (tt + 2) * T, lds_addr(sKn2), w - 4, l);
      }
      if constexpr (PAIR) {
        qk_softmax(sKc, tt * T);                          // (a barrier inside)
        if (wave_on) pv(sKc);
      } else if (wave_on) {
        qk_softmax(sKc, tt * T);
        pv(sKc);
      }
    };
    // Q lands first (its first use is here), then K(0) and K(1) go out
    settle(qreg);
    if constexpr (W4) {
      // two stages, one tile in flight per workgroup (two per CU): K(tt+1)
      // goes out once every wave is done with tile tt-1
      if (nt > 0) issue_k<NW, DQK, VMODE>(a, sRow, 0, lds_addr(sK0), w, l);
      auto step2 = [&](int tt, char* sKc, char* sKn) {
        wait_vmcnt<0>();                                  // K(tt) landed
        wait_lgkm0();
        block_barrier();                                  // ... and tile tt-1 is consumed
        if (tt + 1 < nt) issue_k<NW, DQK, VMODE>(a, sRow, (tt + 1) * T, lds_addr(sKn), w, l);
        if (wave_on) {
          qk_softmax(sKc, tt * T);
          pv(sKc);
        }
      };
      for (int tt = 0; tt < nt; tt += 2) {
        step2(tt, sK0, sK1);
        if (tt + 1 < nt) step2(tt + 1, sK1, sK0);
      }
    } else {
      if (nt > 0) issue_k<NW, DQK, VMODE>(a, sRow, 0, lds_addr(sK0), w, l);
      if (nt > 1) issue_k<NW, DQK, VMODE>(a, sRow, T, lds_addr(sK1), w, l);
      for (int tt = 0; tt < nt; tt += 3) {
        step(tt, sK0, sK2);
        if (tt + 1 < nt) step(tt + 1, sK1, sK0);
        if (tt + 2 < nt) step(tt + 2, sK2, sK1);
      }
    }
  }

  if constexpr (OUTCNT) {
    // this wave's last reads of the stage buffers have returned
    wait_lgkm0();
    if (l == 0) atomicAdd(&sOut, 1);
  }
  float lt[HB], lse2[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    lt[hb] = sum4(l_run[hb]);
    lse2[hb] = lt[hb] > 0.f ? m_run[hb] + __builtin_log2f(lt[hb]) : kNegInf;   // log2 units
  }

  // final output of head block hb from accumulators o (scaled by `scale`)
  // with total weight `den` and log2-domain LSE `l2`
  auto write_final = [&](int hb, float scale, float den, float l2) {
    const int h = h0 + 16 * hb + t;
    if (h >= a.qn) return;
    const float inv = den > 0.f ? scale / den : 0.f;
    uint16_t* op = a.out + ((int64_t)orow * a.qn + h) * 512 + 4 * g + 256 * hf;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      uint2 pk;
      pk.x = (uint32_t)to16<HALF>(o[hb][mb][0] * inv) | ((uint32_t)to16<HALF>(o[hb][mb][1] * inv) << 16);
      pk.y = (uint32_t)to16<HALF>(o[hb][mb][2] * inv) | ((uint32_t)to16<HALF>(o[hb][mb][3] * inv) << 16);
      *(uint2*)(op + 16 * mb) = pk;
    }
    if (a.lse && g == 0 && hf == 0) a.lse[(int64_t)orow * a.qn + h] = den > 0.f ? l2 * kLn2 : kNegInf;
  };

  if (nsplit == 1) {
    if (!wave_on) return;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = h0 + 16 * hb + t;
      float den = lt[hb];
      if (a.has_sinks && lt[hb] > 0.f && h < a.qn)
        den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - m_run[hb]);
      write_final(hb, 1.f, lt[hb] > 0.f ? den : 0.f, lse2[hb]);
    }
    return;
  }

  // ---- split rows.  Loader-only waves hold no partial (their h0 lies in
  // another group's heads).
  if (!wave_on) return;
  static_assert(NW * 8 <= kCounterInts, "arrival counters per row: head groups (<= 8) x waves");
  const int HP = a.groups * NPW * HPW;             // heads per row, padded
  constexpr int NFR = NMB / 2;                      // 1 KB fragments per head block
  constexpr int WAVE_BYTES = HB * NFR * 64 * 16;   // one wave's partial
  // every split, head group and wave of this query row (< 2^31 bytes: at
  // most 4096 splits x 128 heads x 1 KB)
  const int64_t row_bytes = (int64_t)a.max_splits * a.groups * NW * WAVE_BYTES;
  const __amdgpu_buffer_rsrc_t rs = buf_rsrc((char*)a.ws_ob + row * row_bytes, row_bytes);
  const int wave_off = ((split * a.groups + hg) * NW + w) * WAVE_BYTES;
  // arrival counter of this (row, head group, wave) over the splits
  int32_t* ctr = a.counters + (int64_t)row * kCounterInts + hg * NW + w;

  // Owned merges (bf16 rows).  The partials of wave w's 16 heads are merged
  // in the workgroup of split w % nsplit, their owner, when the launch lets it
  // wait (every workgroup of the launch is resident at once, so the other
  // splits make progress meanwhile):
  //   - the owning wave writes its own partial to an LDS slot (the bits a
  //     store would have written), waits until the other nsplit - 1 splits
  //     have counted in, computes the split weights, lands their partials in
  //     LDS slots with one round of DMA and raises a flag;
  //   - every head-holding wave of the workgroup then merges a share of the
  //     owned heads' 16 fragments from LDS (the merge runs on all SIMDs).
  // The wait is bounded: past a.merge_wait_ticks the owner stores its partial
  // and counts in like the others, and the last to arrive merges (below),
  // which gives the same bits.  Non-owning waves store and count in, then
  // help.  After the last split's loop the critical path is one store, one
  // count, one load round and a merge spread over the workgroup.
  constexpr int OSLOT = 8;                          // LDS slots of 16 KB
  const int n_on = min(a.bpg, (a.qn - hg * a.bpg * HPW + HPW - 1) / HPW);   // waves with heads
  const int n_own = split < n_on ? (n_on - 1 - split) / nsplit + 1 : 0;    // owned waves here
  // (only where every wave of the workgroup holds heads, so the shared
  // merge runs on all SIMDs: with fewer head waves the last split to
  // arrive merges sooner, measured)
  const bool own_mode = !PK && !TILED && !PAIR && !W4 && a.merge_wait_ticks > 0 && nsplit <= kMaxOwnerSplits &&
                        n_on == NW && n_own > 0 && n_own * nsplit <= OSLOT;
  auto slot_addr = [&](int q) -> uint32_t {          // slot q: two per stage buffer
    const int b = q >> 1;
    const uint32_t base = VMODE ? (b == 0 ? lds_addr(sK0) : b == 1 ? lds_addr(sK1)
                                   : b == 2 ? lds_addr(sV0) : lds_addr(sV1))
                                : (b == 0 ? lds_addr(sK0) : b == 1 ? lds_addr(sK1)
                                   : b == 2 ? lds_addr(sK2) : lds_addr(sM));
    return __builtin_amdgcn_readfirstlane(base + (q & 1) * 16384);
  };
  // the last-arriver merge of this wave's heads (every split's partial from
  // memory, this split's own included)
  auto merge_last = [&](auto ms_c, auto jb_c, auto one_c) __attribute__((always_inline)) {
    // merge from the stored partials (this split's own included).  Round r
    // loads column blocks [JB*(r / ns4), +JB) of MS splits (MS*JB loads of 16
    // bytes per lane in flight: 16, or 32 where one wave per SIMD or a wave
    // pair's half-width partials leave the registers); the first round
    // travels together with the loads of the LSEs, which give the max and
    // the normaliser in one pass.  MS only groups the loads: the splits are
    // added in the same order whatever its value.  ONE: MS >= nsplit, so a
    // round holds every split of its columns and each column block is
    // finished (and its accumulators free) before the next.
    constexpr int MS = decltype(ms_c)::value, JB = decltype(jb_c)::value, NJ = NFR / JB;
    constexpr bool ONE = decltype(one_c)::value;
    const int ns4 = (nsplit + MS - 1) / MS;               // split chunks per column round
    const int R = NJ * ns4;                               // load rounds
    const int split_bytes = a.groups * NW * WAVE_BYTES;
    // Staged output: rounds write their results to LDS and the wave stores all
    // 16 heads at the end.  Vector-memory stores count in vmcnt with the loads
    // and complete in order, so stores between rounds would make each next
    // round's wait include them.  Every wave of the workgroup counts itself
    // out right after its main loop, so this wait ends.  Not while owning
    // waves of this workgroup use the same buffers (owned merges): this
    // merge is then the rare fallback after a time-out and stores directly.
    char* stg = nullptr;
    const bool stage = STAGE && !own_mode;
    if (stage) {
      stg = (w < 2 ? sK0 : w < 4 ? sK1 : w < 6 ? sV0 : sV1) + (w & 1) * 16 * kStgRow;
      while (*(volatile int32_t*)&sOut < NW) __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = h0 + 16 * hb + t;
      const float* lp = a.ws_lse + (int64_t)row * a.max_splits * HP + h;
      const int off0 = (hg * NW + w) * WAVE_BYTES + ((hb * NFR) * 64 + l) * 16;  // split 0
      u32x4 v[MS][JB];
      float wl[MS];
      auto issue = [&](int r) {
        const int jr = r / ns4, s0 = (r - jr * ns4) * MS;
#pragma unroll
        for (int q = 0; q < MS; ++q) {
          const int s2 = min(s0 + q, nsplit - 1);
          wl[q] = ld_agent(lp + (int64_t)s2 * HP);
#pragma unroll
          for (int j = 0; j < JB; ++j)
            v[q][j] = __builtin_amdgcn_raw_buffer_load_b128(
                rs, off0 + s2 * split_bytes + (jr * JB + j) * 64 * 16, 0, kSc1);
        }
      };
      issue(0);
      // max and normaliser over every split's LSE (the first chunk is wl)
      float M = kNegInf, tot = 0.f;
#pragma unroll
      for (int q = 0; q < MS; ++q)
        if (q < nsplit) M = fmaxf(M, wl[q]);
#pragma unroll 1
      for (int s0 = MS; s0 < nsplit; s0 += MS) {
#pragma unroll
        for (int q = 0; q < MS; ++q)
          if (s0 + q < nsplit) M = fmaxf(M, ld_agent(lp + (int64_t)(s0 + q) * HP));
      }
      const float Mu = M == kNegInf ? 0.f : M;
#pragma unroll
      for (int q = 0; q < MS; ++q)
        if (q < nsplit) tot += __builtin_amdgcn_exp2f(wl[q] - Mu);
#pragma unroll 1
      for (int s0 = MS; s0 < nsplit; s0 += MS) {
#pragma unroll
        for (int q = 0; q < MS; ++q)
          if (s0 + q < nsplit) tot += __builtin_amdgcn_exp2f(ld_agent(lp + (int64_t)(s0 + q) * HP) - Mu);
      }
      float den = tot;
      if (a.has_sinks && h < a.qn && tot > 0.f)
        den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - Mu);
      const float inv = tot > 0.f ? 1.f / den : 0.f;
      const bool on = h < a.qn;
      uint16_t* op = a.out + ((int64_t)row * a.qn + (on ? h : 0)) * 512 + 4 * g + 256 * hf;
      // column block jj of this head from the merged accumulators c
      auto put = [&](int jj, const float* c) __attribute__((always_inline)) {
        uint2 p0, p1;
        p0.x = (uint32_t)to16<HALF>(c[0] * inv) | ((uint32_t)to16<HALF>(c[1] * inv) << 16);
        p0.y = (uint32_t)to16<HALF>(c[2] * inv) | ((uint32_t)to16<HALF>(c[3] * inv) << 16);
        p1.x = (uint32_t)to16<HALF>(c[4] * inv) | ((uint32_t)to16<HALF>(c[5] * inv) << 16);
        p1.y = (uint32_t)to16<HALF>(c[6] * inv) | ((uint32_t)to16<HALF>(c[7] * inv) << 16);
        if (stage) {
          char* sp = stg + (16 * hb + t) * kStgRow + 2 * (32 * jj + 4 * g);
          *(uint2*)sp = p0;
          *(uint2*)(sp + 32) = p1;
        } else {
          *(uint2*)(op + 16 * (2 * jj)) = p0;
          *(uint2*)(op + 16 * (2 * jj + 1)) = p1;
        }
      };
      float acc[JB][8];                                    // (unused where ONE)
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
#pragma unroll 1
      for (int r = 0; r < R; ++r) {
        if (r > 0) issue(r);
        const int jr = r / ns4, s0 = (r - jr * ns4) * MS;
        if constexpr (ONE) {
          float ws[MS];
#pragma unroll
          for (int q = 0; q < MS; ++q) ws[q] = q < nsplit ? __builtin_amdgcn_exp2f(wl[q] - Mu) : 0.f;
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            float c[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < MS; ++q) {
              const uint32_t u[4] = {v[q][j].x, v[q][j].y, v[q][j].z, v[q][j].w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                c[2 * e] = __builtin_fmaf(ws[q], lo16<HALF>(u[e]), c[2 * e]);
                c[2 * e + 1] = __builtin_fmaf(ws[q], hi16<HALF>(u[e]), c[2 * e + 1]);
              }
            }
            if (stage || on) put(jr * JB + j, c);
          }
          continue;
        }
#pragma unroll
        for (int q = 0; q < MS; ++q) {
          const float ws = s0 + q < nsplit ? __builtin_amdgcn_exp2f(wl[q] - Mu) : 0.f;
#pragma unroll
          for (int j = 0; j < JB; ++j) {
            const uint32_t u[4] = {v[q][j].x, v[q][j].y, v[q][j].z, v[q][j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[j][2 * e] = __builtin_fmaf(ws, lo16<HALF>(u[e]), acc[j][2 * e]);
              acc[j][2 * e + 1] = __builtin_fmaf(ws, hi16<HALF>(u[e]), acc[j][2 * e + 1]);
            }
          }
        }
        if (s0 + MS < nsplit) continue;                    // more splits for these columns
        if (stage || on) {
#pragma unroll
          for (int j = 0; j < JB; ++j) put(jr * JB + j, acc[j]);
        }
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
      }
      if (on && a.lse && g == 0 && hf == 0)
        a.lse[(int64_t)row * a.qn + h] = tot > 0.f ? (Mu + __builtin_log2f(tot)) * kLn2 : kNegInf;
    }
    if (stage) {
      // the staged heads (1 KB each, contiguous in the output) go out 16 bytes
      // a lane; heads past q_n are not written
      wait_lgkm0();
      // (heads past q_n are read and not written, so that every row read
      // is one unconditional instruction)
#pragma unroll
      for (int i = 0; i < 16 * HB; ++i) {
        const uint4 r = *(const uint4*)(stg + i * kStgRow + 16 * l);
        if (h0 + i < a.qn) *(uint4*)(a.out + ((int64_t)row * a.qn + h0 + i) * 512 + 8 * l) = r;
      }
    }
  };

  bool owned_here = false;                          // this wave's heads are merged here
  if constexpr (!PK && !PAIR) {
    static_assert(HB == 1, "owned merge: one 16-head block per wave");
    if (own_mode && w % nsplit == split) {
      const int ow = w / nsplit;
      // the stage buffers are free once every wave has counted out
      while (*(volatile int32_t*)&sOut < NW) __builtin_amdgcn_s_sleep(1);
      {
        const float io = lt[0] > 0.f ? 1.f / lt[0] : 0.f;
        const uint32_t dst = slot_addr(ow * nsplit + split) + 16 * l;
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          v4u pk;
          pk.x = (uint32_t)to16<HALF>(o[0][2 * j][0] * io) | ((uint32_t)to16<HALF>(o[0][2 * j][1] * io) << 16);
          pk.y = (uint32_t)to16<HALF>(o[0][2 * j][2] * io) | ((uint32_t)to16<HALF>(o[0][2 * j][3] * io) << 16);
          pk.z = (uint32_t)to16<HALF>(o[0][2 * j + 1][0] * io) |
                 ((uint32_t)to16<HALF>(o[0][2 * j + 1][1] * io) << 16);
          pk.w = (uint32_t)to16<HALF>(o[0][2 * j + 1][2] * io) |
                 ((uint32_t)to16<HALF>(o[0][2 * j + 1][3] * io) << 16);
          *(__attribute__((address_space(3))) v4u*)(uintptr_t)(dst + j * 1024) = pk;
        }
      }
      int seen = 0;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        seen = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (seen >= nsplit - 1) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > (uint64_t)a.merge_wait_ticks) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (__builtin_amdgcn_readfirstlane(seen) >= nsplit - 1) {
        owned_here = true;
        if (l == 0)                                   // ready for the next call
          __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int h = h0 + t;
        const float* lp0 = a.ws_lse + (int64_t)row * a.max_splits * HP + h;
        float wl[kMaxOwnerSplits];
#pragma unroll
        for (int s2 = 0; s2 < kMaxOwnerSplits; ++s2)
          wl[s2] = s2 >= nsplit ? kNegInf : s2 == split ? lse2[0] : ld_agent(lp0 + (int64_t)s2 * HP);
        const char* part0 = (const char*)a.ws_ob + row * row_bytes +
                            (int64_t)(hg * NW + w) * WAVE_BYTES + 16 * l;   // split 0
        const int split_bytes = a.groups * NW * WAVE_BYTES;
#pragma unroll 1
        for (int sp = 0; sp < nsplit; ++sp) {
          if (sp == split) continue;
          const uint32_t dst = slot_addr(ow * nsplit + sp);
          wait_vmcnt<63 - 16>();                      // the 6-bit counter never overflows
#pragma unroll
          for (int j = 0; j < 16; ++j)
            dma16_sc1(part0 + (int64_t)sp * split_bytes + j * 1024, dst + j * 1024);
        }
        float M = kNegInf;
#pragma unroll
        for (int s2 = 0; s2 < kMaxOwnerSplits; ++s2) M = fmaxf(M, wl[s2]);
        const float Mu = M == kNegInf ? 0.f : M;
        float tot = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kMaxOwnerSplits; ++s2)
          if (s2 < nsplit) tot += __builtin_amdgcn_exp2f(wl[s2] - Mu);
        float den = tot;
        if (a.has_sinks && h < a.qn && tot > 0.f)
          den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - Mu);
        if (g == 0) {
#pragma unroll
          for (int s2 = 0; s2 < kMaxOwnerSplits; ++s2)
            if (s2 < nsplit) sWs[ow][s2][t] = __builtin_amdgcn_exp2f(wl[s2] - Mu);
          sInv[ow][t] = tot > 0.f ? 1.f / den : 0.f;
          if (h < a.qn && a.lse)
            a.lse[(int64_t)row * a.qn + h] = tot > 0.f ? (Mu + __builtin_log2f(tot)) * kLn2 : kNegInf;
        }
        wait_vmcnt<0>();                              // the partials have landed
        wait_lgkm0();
        if (l == 0) *(volatile int32_t*)&sReady[ow] = 1;
      } else {
        // timed out: hand these heads to the last split to arrive
        if (l == 0) *(volatile int32_t*)&sReady[ow] = 2;
      }
    }
  }

  // this split's partial (bf16, in the lanes' fragment order: instruction j
  // of a wave writes 1 KB contiguously) and its LSEs
  auto store_partial = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const float inv = lt[hb] > 0.f ? 1.f / lt[hb] : 0.f;
#pragma unroll
      for (int j = 0; j < NFR; ++j) {
        uint4 pk;
        pk.x = (uint32_t)to16<HALF>(o[hb][2 * j][0] * inv) | ((uint32_t)to16<HALF>(o[hb][2 * j][1] * inv) << 16);
        pk.y = (uint32_t)to16<HALF>(o[hb][2 * j][2] * inv) | ((uint32_t)to16<HALF>(o[hb][2 * j][3] * inv) << 16);
        pk.z = (uint32_t)to16<HALF>(o[hb][2 * j + 1][0] * inv) |
               ((uint32_t)to16<HALF>(o[hb][2 * j + 1][1] * inv) << 16);
        pk.w = (uint32_t)to16<HALF>(o[hb][2 * j + 1][2] * inv) |
               ((uint32_t)to16<HALF>(o[hb][2 * j + 1][3] * inv) << 16);
        const u32x4 d = {pk.x, pk.y, pk.z, pk.w};
        __builtin_amdgcn_raw_buffer_store_b128(d, rs, wave_off + ((hb * NFR + j) * 64 + l) * 16, 0, kSc1);
      }
      if (g == 0)
        st_agent(a.ws_lse + ((int64_t)row * a.max_splits + split) * HP + h0 + 16 * hb + t, lse2[hb]);
    }
  };

  // Rows of two splits (no owned merge): arrival is counted before the
  // partial is stored.  The first split to arrive stores its partial and
  // then counts it stored (the counter's upper half); the second waits for
  // that count and merges the stored partial with its own, still in
  // registers, so it neither stores its own partial nor loads it back.  Its
  // own partial's bits are formed as the store forms them and the two are
  // added in split order, so the result is the bits of the merge below.
  // (Not in the four-wave kernel, whose rows take one split, nor with wave
  // pairs, whose small launches measured slower with it.)
  auto two_splits = [&]() __attribute__((always_inline)) {
    int old = 0;
    if (l == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((__builtin_amdgcn_readfirstlane(old) & 0xffff) == 0) {
      store_partial();
      drain_vmem();                                 // stored before it is counted
      if (l == 0) __hip_atomic_fetch_add(ctr, 1 << 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    // the other split has arrived and is storing (it waits for nothing)
    for (;;) {
      const int c = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__builtin_amdgcn_readfirstlane(c) >> 16) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (l == 0)                                     // ready for the next call
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int other = 1 - split;
    const int split_bytes = a.groups * NW * WAVE_BYTES;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = h0 + 16 * hb + t;
      const float* lp = a.ws_lse + (int64_t)row * a.max_splits * HP + h;
      const int off = other * split_bytes + (hg * NW + w) * WAVE_BYTES + ((hb * NFR) * 64 + l) * 16;
      const float lx = ld_agent(lp + (int64_t)other * HP);
      u32x4 v[NFR];
#pragma unroll
      for (int j = 0; j < NFR; ++j)
        v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + j * 64 * 16, 0, kSc1);
      const float l0 = split == 0 ? lse2[hb] : lx, l1 = split == 0 ? lx : lse2[hb];
      const float M = fmaxf(fmaxf(kNegInf, l0), l1);
      const float Mu = M == kNegInf ? 0.f : M;
      const float e0 = __builtin_amdgcn_exp2f(l0 - Mu), e1 = __builtin_amdgcn_exp2f(l1 - Mu);
      float tot = 0.f;
      tot += e0;
      tot += e1;
      float den = tot;
      if (a.has_sinks && h < a.qn && tot > 0.f)
        den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - Mu);
      const float inv = tot > 0.f ? 1.f / den : 0.f;
      const float io = lt[hb] > 0.f ? 1.f / lt[hb] : 0.f;   // as the store scales it
      const bool on = h < a.qn;
      uint16_t* op = a.out + ((int64_t)row * a.qn + (on ? h : 0)) * 512 + 4 * g + 256 * hf;
#pragma unroll
      for (int j = 0; j < NFR; ++j) {
        uint32_t own[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4& oc = o[hb][2 * j + (e >> 1)];
          own[e] = (uint32_t)to16<HALF>(oc[2 * (e & 1)] * io) |
                   ((uint32_t)to16<HALF>(oc[2 * (e & 1) + 1] * io) << 16);
        }
        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        float c[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x0 = split == 0 ? own[e] : u[e];
          c[2 * e] = __builtin_fmaf(e0, lo16<HALF>(x0), c[2 * e]);
          c[2 * e + 1] = __builtin_fmaf(e0, hi16<HALF>(x0), c[2 * e + 1]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x1 = split == 0 ? u[e] : own[e];
          c[2 * e] = __builtin_fmaf(e1, lo16<HALF>(x1), c[2 * e]);
          c[2 * e + 1] = __builtin_fmaf(e1, hi16<HALF>(x1), c[2 * e + 1]);
        }
        if (on) {
          uint2 p0, p1;
          p0.x = (uint32_t)to16<HALF>(c[0] * inv) | ((uint32_t)to16<HALF>(c[1] * inv) << 16);
          p0.y = (uint32_t)to16<HALF>(c[2] * inv) | ((uint32_t)to16<HALF>(c[3] * inv) << 16);
          p1.x = (uint32_t)to16<HALF>(c[4] * inv) | ((uint32_t)to16<HALF>(c[5] * inv) << 16);
          p1.y = (uint32_t)to16<HALF>(c[6] * inv) | ((uint32_t)to16<HALF>(c[7] * inv) << 16);
          *(uint2*)(op + 16 * (2 * j)) = p0;
          *(uint2*)(op + 16 * (2 * j + 1)) = p1;
        }
      }
      if (on && a.lse && g == 0 && hf == 0)
        a.lse[(int64_t)row * a.qn + h] = tot > 0.f ? (Mu + __builtin_log2f(tot)) * kLn2 : kNegInf;
    }
  };

  bool two = false;
  if constexpr (!W4 && !PAIR) two = nsplit == 2 && !own_mode;
  if (two) {
    two_splits();
  } else if (!owned_here) {
    // store this split's partial, count in; the last to arrive merges every
    // split's partial of these heads
    store_partial();
    drain_vmem();                                   // this wave's partial is stored
    // Arrival is counted per (row, head group, wave): the last of the
    // splits' waves for these 16 heads merges them (unless their owner
    // does), so the merges of one row spread over the splits' workgroups
    // and no workgroup barrier is needed.
    int last = 0;
    if (l == 0)
      last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
    if (__builtin_amdgcn_readfirstlane(last)) {
      if (l == 0)                                   // ready for the next call
        __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // splits per round: two where the row has at most two (every column
      // block in one or two rounds, no spare slot), else four; eight where
      // a wave pair's row has more than four (32 loads per lane of its
      // half-width partials: more registers are free than where a wave
      // holds all 512 columns).  Spare slots load the last split again and
      // weigh it zero.
      if constexpr (PAIR) {
        if (nsplit <= 2) merge_last(IntC<2>{}, IntC<8>{}, IntC<1>{});
        else if (nsplit <= 4) merge_last(IntC<4>{}, IntC<4>{}, IntC<0>{});
        else merge_last(IntC<8>{}, IntC<4>{}, IntC<0>{});
      } else if constexpr (NW <= 4 && !W4) {
        merge_last(IntC<8>{}, IntC<4>{}, IntC<0>{});
      } else if constexpr (W4) {
        // (prefill rows, one split: the kernel stays as small as it was,
        // measured faster)
        merge_last(IntC<4>{}, IntC<4>{}, IntC<0>{});
      } else {
        if (nsplit <= 2) merge_last(IntC<2>{}, IntC<8>{}, IntC<1>{});
        else merge_last(IntC<4>{}, IntC<4>{}, IntC<0>{});
      }
    }
  }

  if constexpr (!PK && !PAIR) {
    if (own_mode) {
      // share of the owned heads' merge: fragment j (head t, value columns
      // [32 j, 32 j + 32)) of owned wave ow goes to head-holding wave
      // j mod n_on; weights and normalisers come from the owner
#pragma unroll 1
      for (int ow = 0; ow < n_own; ++ow) {
        int st;
        while ((st = *(volatile int32_t*)&sReady[ow]) == 0) __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_readfirstlane(st) != 1) continue;   // handed off
        const int wo = split + ow * nsplit;                      // the owned wave
        const int ho = (hg * a.bpg + wo) * HPW + t;
        const float inv = sInv[ow][t];
        uint16_t* op = a.out + ((int64_t)row * a.qn + (ho < a.qn ? ho : 0)) * 512 + 4 * g;
#pragma unroll 1
        for (int j = w; j < 16; j += n_on) {
          float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
          for (int sp = 0; sp < nsplit; ++sp) {
            const float ws = sWs[ow][sp][t];
            const uint4 v = lds_ld16(slot_addr(ow * nsplit + sp) + j * 1024 + 16 * l);
            const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[2 * e] = __builtin_fmaf(ws, lo16<HALF>(u[e]), acc[2 * e]);
              acc[2 * e + 1] = __builtin_fmaf(ws, hi16<HALF>(u[e]), acc[2 * e + 1]);
            }
          }
          if (ho < a.qn) {
            uint2 p0, p1;
            p0.x = (uint32_t)to16<HALF>(acc[0] * inv) | ((uint32_t)to16<HALF>(acc[1] * inv) << 16);
            p0.y = (uint32_t)to16<HALF>(acc[2] * inv) | ((uint32_t)to16<HALF>(acc[3] * inv) << 16);
            p1.x = (uint32_t)to16<HALF>(acc[4] * inv) | ((uint32_t)to16<HALF>(acc[5] * inv) << 16);
            p1.y = (uint32_t)to16<HALF>(acc[6] * inv) | ((uint32_t)to16<HALF>(acc[7] * inv) << 16);
            *(uint2*)(op + 16 * (2 * j)) = p0;
            *(uint2*)(op + 16 * (2 * j + 1)) = p1;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge of split partials
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x, h = blockIdx.y;
  const int np = a.n_parts;
  const float* lp = a.part_lse + row * a.lse_row_stride + h;
  // Weights are taken relative to the largest part LSE only, so the sum of
  // the parts' weights is >= 1 whenever a part is non-empty and the merged
  // LSE stays finite however far the sink lies above it; the sink enters the
  // denominator alone (a sink far above every part drives O to 0).
  float m = kNegInf;
  for (int k = 0; k < np; ++k) m = fmaxf(m, lp[k * a.lse_part_stride]);
  const float ref = m == kNegInf ? 0.f : m;
  float tot = 0.f;
  for (int k = 0; k < np; ++k) tot += expf(lp[k * a.lse_part_stride] - ref);
  const float den = tot + (a.sinks ? expf(a.sinks[h] - ref) : 0.f);
  const float inv = tot > 0.f ? 1.f / den : 0.f;
  const float* op = a.part_o + row * a.o_row_stride + (int64_t)h * a.dv;
  uint16_t* out = a.out + ((int64_t)row * a.heads + h) * a.dv;
  for (int c = threadIdx.x * 4; c < a.dv; c += blockDim.x * 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < np; ++k) {
      const float wk = expf(lp[k * a.lse_part_stride] - ref);
      const float4 v = *(const float4*)(op + k * a.o_part_stride + c);
      acc[0] += wk * v.x; acc[1] += wk * v.y; acc[2] += wk * v.z; acc[3] += wk * v.w;
    }
    uint2 pk;
    pk.x = (uint32_t)f2bf(acc[0] * inv) | ((uint32_t)f2bf(acc[1] * inv) << 16);
    pk.y = (uint32_t)f2bf(acc[2] * inv) | ((uint32_t)f2bf(acc[3] * inv) << 16);
    *(uint2*)(out + c) = pk;
  }
  if (a.lse_out && threadIdx.x == 0)
    a.lse_out[(int64_t)row * a.heads + h] = tot > 0.f ? logf(tot) + ref : kNegInf;
}

// ---------------------------------------------------------------------------
// debug: resolved rows in canonical order
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void resolve_kernel(FwdArgs a) {
  __shared__ int32_t sFlag[256];
  __shared__ int32_t sBase;
  const int row = blockIdx.x;
  if (!plan_matches(a, *(const int4*)a.meta)) {
    if (threadIdx.x == 0) {
      a.dbg_counts[row] = -1;
      if (a.status) atomicOr(a.status, SFMLA_STATUS_METADATA_MISMATCH);
    }
    return;
  }
  const int32_t* rec = a.meta + kHeaderInts + (int64_t)row * kRecInts;
  const int n = rec[R_NTOTAL];
  int64_t* dst = a.dbg_rows + (int64_t)row * a.dbg_max_rows;
  for (int k = threadIdx.x; k < a.dbg_max_rows; k += blockDim.x) dst[k] = -1;
  if (threadIdx.x == 0) sBase = 0;
  __syncthreads();
  for (int k0 = 0; k0 < n; k0 += 256) {
    const int k = k0 + threadIdx.x;
    int side = 0;
    int64_t phys = -1;
    if (k < n) phys = resolve_pos(a, rec, row, k, &side);
    sFlag[threadIdx.x] = phys >= 0;
    __syncthreads();
    if (threadIdx.x == 0) {          // exclusive scan (debug path: serial is fine)
      int acc = sBase;
      for (int i = 0; i < 256; ++i) { const int f = sFlag[i]; sFlag[i] = acc; acc += f; }
      sBase = acc;
    }
    __syncthreads();
    if (phys >= 0) {
      const int pos = sFlag[threadIdx.x];
      if (pos < a.dbg_max_rows) dst[pos] = phys | ((int64_t)side << 62);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) a.dbg_counts[row] = sBase;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

constexpr int kMaxDevices = 64;

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int threads = kPlanThreads;
  const int blocks = (a.p.q_t + threads - 1) / threads;
  hipLaunchKernelGGL(plan_kernel, dim3(blocks > 0 ? blocks : 1), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// Workgroups of this kernel the current device holds at once (cached per
// device and kernel; 0 if the runtime cannot tell).
// 16-head blocks each wave holds
template <int NW, int FMT>
constexpr int kHeadBlocks = 1;

template <int NW, int DQK, int VMODE, int FMT>
static int64_t resident_capacity() {
  static std::atomic<int64_t> cap[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int64_t c = cap[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    // the runtime's occupancy, bounded by what the LDS holds (the larger
    // of the two was seen to over-count for workgroups of ~147 KB of LDS)
    const void* fn = reinterpret_cast<const void*>(&fwd_kernel<NW, kHeadBlocks<NW, FMT>, DQK, VMODE, FMT>);
    int per_cu = 0, cus = 0, lds_cu = 0;
    hipFuncAttributes fa;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, NW * 64, 0) != hipSuccess ||
        hipFuncGetAttributes(&fa, fn) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (fa.sharedSizeBytes > 0) per_cu = std::min<int>(per_cu, lds_cu / (int)fa.sharedSizeBytes);
    c = (int64_t)std::max(per_cu, 0) * cus;
    cap[dev].store(c > 0 ? c : -1, std::memory_order_relaxed);
  }
  return c > 0 ? c : 0;
}

template <int NW, int DQK, int VMODE, int FMT>
static hipError_t launch_fwd_t(const FwdArgs& a, int groups, int merge_wait_us, hipStream_t s,
                               hipEvent_t t0, hipEvent_t t1) {
  FwdArgs b = a;
  b.groups = groups;
  if (b.bpg < 1 || b.bpg > NW) return hipErrorInvalidConfiguration;
  const int64_t blocks = (int64_t)(a.q_t + 7) / 8 * 8 * a.max_splits * groups;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  // an owning wave may wait for the other splits of its row only when every
  // workgroup of the launch is resident at once (s_memrealtime: 100 MHz)
  b.merge_wait_ticks = 0;
  if (merge_wait_us > 0 && blocks <= resident_capacity<NW, DQK, VMODE, FMT>())
    b.merge_wait_ticks = merge_wait_us * 100;
  if (t0 || t1)   // events that the dispatch itself stamps at the kernel's start and end
    hipExtLaunchKernelGGL((fwd_kernel<NW, kHeadBlocks<NW, FMT>, DQK, VMODE, FMT>), dim3((unsigned)blocks),
                          dim3(NW * 64), 0, s, t0, t1, 0, b);
  else
    hipLaunchKernelGGL((fwd_kernel<NW, kHeadBlocks<NW, FMT>, DQK, VMODE, FMT>), dim3((unsigned)blocks),
                       dim3(NW * 64), 0, s, b);
  return hipGetLastError();
}

// Wave pairs (16-bit rows): eight waves, four pairs of 16 heads each
template <int DQK, int VMODE, int FMT>
static hipError_t launch_pair_t(const FwdArgs& a, int groups, hipStream_t s, hipEvent_t t0,
                                hipEvent_t t1) {
  FwdArgs b = a;
  b.groups = groups;
  if (b.bpg < 1 || b.bpg > 4) return hipErrorInvalidConfiguration;
  const int64_t blocks = (int64_t)(a.q_t + 7) / 8 * 8 * a.max_splits * groups;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  b.merge_wait_ticks = 0;                           // no owned merges
  if (t0 || t1)
    hipExtLaunchKernelGGL((fwd_kernel<8, 1, DQK, VMODE, FMT, false, true>), dim3((unsigned)blocks),
                          dim3(512), 0, s, t0, t1, 0, b);
  else
    hipLaunchKernelGGL((fwd_kernel<8, 1, DQK, VMODE, FMT, false, true>), dim3((unsigned)blocks),
                       dim3(512), 0, s, b);
  return hipGetLastError();
}

// Packed rows: eight waves per workgroup (two per SIMD; the gather and the
// decode of a tile spread over all of them)
template <int FMT>
static hipError_t launch_packed(const FwdArgs& a, int nw, int dqk, int vmode, int groups, int mw,
                                hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (nw != 8) return hipErrorInvalidConfiguration;
  if (vmode)   // value codes from their own tensor
    return dqk == 512 ? launch_fwd_t<8, 512, 1, FMT>(a, groups, mw, s, t0, t1)
                      : launch_fwd_t<8, 576, 1, FMT>(a, groups, mw, s, t0, t1);
  return dqk == 512 ? launch_fwd_t<8, 512, 0, FMT>(a, groups, mw, s, t0, t1)
                    : launch_fwd_t<8, 576, 0, FMT>(a, groups, mw, s, t0, t1);
}

hipError_t launch_forward(const FwdArgs& a, int nw, bool pair, int dqk, int vmode, int fmt,
                          int groups, int mw, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  if (pair) {
    if (nw != 8) return hipErrorInvalidConfiguration;
    if (fmt == SFMLA_KV_BF16) {
      if (dqk == 512) return vmode ? launch_pair_t<512, 1, 0>(a, groups, s, t0, t1)
                                   : launch_pair_t<512, 0, 0>(a, groups, s, t0, t1);
      return vmode ? launch_pair_t<576, 1, 0>(a, groups, s, t0, t1)
                   : launch_pair_t<576, 0, 0>(a, groups, s, t0, t1);
    }
    if (fmt == SFMLA_KV_FP16) {
      if (dqk == 512) return vmode ? launch_pair_t<512, 1, SFMLA_KV_FP16>(a, groups, s, t0, t1)
                                   : launch_pair_t<512, 0, SFMLA_KV_FP16>(a, groups, s, t0, t1);
      return vmode ? launch_pair_t<576, 1, SFMLA_KV_FP16>(a, groups, s, t0, t1)
                   : launch_pair_t<576, 0, SFMLA_KV_FP16>(a, groups, s, t0, t1);
    }
    if (fmt == SFMLA_KV_INT8_PACKED) {
      if (vmode)
        return dqk == 512 ? launch_pair_t<512, 1, SFMLA_KV_INT8_PACKED>(a, groups, s, t0, t1)
                          : launch_pair_t<576, 1, SFMLA_KV_INT8_PACKED>(a, groups, s, t0, t1);
      return dqk == 512 ? launch_pair_t<512, 0, SFMLA_KV_INT8_PACKED>(a, groups, s, t0, t1)
                        : launch_pair_t<576, 0, SFMLA_KV_INT8_PACKED>(a, groups, s, t0, t1);
    }
    if (fmt == SFMLA_KV_FP8_E4M3_PACKED) {
      if (vmode)
        return dqk == 512 ? launch_pair_t<512, 1, SFMLA_KV_FP8_E4M3_PACKED>(a, groups, s, t0, t1)
                          : launch_pair_t<576, 1, SFMLA_KV_FP8_E4M3_PACKED>(a, groups, s, t0, t1);
      return dqk == 512 ? launch_pair_t<512, 0, SFMLA_KV_FP8_E4M3_PACKED>(a, groups, s, t0, t1)
                        : launch_pair_t<576, 0, SFMLA_KV_FP8_E4M3_PACKED>(a, groups, s, t0, t1);
    }
    return hipErrorInvalidConfiguration;
  }
  switch (fmt) {
    case SFMLA_KV_INT8_PACKED:
      return launch_packed<SFMLA_KV_INT8_PACKED>(a, nw, dqk, vmode, groups, mw, s, t0, t1);
    case SFMLA_KV_FP8_E4M3_PACKED:
      return launch_packed<SFMLA_KV_FP8_E4M3_PACKED>(a, nw, dqk, vmode, groups, mw, s, t0, t1);
    case SFMLA_KV_FP16:
      if (nw == 4)   // d_qk 512, V = K nope: two workgroups per CU
        return dqk == 512 && !vmode ? launch_fwd_t<4, 512, 0, SFMLA_KV_FP16>(a, groups, mw, s, t0, t1)
                                    : hipErrorInvalidConfiguration;
      if (nw != 8) return hipErrorInvalidConfiguration;
      if (dqk == 512) return vmode ? launch_fwd_t<8, 512, 1, SFMLA_KV_FP16>(a, groups, mw, s, t0, t1)
                                   : launch_fwd_t<8, 512, 0, SFMLA_KV_FP16>(a, groups, mw, s, t0, t1);
      return vmode ? launch_fwd_t<8, 576, 1, SFMLA_KV_FP16>(a, groups, mw, s, t0, t1)
                   : launch_fwd_t<8, 576, 0, SFMLA_KV_FP16>(a, groups, mw, s, t0, t1);
    default:
      if (nw == 4)
        return dqk == 512 && !vmode ? launch_fwd_t<4, 512, 0, 0>(a, groups, mw, s, t0, t1)
                                    : hipErrorInvalidConfiguration;
      if (nw != 8) return hipErrorInvalidConfiguration;
      if (dqk == 512) return vmode ? launch_fwd_t<8, 512, 1, 0>(a, groups, mw, s, t0, t1)
                                   : launch_fwd_t<8, 512, 0, 0>(a, groups, mw, s, t0, t1);
      return vmode ? launch_fwd_t<8, 576, 1, 0>(a, groups, mw, s, t0, t1)
                   : launch_fwd_t<8, 576, 0, 0>(a, groups, mw, s, t0, t1);
  }
}

template <int DQK, int VMODE, int FMT>
static hipError_t launch_tiled_t(const FwdArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  // a tile's rows and head blocks fill at most the 8 waves; the tiles'
  // workgroups are a multiple of 8 (the rows' XCD mapping follows them)
  if (a.tq < 2 || a.tq > 8 || a.nb < 1 || a.tq * a.nb > 8 || a.tile_units < 8 ||
      a.tile_units % 8)
    return hipErrorInvalidConfiguration;
  FwdArgs b = a;
  b.groups = 1;
  b.bpg = 8;
  b.merge_wait_ticks = 0;
  const int64_t blocks = (int64_t)a.tile_units + (int64_t)(a.q_t + 7) / 8 * 8 * a.max_splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (t0 || t1)
    hipExtLaunchKernelGGL((fwd_kernel<8, 1, DQK, VMODE, FMT, true>), dim3((unsigned)blocks),
                          dim3(512), 0, s, t0, t1, 0, b);
  else
    hipLaunchKernelGGL((fwd_kernel<8, 1, DQK, VMODE, FMT, true>), dim3((unsigned)blocks),
                       dim3(512), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_forward_tiled(const FwdArgs& a, int dqk, int vmode, int fmt, hipStream_t s,
                                hipEvent_t t0, hipEvent_t t1) {
  switch (fmt) {
    case SFMLA_KV_BF16:
      if (dqk == 512) return vmode ? launch_tiled_t<512, 1, 0>(a, s, t0, t1)
                                   : launch_tiled_t<512, 0, 0>(a, s, t0, t1);
      return vmode ? launch_tiled_t<576, 1, 0>(a, s, t0, t1) : launch_tiled_t<576, 0, 0>(a, s, t0, t1);
    case SFMLA_KV_FP16:
      if (dqk == 512) return vmode ? launch_tiled_t<512, 1, SFMLA_KV_FP16>(a, s, t0, t1)
                                   : launch_tiled_t<512, 0, SFMLA_KV_FP16>(a, s, t0, t1);
      return vmode ? launch_tiled_t<576, 1, SFMLA_KV_FP16>(a, s, t0, t1)
                   : launch_tiled_t<576, 0, SFMLA_KV_FP16>(a, s, t0, t1);
    default:
      return hipErrorInvalidConfiguration;   // packed rows are not tiled
  }
}

// ---------------------------------------------------------------------------
// library-owned split workspace (sfmla_forward_static_workspace)
// ---------------------------------------------------------------------------

// Every GPU the library runs on holds one copy of this array from the time
// the code object is loaded on it until the process ends.  Its name is a
// host-side stand-in: kernels get the device address that
// hipGetSymbolAddress returns for the current device, never the name.
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

namespace {
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_workspace(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // once per device, with that device current (two threads racing here
    // read the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  int threads = (a.dv / 4 + 63) / 64 * 64;
  if (threads > 256) threads = 256;
  if (threads < 64) threads = 64;
  hipLaunchKernelGGL(combine_kernel, dim3(a.rows, a.heads), dim3(threads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_debug_resolve(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(resolve_kernel, dim3(a.q_t), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sfmla
