// gfx950 kernels of shared-KV sparse flash MLA attention.
//
//   plan_kernel        one thread per query row: lengths, position, extents of
//                      the window / list rules, split count (the metadata
//                      step of the sparse_flash_mla API page).
//   fwd_kernel         one workgroup per (split, query row, head group):
//                      resolve the split's list positions to physical rows,
//                      gather them into LDS, S^T = K Q^T on bf16 MFMA,
//                      online softmax, O^T += V^T P^T on bf16 MFMA, then the
//                      final output or a partial for the merge.
//   combine_kernel     LSE merge of split partials with the sink applied once.
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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sfmla_internal.h"

namespace sfmla {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ int64_t map_row(int layout, int64_t base, int bs, int bt_cols,
                                           const int32_t* bt, int b, int j, int64_t pool_rows,
                                           int32_t* status) {
  int64_t phys;
  if (layout == SFMLA_LAYOUT_PA_BSND) {
    int blk = j / bs;
    if (blk >= bt_cols) {
      if (status) atomicOr(status, SFMLA_STATUS_ROW_OUT_OF_RANGE);
      return -1;
    }
    phys = (int64_t)bt[(int64_t)b * bt_cols + blk] * bs + (j - blk * bs);
  } else {
    phys = base + j;
  }
  if (phys < 0 || phys >= pool_rows) {
    if (status) atomicOr(status, SFMLA_STATUS_ROW_OUT_OF_RANGE);
    return -1;
  }
  return phys;
}

// List position k of query row `row` -> physical row (or -1 if the slot is
// empty / masked).  *is_cmp tells which KV the row lives in.
__device__ __forceinline__ int64_t resolve_pos(const FwdArgs& a, const int32_t* rec, int row,
                                               int k, int* is_cmp) {
  const int ori_cnt = rec[R_ORI_CNT];
  const int b = rec[R_B];
  if (k < ori_cnt) {
    *is_cmp = 0;
    int j;
    if (a.ori_topk > 0) {
      const int v = a.ori_idx[(int64_t)row * a.ori_topk + k];
      if (v < 0 || v >= rec[R_ORI_LEN]) return -1;
      const int p = rec[R_P];
      if (a.ori_mode == SFMLA_MASK_CAUSAL && v > p) return -1;
      if (a.ori_mode == SFMLA_MASK_BAND &&
          ((a.win_l >= 0 && v < p - a.win_l) || (a.win_r >= 0 && v > p + a.win_r)))
        return -1;
      j = v;
    } else {
      j = rec[R_ORI_LO] + k;
    }
    return map_row(a.layout_kv, rec[R_ORI_BASE], a.ori_bs, a.ori_bt_cols, a.ori_bt, b, j,
                   a.ori_rows, a.status);
  }
  *is_cmp = 1;
  k -= ori_cnt;
  int j;
  if (a.cmp_topk > 0) {
    const int v = a.cmp_idx[(int64_t)row * a.cmp_topk + k];
    if (v < 0 || v >= rec[R_CMP_LIMIT]) return -1;
    j = v;
  } else {
    j = k;
  }
  return map_row(a.layout_kv, rec[R_CMP_BASE], a.cmp_bs, a.cmp_bt_cols, a.cmp_bt, b, j,
                 a.cmp_rows, a.status);
}

// ---------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------

__global__ void plan_kernel(PlanArgs a) {
  const sfmla_params& p = a.p;
  const int row = blockIdx.x * blockDim.x + threadIdx.x;
  if (row == 0) {
    a.meta[0] = kMagic;
    a.meta[1] = (int32_t)a.fingerprint;
    a.meta[2] = p.q_t;
    a.meta[3] = a.max_splits;
    for (int i = 4; i < kHeaderInts; ++i) a.meta[i] = 0;
  }
  if (row >= p.q_t) return;
  int b, i, q_len;
  if (p.layout_q == SFMLA_LAYOUT_BSND) {
    b = row / p.q_s;
    i = row - b * p.q_s;
    q_len = p.q_s;
  } else {
    int lo = 0, hi = p.batch_size - 1;  // last b with cu[b] <= row
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.len.cu_seqlens_q[mid] <= row) lo = mid; else hi = mid - 1;
    }
    b = lo;
    i = row - a.len.cu_seqlens_q[b];
    q_len = a.len.cu_seqlens_q[b + 1] - a.len.cu_seqlens_q[b];
  }
  int q_used = a.len.seqused_q ? a.len.seqused_q[b] : q_len;
  q_used = q_used < 0 ? 0 : (q_used > q_len ? q_len : q_used);

  int ori_len, ori_base = 0;
  if (a.len.seqused_ori_kv) ori_len = a.len.seqused_ori_kv[b];
  else if (p.layout_kv == SFMLA_LAYOUT_TND)
    ori_len = a.len.cu_seqlens_ori_kv[b + 1] - a.len.cu_seqlens_ori_kv[b];
  else ori_len = p.ori_kv_s;
  if (p.layout_kv == SFMLA_LAYOUT_TND) ori_base = a.len.cu_seqlens_ori_kv[b];
  else if (p.layout_kv == SFMLA_LAYOUT_BSND) ori_base = b * p.ori_kv_s;

  int cmp_len = 0, cmp_base = 0, res = 0;
  if (p.has_cmp_kv) {
    if (a.len.seqused_cmp_kv) cmp_len = a.len.seqused_cmp_kv[b];
    else if (p.layout_kv == SFMLA_LAYOUT_TND)
      cmp_len = a.len.cu_seqlens_cmp_kv[b + 1] - a.len.cu_seqlens_cmp_kv[b];
    else cmp_len = p.cmp_kv_s;
    if (p.layout_kv == SFMLA_LAYOUT_TND) cmp_base = a.len.cu_seqlens_cmp_kv[b];
    else if (p.layout_kv == SFMLA_LAYOUT_BSND) cmp_base = b * p.cmp_kv_s;
    if (a.len.cmp_residual_kv) res = a.len.cmp_residual_kv[b];
  }

  const int valid = i < q_used;
  const int pos = ori_len - q_used + i;
  const int pos_c = cmp_len * p.cmp_ratio + res - q_used + i;

  int ori_lo = 0, ori_cnt = 0;
  if (p.ori_topk > 0) {
    ori_cnt = p.ori_topk;
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
  int nsplit = n > 0 ? (n + kSplitRows - 1) / kSplitRows : 1;
  int chunk = kSplitRows;
  if (nsplit > a.max_splits) {
    nsplit = a.max_splits;
    chunk = (n + nsplit - 1) / nsplit;
    chunk = (chunk + kTile - 1) / kTile * kTile;
  }
  int32_t* r = a.meta + kHeaderInts + (int64_t)row * kRecInts;
  r[R_B] = b; r[R_I] = i; r[R_VALID] = valid; r[R_P] = pos; r[R_PC] = pos_c;
  r[R_ORI_LO] = ori_lo; r[R_ORI_CNT] = ori_cnt; r[R_CMP_CNT] = cmp_cnt;
  r[R_ORI_BASE] = ori_base; r[R_CMP_BASE] = cmp_base; r[R_ORI_LEN] = ori_len;
  r[R_CMP_LEN] = cmp_len; r[R_NSPLIT] = nsplit; r[R_CHUNK] = chunk;
  r[R_CMP_LIMIT] = cmp_limit; r[R_NTOTAL] = n;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

__device__ __forceinline__ bool plan_matches(const FwdArgs& a) {
  return a.meta[0] == kMagic && (uint32_t)a.meta[1] == a.fingerprint && a.meta[2] == a.q_t &&
         a.meta[3] == a.max_splits;
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
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
      f[0] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 0);
      f[1] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 1);
      f[2] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 2);
      f[3] = __builtin_amdgcn_cvt_f32_fp8((int)w[q], 3);
    }
    o[2 * q] = (__builtin_bit_cast(uint32_t, f[0]) >> 16) |
               (__builtin_bit_cast(uint32_t, f[1]) & 0xffff0000u);
    o[2 * q + 1] = (__builtin_bit_cast(uint32_t, f[2]) >> 16) |
                   (__builtin_bit_cast(uint32_t, f[3]) & 0xffff0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

template <int DQK, int VMODE, int FMT>
struct Lds {
  static constexpr int KSTR = DQK * 2 + 16;   // padded K row (bytes)
  static constexpr int VSTR = 512 * 2 + 16;   // padded V row (bytes)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + kTile * KSTR;
  static constexpr int SC_OFF = V_OFF + (VMODE ? kTile * VSTR : 0);
  static constexpr int PHYS_OFF = SC_OFF + kTile * 16;
  static constexpr int SIDE_OFF = PHYS_OFF + kTile * 8;
  static constexpr int BYTES = SIDE_OFF + kTile * 4;
};

template <int NW, int DQK, int VMODE, int FMT>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdArgs a) {
  using L = Lds<DQK, VMODE, FMT>;
  constexpr int NKS = DQK / 32;                 // k-steps of the QK product
  constexpr int NTHR = NW * 64;
  extern __shared__ __align__(16) char smem[];
  char* sK = smem + L::K_OFF;
  char* sV = VMODE ? smem + L::V_OFF : sK;
  constexpr int VS = VMODE ? L::VSTR : L::KSTR;
  float* sScale = (float*)(smem + L::SC_OFF);
  int64_t* sPhys = (int64_t*)(smem + L::PHYS_OFF);
  int32_t* sSide = (int32_t*)(smem + L::SIDE_OFF);

  const int row = blockIdx.x, split = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int g = l >> 4, t = l & 15;
  const int h0 = (hg * NW + w) * 16;
  const int h = h0 + t;
  const bool wave_on = h0 < a.qn;
  const bool head_on = h < a.qn;

  if (!plan_matches(a)) {
    if (split == 0 && head_on && row < a.q_t) {
      const float nan = __builtin_nanf("");
      uint16_t* op = a.out + ((int64_t)row * a.qn + h) * 512;
      for (int c = g; c < 512; c += 4) op[c] = f2bf(nan);
      if (a.lse && g == 0) a.lse[(int64_t)row * a.qn + h] = nan;
      if (a.status && tid == 0) atomicOr(a.status, SFMLA_STATUS_METADATA_MISMATCH);
    }
    return;
  }
  const int32_t* rec = a.meta + kHeaderInts + (int64_t)row * kRecInts;
  const int nsplit = rec[R_NSPLIT];
  if (split >= nsplit) return;
  const int n = rec[R_NTOTAL];
  const int chunk = rec[R_CHUNK];
  const int k0 = split * chunk;
  const int k1 = min(n, k0 + chunk);

  // this lane's slice of Q: B operand (k = d, n = head)
  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = a.q + ((int64_t)row * a.qn + (head_on ? h : 0)) * DQK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      uint4 v = head_on ? *(const uint4*)(qp + 32 * ks) : make_uint4(0, 0, 0, 0);
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[32];
#pragma unroll
  for (int mb = 0; mb < 32; ++mb) o[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf;
  float l_run = 0.f;

  for (int t0 = k0; t0 < k1; t0 += kTile) {
    // ---- resolve this tile's list positions
    if (tid < kTile) {
      const int k = t0 + tid;
      int side = 0;
      int64_t phys = -1;
      if (k < k1) phys = resolve_pos(a, rec, row, k, &side);
      sPhys[tid] = phys;
      sSide[tid] = side;
    }
    __syncthreads();

    // ---- gather the rows into LDS (16 bytes per thread per step)
    if constexpr (FMT == SFMLA_KV_BF16) {
      constexpr int CK = 64 + (DQK - 512) / 8;          // K chunks per row
      constexpr int CH = CK + (VMODE ? 64 : 0);
      for (int c = tid; c < kTile * CH; c += NTHR) {
        const int r = c / CH, cc = c - r * CH;
        const int64_t phys = sPhys[r];
        uint4 v = make_uint4(0, 0, 0, 0);
        char* dst;
        if (cc < 64) dst = sK + r * L::KSTR + cc * 16;
        else if (cc < CK) dst = sK + r * L::KSTR + 1024 + (cc - 64) * 16;
        else dst = sV + r * L::VSTR + (cc - CK) * 16;
        if (phys >= 0) {
          const int side = sSide[r];
          const char* kbase = side ? a.cmp_kv + phys * a.cmp_stride : a.ori_kv + phys * a.ori_stride;
          const char* src;
          if (cc < 64) {
            src = kbase + cc * 16;
          } else if (cc < CK) {
            const char* rp = side ? a.cmp_rope : a.ori_rope;
            const int64_t rs = side ? a.cmp_rope_stride : a.ori_rope_stride;
            src = (rp ? rp + phys * rs : kbase + 1024) + (cc - 64) * 16;
          } else {
            src = (side || !a.ori_v ? kbase : a.ori_v + phys * a.ori_v_stride) + (cc - CK) * 16;
          }
          v = *(const uint4*)src;
        }
        *(uint4*)dst = v;
      }
    } else {
      constexpr int CR = (DQK - 512) / 8;               // rope chunks
      constexpr int CH = 32 + CR + 1;
      for (int c = tid; c < kTile * CH; c += NTHR) {
        const int r = c / CH, cc = c - r * CH;
        const int64_t phys = sPhys[r];
        const char* rowp = nullptr;
        if (phys >= 0)
          rowp = sSide[r] ? a.cmp_kv + phys * a.cmp_stride : a.ori_kv + phys * a.ori_stride;
        if (cc < 32) {
          uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
          if (rowp) codes_to_bf16<FMT>(*(const uint4*)(rowp + cc * 16), lo, hi);
          *(uint4*)(sK + r * L::KSTR + cc * 32) = lo;
          *(uint4*)(sK + r * L::KSTR + cc * 32 + 16) = hi;
        } else if (cc < 32 + CR) {
          uint4 v = rowp ? *(const uint4*)(rowp + 512 + (cc - 32) * 16) : make_uint4(0, 0, 0, 0);
          *(uint4*)(sK + r * L::KSTR + 1024 + (cc - 32) * 16) = v;
        } else {
          uint4 v = rowp ? *(const uint4*)(rowp + 512 + 2 * (DQK - 512)) : make_uint4(0, 0, 0, 0);
          *(uint4*)(sScale + r * 4) = v;
        }
      }
    }
    __syncthreads();

    if (wave_on) {
      // ---- S^T = K Q^T : two 16-row blocks, M = rows, N = heads, K = d
      f32x4 s[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* kp = sK + (rb * 16 + t) * L::KSTR + 16 * g;
        if constexpr (FMT == SFMLA_KV_BF16) {
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            bf16x8 kv = *(const bf16x8*)(kp + 64 * ks);
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qreg[ks], s[rb], 0, 0, 0);
          }
        } else {
          // per-128-dim tile partial sums, scaled by that tile's fp32 scale
#pragma unroll
          for (int t4 = 0; t4 < 4; ++t4) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              bf16x8 kv = *(const bf16x8*)(kp + 64 * (4 * t4 + kk));
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qreg[4 * t4 + kk], acc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
              s[rb][i] += acc[i] * sScale[(rb * 16 + 4 * g + i) * 4 + t4];
          }
#pragma unroll
          for (int ks = 16; ks < NKS; ++ks) {
            bf16x8 kv = *(const bf16x8*)(kp + 64 * ks);
            s[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qreg[ks], s[rb], 0, 0, 0);
          }
        }
      }

      // ---- online softmax (log2 domain); lane holds head t, rows
      //      {4g+i, 16+4g+i}, i < 4
      float x[8];
      float mx = kNegInf;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = sPhys[rb * 16 + 4 * g + i] >= 0;
          const float v = ok ? s[rb][i] * a.scale_log2 : kNegInf;
          x[rb * 4 + i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(x[j] - m_use);
        psum += p[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int mb = 0; mb < 32; ++mb) o[mb] *= alpha;
      }

      // ---- O^T += V^T P^T : M = 16 value columns per block, N = heads,
      //      K = 32 rows with k = 8g+i <-> row (i<4 ? 4g+i : 16+4g+i-4)
      const char* vp = sV + (4 * g + (t >> 2)) * VS + 8 * (t & 3);
      if constexpr (FMT == SFMLA_KV_BF16) {
        bf16x8 pb;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];
#pragma unroll
        for (int mb = 0; mb < 32; ++mb) {
          s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 32 * mb));
          s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 16 * VS + 32 * mb));
          bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[mb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
          bf16x8 pb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int rr = (j < 4) ? 4 * g + j : 16 + 4 * g + (j - 4);
            pb[j] = (__bf16)(p[j] * sScale[rr * 4 + t4]);
          }
#pragma unroll
          for (int mb = 8 * t4; mb < 8 * t4 + 8; ++mb) {
            s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 32 * mb));
            s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp + 16 * VS + 32 * mb));
            bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, o[mb], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();
  }

  if (!wave_on) return;
  float lt = l_run + __shfl_xor(l_run, 16);
  lt += __shfl_xor(lt, 32);
  if (!head_on) return;
  const float lse2 = lt > 0.f ? m_run + __builtin_log2f(lt) : kNegInf;  // log2 units
  if (nsplit == 1) {
    float den = lt;
    if (a.has_sinks && lt > 0.f) den += __builtin_amdgcn_exp2f(a.sinks[h] * kLog2e - m_run);
    const float inv = lt > 0.f ? 1.f / den : 0.f;
    uint16_t* op = a.out + ((int64_t)row * a.qn + h) * 512 + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(o[mb][0] * inv) | ((uint32_t)f2bf(o[mb][1] * inv) << 16);
      pk.y = (uint32_t)f2bf(o[mb][2] * inv) | ((uint32_t)f2bf(o[mb][3] * inv) << 16);
      *(uint2*)(op + 16 * mb) = pk;
    }
    if (a.lse && g == 0) a.lse[(int64_t)row * a.qn + h] = lt > 0.f ? lse2 * kLn2 : kNegInf;
  } else {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t slot = ((int64_t)row * a.max_splits + split) * a.qn + h;
    float* wp = a.ws_o + slot * 512 + 4 * g;
#pragma unroll
    for (int mb = 0; mb < 32; ++mb) {
      float4 v = make_float4(o[mb][0] * inv, o[mb][1] * inv, o[mb][2] * inv, o[mb][3] * inv);
      *(float4*)(wp + 16 * mb) = v;
    }
    if (g == 0) a.ws_lse[slot] = lt > 0.f ? lse2 * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// merge of split partials
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int row = blockIdx.x, h = blockIdx.y;
  int np = a.n_parts;
  if (a.meta) {
    const int32_t* rec = a.meta + kHeaderInts + (int64_t)row * kRecInts;
    np = rec[R_NSPLIT];
    if (np <= 1) return;   // written directly by the forward
  }
  const float* lp = a.part_lse + row * a.lse_row_stride + h;
  float m = kNegInf;
  for (int k = 0; k < np; ++k) m = fmaxf(m, lp[k * a.lse_part_stride]);
  float mm = m;
  const bool sink = a.sinks != nullptr;
  const float sig = sink ? a.sinks[h] : kNegInf;
  if (sink) mm = fmaxf(mm, sig);
  const float ref = mm == kNegInf ? 0.f : mm;
  float tot = 0.f;
  for (int k = 0; k < np; ++k) tot += expf(lp[k * a.lse_part_stride] - ref);
  const float den = tot + (sink ? expf(sig - ref) : 0.f);
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
  if (!plan_matches(a)) {
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

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  const int threads = 128;
  const int blocks = (a.p.q_t + threads - 1) / threads;
  hipLaunchKernelGGL(plan_kernel, dim3(blocks > 0 ? blocks : 1), dim3(threads), 0, s, a);
  return hipGetLastError();
}

size_t forward_lds_bytes(int dqk, int vmode, int /*fmt*/) {
  if (dqk == 512) return vmode ? Lds<512, 1, 0>::BYTES : Lds<512, 0, 0>::BYTES;
  return vmode ? Lds<576, 1, 0>::BYTES : Lds<576, 0, 0>::BYTES;
}

template <int NW, int DQK, int VMODE, int FMT>
static hipError_t launch_fwd_t(const FwdArgs& a, int groups, hipStream_t s) {
  const size_t lds = Lds<DQK, VMODE, FMT>::BYTES;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)fwd_kernel<NW, DQK, VMODE, FMT>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((fwd_kernel<NW, DQK, VMODE, FMT>), dim3(a.q_t, a.max_splits, groups),
                     dim3(NW * 64), lds, s, a);
  return hipGetLastError();
}

template <int NW>
static hipError_t launch_fwd_nw(const FwdArgs& a, int dqk, int vmode, int fmt, int groups,
                                hipStream_t s) {
  if (fmt == SFMLA_KV_BF16) {
    if (dqk == 512) return vmode ? launch_fwd_t<NW, 512, 1, 0>(a, groups, s)
                                 : launch_fwd_t<NW, 512, 0, 0>(a, groups, s);
    return vmode ? launch_fwd_t<NW, 576, 1, 0>(a, groups, s)
                 : launch_fwd_t<NW, 576, 0, 0>(a, groups, s);
  }
  if (fmt == SFMLA_KV_INT8_PACKED)
    return dqk == 512 ? launch_fwd_t<NW, 512, 0, 1>(a, groups, s)
                      : launch_fwd_t<NW, 576, 0, 1>(a, groups, s);
  return dqk == 512 ? launch_fwd_t<NW, 512, 0, 2>(a, groups, s)
                    : launch_fwd_t<NW, 576, 0, 2>(a, groups, s);
}

hipError_t launch_forward(const FwdArgs& a, int nw, int dqk, int vmode, int fmt, int groups,
                          hipStream_t s) {
  switch (nw) {
    case 1: return launch_fwd_nw<1>(a, dqk, vmode, fmt, groups, s);
    case 2: return launch_fwd_nw<2>(a, dqk, vmode, fmt, groups, s);
    case 4: return launch_fwd_nw<4>(a, dqk, vmode, fmt, groups, s);
    default: return launch_fwd_nw<8>(a, dqk, vmode, fmt, groups, s);
  }
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
