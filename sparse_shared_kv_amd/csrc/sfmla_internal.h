// Internal definitions shared by the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "sfmla.h"

namespace sfmla {

constexpr int kTile = 32;          // KV rows staged in LDS per step
constexpr int kMaxSplitRows = 2048;   // most KV rows per split of one query row (LDS row table)
constexpr int kQueriesPerStep = 8;    // queries of a sequence per step of longer splits
constexpr int kHeaderInts = 16;
constexpr int kRecInts = 16;
constexpr int kCounterInts = 64;   // arrival counters per query row (one per head group x wave)
constexpr int kMinTileQueries = 16;   // query tiles by rule from this max_seqlen_q on
constexpr int kTileDescInts = 2;      // per query tile: first query row, row count
constexpr int32_t kMagic = 0x534d4c41;
// size of the library-owned split workspace (one static device array per GPU)
constexpr size_t kStaticWorkspaceBytes = SFMLA_STATIC_WORKSPACE_BYTES;

// Per-query-row plan record written by the planner (int32 each).
enum RecField {
  R_B = 0,       // batch index
  R_I,           // index of the query row inside its batch
  R_VALID,       // bit 0: i < seqused_q (else the row attends to nothing);
                 // bit 1: the row's sequence goes in query tiles
  R_P,           // original-KV position p = ori_len - q_used + i
  R_PC,          // compressed-side position cmp_len*ratio + residual - q_used + i
  R_ORI_LO,      // first row of the window rule
  R_ORI_CNT,     // window row count, or TopK slot count
  R_CMP_CNT,     // HCA visible count, or CSA slot count
  R_ORI_BASE,    // physical row of logical position 0 (BSND / TND)
  R_CMP_BASE,
  R_ORI_LEN,
  R_CMP_LEN,
  R_NSPLIT,      // number of splits of this row's list
  R_CHUNK,       // list positions per split
  R_CMP_LIMIT,   // compressed rows [0, limit) are visible
  R_NTOTAL       // list length (ori part + cmp part)
};

struct PlanArgs {
  sfmla_params p;
  sfmla_lengths len;
  int32_t* meta;
  uint32_t fingerprint;
  int32_t max_splits;
  int32_t split_rows;               // KV rows per split (multiple of the tile, <= kMaxSplitRows)
  int32_t split_rows_long;          // the longest split of a row of a sequence with many queries
  int32_t tq;                       // most query rows per tile (1: no tiles)
  int32_t tile_auto;                // rows per tile by each sequence's valid queries (else tq)
  int32_t tile_min_queries;         // valid queries from which a sequence is tiled
  int32_t tile_bound;               // tile descriptors written
  int64_t tile_off;                 // int offset of the descriptors in meta
};

struct FwdArgs {
  int32_t qn, q_t, layout_kv, rope;
  int32_t ori_bs, cmp_bs, ori_bt_cols, cmp_bt_cols;
  int64_t ori_rows, cmp_rows;
  int32_t ori_topk, cmp_topk, ori_mode, win_l, win_r, has_cmp;
  int32_t ori_sbs_log2;             // log2 of the tokens per ori TopK entry (block-wise TopK)
  int32_t max_splits, has_sinks;
  int32_t groups;                   // head groups of the launch
  int32_t bpg;                      // 16-head blocks per head group (<= waves; spare waves only load)
  int32_t split_rows;               // list positions per split of a short-query row
  int32_t merge_wait_ticks;         // owned-merge wait bound (s_memrealtime ticks; 0: none)
  int32_t tq;                       // most query rows per tile (tiled launch)
  int32_t nb;                       // 16-head blocks per query row (tiled launch)
  int32_t tile_units;               // tiled launch: workgroups of the tiles (a multiple of 8);
                                    // the rows of untiled sequences follow
  int64_t tile_off;                 // int offset of the tile descriptors in meta
  uint32_t fingerprint;
  float scale_log2;                 // softmax_scale * log2(e)
  const int32_t* meta;
  const uint16_t* q;
  const uint16_t* q_rope;           // rope part of the query stored apart (else null)
  uint32_t q_stride;                // elements per (row, head) of q: 512 + rope, or 512
  // row strides in bytes (< 2^31, so a row's offset is one 32 x 32 -> 64 multiply-add)
  const char* ori_kv;   uint32_t ori_stride;
  const char* ori_rope; uint32_t ori_rope_stride;
  const char* ori_v;    uint32_t ori_v_stride;
  const char* cmp_kv;   uint32_t cmp_stride;
  const char* cmp_rope; uint32_t cmp_rope_stride;
  const int32_t* ori_bt;
  const int32_t* cmp_bt;
  const int32_t* ori_idx;
  const int32_t* cmp_idx;
  const float* sinks;
  uint16_t* out;
  float* lse;
  int32_t* status;
  float* ws_lse;                    // [q_t][max_splits][heads] (bf16 path: log2 units)
  uint16_t* ws_ob;                  // bf16 path: partial O, per-wave fragment order
  int32_t* counters;                // [q_t][kCounterInts] arrival counters of split partials
  // debug resolve
  int64_t* dbg_rows;
  int32_t* dbg_counts;
  int32_t dbg_max_rows;
};

struct CombineArgs {
  int32_t rows, heads, dv;
  int32_t n_parts;
  int64_t o_part_stride, o_row_stride;      // in floats
  int64_t lse_part_stride, lse_row_stride;  // in floats
  const float* part_o;
  const float* part_lse;
  const float* sinks;
  uint16_t* out;
  float* lse_out;
};

// Kernel launchers (defined in sfmla_kernels.hip).
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// t0 / t1 (may be null): events the dispatch stamps at the kernel's start / end
// merge_wait_us: the owned-merge wait bound when every workgroup of the launch
// can be resident at once (0: never wait); pair: the eight-wave kernel whose
// wave pairs share 16 heads (16-bit rows, a.bpg pairs per head group)
hipError_t launch_forward(const FwdArgs& a, int nw, bool pair, int dqk, int vmode, int fmt,
                          int groups, int merge_wait_us, hipStream_t s, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr);
// launch with query tiles: a.tile_units workgroups for the tiles (one each,
// a.tq rows), then one per (split, row) of the rows of untiled sequences
hipError_t launch_forward_tiled(const FwdArgs& a, int dqk, int vmode, int fmt, hipStream_t s,
                                hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_debug_resolve(const FwdArgs& a, hipStream_t s);
// device address of the library-owned split workspace on the current device
// (looked up once per device; allocates nothing)
hipError_t static_workspace(void** ptr);

}  // namespace sfmla
