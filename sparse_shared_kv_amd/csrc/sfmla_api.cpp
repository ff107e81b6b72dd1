// Host side of libsfmla: parameter validation, plan / workspace sizing, the
// parameter fingerprint, kernel selection and the extern "C" entry points.
//
// The validation rules restate the sparse_flash_mla API page's 约束说明
// (constraints) that can be decided from shapes and attributes alone; rules
// that depend on tensor values are the caller's, as the page says.

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "sfmla_internal.h"

namespace {

thread_local std::string g_err;
// events for the next sfmla_forward launch on this thread (sfmla_time_next_forward)
thread_local void* g_time_start = nullptr;
thread_local void* g_time_stop = nullptr;

sfmla_status fail(sfmla_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

sfmla_status ok() {
  g_err.clear();
  return SFMLA_OK;
}

#define REQUIRE(cond, ...)                                           \
  do {                                                               \
    if (!(cond)) return fail(SFMLA_ERR_INVALID_ARGUMENT, __VA_ARGS__); \
  } while (0)

// FNV-1a over every field, one at a time (no padding bytes enter the hash).
uint32_t fingerprint(const sfmla_params& p) {
  uint32_t h = 2166136261u;
  auto mix = [&h](int64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (uint32_t)((v >> (8 * i)) & 0xff);
      h *= 16777619u;
    }
  };
  const int32_t f32[] = {
      p.num_heads_q, p.num_heads_kv, p.head_dim, p.rope_head_dim, p.batch_size, p.layout_q,
      p.layout_kv, p.q_s, p.q_t, p.ori_kv_s, p.cmp_kv_s, p.ori_block_size, p.cmp_block_size,
      p.ori_block_table_cols, p.cmp_block_table_cols, p.max_seqlen_q, p.max_seqlen_ori_kv,
      p.max_seqlen_cmp_kv, p.ori_topk, p.cmp_topk, p.ori_sparse_block_size, p.cmp_ratio,
      p.ori_mask_mode,
      p.cmp_mask_mode, p.ori_win_left, p.ori_win_right, p.has_ori_kv, p.has_cmp_kv,
      p.kv_dtype, p.has_separate_v, p.has_sinks, p.return_softmax_lse, p.has_seqused_q,
      p.has_seqused_ori_kv, p.has_seqused_cmp_kv, p.has_cmp_residual_kv, p.split_rows,
      p.head_blocks_per_group, p.merge_wait_us, p.query_tile, p.wave_pairs};
  for (int32_t v : f32) mix(v);
  mix(p.ori_kv_rows);
  mix(p.cmp_kv_rows);
  return h;
}

int64_t max_list(const sfmla_params& p);
int max_splits(const sfmla_params& p);
int tile_limit(const sfmla_params& p);
bool tile_eligible(const sfmla_params& p);
// heads each wave holds (one 16-head MFMA block)
void choose_groups(const sfmla_params& p, int* nw, int* groups, int* bpg, bool* pair = nullptr);

// Heads of split partial per wave, in units of 512 columns: 16, or 8 where
// wave pairs split the columns (16 heads x 256 columns per wave).
int heads_per_wave(const sfmla_params& p) {
  int nw, groups, bpg;
  bool pair = false;
  choose_groups(p, &nw, &groups, &bpg, &pair);
  return pair ? 8 : 16;
}
bool pair_eligible(const sfmla_params& p);

sfmla_status validate(const sfmla_params* pp) {
  REQUIRE(pp != nullptr, "params is NULL");
  const sfmla_params& p = *pp;
  REQUIRE(p.num_heads_q >= 1 && p.num_heads_q <= 128, "num_heads_q must be in 1..128 (got %d)",
          p.num_heads_q);
  REQUIRE(p.num_heads_kv == 1, "num_heads_kv must be 1 (got %d)", p.num_heads_kv);
  REQUIRE(p.head_dim == 512, "head_dim must be 512 (got %d)", p.head_dim);
  REQUIRE(p.rope_head_dim == 0 || p.rope_head_dim == 64, "rope_head_dim must be 0 or 64 (got %d)",
          p.rope_head_dim);
  REQUIRE(p.batch_size > 0, "batch_size must be > 0");
  REQUIRE(p.layout_q == SFMLA_LAYOUT_BSND || p.layout_q == SFMLA_LAYOUT_TND,
          "layout_q must be BSND or TND");
  REQUIRE(p.layout_kv == SFMLA_LAYOUT_BSND || p.layout_kv == SFMLA_LAYOUT_TND ||
              p.layout_kv == SFMLA_LAYOUT_PA_BSND,
          "layout_kv must be BSND, TND or PA_BSND");
  REQUIRE(p.layout_kv == SFMLA_LAYOUT_PA_BSND || p.layout_kv == p.layout_q,
          "a non-paged layout_kv must equal layout_q");
  if (p.layout_q == SFMLA_LAYOUT_BSND) {
    REQUIRE(p.q_s > 0, "BSND q needs q_s > 0");
    REQUIRE((int64_t)p.q_t == (int64_t)p.batch_size * p.q_s, "BSND q_t must be batch_size*q_s");
  } else {
    REQUIRE(p.q_t > 0, "TND q needs q_t > 0");
  }
  REQUIRE(p.max_seqlen_q > 0, "max_seqlen_q must be > 0");
  REQUIRE((int64_t)p.q_t * p.num_heads_q < ((int64_t)1 << 31), "q_t * num_heads_q must be < 2^31");
  REQUIRE(p.has_ori_kv == 1, "ori_kv is required");
  REQUIRE(p.max_seqlen_ori_kv > 0, "max_seqlen_ori_kv must be > 0");
  REQUIRE(p.ori_kv_rows > 0, "ori_kv_rows must be > 0");
  REQUIRE(p.ori_kv_rows < ((int64_t)1 << 31) - 1, "ori_kv_rows must be < 2^31 - 1");
  REQUIRE(p.ori_win_left >= -1 && p.ori_win_right >= -1, "window bounds must be -1 or >= 0");
  REQUIRE(p.ori_topk >= 0 && p.cmp_topk >= 0, "topk must be >= 0");
  {
    const int s = p.ori_sparse_block_size;
    REQUIRE(s >= 1 && s <= 128 && (s & (s - 1)) == 0,
            "ori_sparse_block_size must be a power of two in 1..128");
    REQUIRE(s == 1 || p.ori_topk > 0, "ori_sparse_block_size > 1 needs an ori TopK list");
    REQUIRE(p.layout_kv != SFMLA_LAYOUT_PA_BSND || s == 1 || p.ori_block_size % s == 0,
            "ori_sparse_block_size must divide ori_block_size");
    REQUIRE((int64_t)p.ori_topk * s <= ((int64_t)1 << 30), "ori_topk * ori_sparse_block_size too large");
  }
  REQUIRE(p.ori_mask_mode == 0 || p.ori_mask_mode == 3 || p.ori_mask_mode == 4,
          "ori_mask_mode must be 0, 3 or 4");
  REQUIRE(p.kv_dtype == SFMLA_KV_BF16 || p.kv_dtype == SFMLA_KV_FP16 ||
              p.kv_dtype == SFMLA_KV_INT8_PACKED ||
              p.kv_dtype == SFMLA_KV_FP8_E4M3_PACKED,
          "unknown kv_dtype");
  REQUIRE(!(p.has_separate_v && p.has_cmp_kv &&
            (p.kv_dtype == SFMLA_KV_INT8_PACKED || p.kv_dtype == SFMLA_KV_FP8_E4M3_PACKED)),
          "a value tensor with packed KV is for the token-wise TopK form (no cmp_kv)");
  REQUIRE(p.split_rows == 0 ||
              (p.split_rows >= sfmla::kTile && p.split_rows <= sfmla::kMaxSplitRows &&
               p.split_rows % sfmla::kTile == 0),
          "split_rows must be 0 or a multiple of %d in %d..%d", sfmla::kTile, sfmla::kTile,
          sfmla::kMaxSplitRows);
  REQUIRE(p.head_blocks_per_group == 0 || p.head_blocks_per_group == 1 ||
              p.head_blocks_per_group == 2 || p.head_blocks_per_group == 4 ||
              p.head_blocks_per_group == 8,
          "head_blocks_per_group must be 0, 1, 2, 4 or 8");
  REQUIRE(p.merge_wait_us >= -1 && p.merge_wait_us <= 10000,
          "merge_wait_us must be -1, 0 or 1..10000");
  REQUIRE(p.query_tile == 0 || p.query_tile == 1 || p.query_tile == 2 || p.query_tile == 4 ||
              p.query_tile == 8,
          "query_tile must be 0, 1, 2, 4 or 8");
  REQUIRE(p.wave_pairs >= 0 && p.wave_pairs <= 2, "wave_pairs must be 0, 1 or 2");
  if (p.wave_pairs == 2)
    REQUIRE(pair_eligible(p),
            "wave_pairs 2 needs a call without query tiles");
  if (p.query_tile > 1) {
    REQUIRE(tile_eligible(p) && p.query_tile <= tile_limit(p),
            "query_tile %d needs rule lists (ori_topk = cmp_topk = 0), bf16 or float16 KV "
            "and %d rows x 16-head blocks <= 8",
            p.query_tile, p.query_tile);
  }
  if (p.layout_kv == SFMLA_LAYOUT_BSND) REQUIRE(p.ori_kv_s > 0, "BSND ori_kv needs ori_kv_s > 0");
  if (p.layout_kv == SFMLA_LAYOUT_PA_BSND) {
    REQUIRE(p.ori_block_size >= 1 && p.ori_block_size <= 1024, "ori_block_size must be in 1..1024");
    REQUIRE(p.ori_block_table_cols > 0, "PA needs ori_block_table_cols > 0");
    REQUIRE(p.has_seqused_ori_kv, "PA needs seqused_ori_kv");
  }
  if (p.has_cmp_kv) {
    REQUIRE(p.has_cmp_kv == 1, "has_cmp_kv must be 0 or 1");
    REQUIRE(p.cmp_ratio >= 1, "cmp_ratio must be >= 1");
    REQUIRE(p.cmp_mask_mode == 0 || p.cmp_mask_mode == 3, "cmp_mask_mode must be 0 or 3");
    REQUIRE(p.cmp_kv_rows > 0 && p.cmp_kv_rows < ((int64_t)1 << 31) - 1,
            "cmp_kv_rows must be in 1..2^31 - 2");
    if (p.cmp_mask_mode == 3)
      REQUIRE(p.has_cmp_residual_kv, "cmp_mask_mode 3 needs cmp_residual_kv");
    if (p.layout_kv == SFMLA_LAYOUT_BSND) REQUIRE(p.cmp_kv_s > 0, "BSND cmp_kv needs cmp_kv_s > 0");
    if (p.layout_kv == SFMLA_LAYOUT_PA_BSND) {
      REQUIRE(p.cmp_block_size >= 1 && p.cmp_block_size <= 1024, "cmp_block_size must be in 1..1024");
      REQUIRE(p.cmp_block_table_cols > 0, "PA cmp_kv needs cmp_block_table_cols > 0");
      REQUIRE(p.has_seqused_cmp_kv, "PA cmp_kv needs seqused_cmp_kv");
    }
  } else {
    REQUIRE(p.cmp_topk == 0, "cmp_topk must be 0 without cmp_kv");
    REQUIRE(p.cmp_ratio == 1, "cmp_ratio must be 1 without cmp_kv");
  }
  // A query row's list goes in at most 4096 splits of at most kMaxSplitRows
  // rows (the kernel's LDS row table), and one row's split partials are
  // addressed with 32-bit offsets.
  const int64_t n = max_list(p);
  REQUIRE(n <= (int64_t)4096 * sfmla::kMaxSplitRows,
          "a query row's list may hold %lld rows; at most %lld are supported", (long long)n,
          (long long)4096 * sfmla::kMaxSplitRows);
  int nw, groups, bpg;
  choose_groups(p, &nw, &groups, &bpg);
  const int64_t part_bytes = (int64_t)max_splits(p) * groups * nw * heads_per_wave(p) * 512 * 2;
  REQUIRE(part_bytes < ((int64_t)1 << 31),
          "split partials of one query row would take %lld bytes (limit 2^31)",
          (long long)part_bytes);
  return ok();
}

int64_t max_list(const sfmla_params& p) {
  int64_t n;
  if (p.ori_topk > 0) {
    n = (int64_t)p.ori_topk * p.ori_sparse_block_size;
  } else if (p.ori_mask_mode == 4 && p.ori_win_left >= 0 && p.ori_win_right >= 0) {
    n = std::min<int64_t>(p.max_seqlen_ori_kv, (int64_t)p.ori_win_left + p.ori_win_right + 1);
  } else {
    n = p.max_seqlen_ori_kv;
  }
  if (p.has_cmp_kv) n += p.cmp_topk > 0 ? p.cmp_topk : p.max_seqlen_cmp_kv;
  return n;
}

// KV rows per split: a function of the parameters only (never of the batch),
// so a query row is split the same way in any batch (the planner lengthens
// the splits of rows of sequences with many queries, one more step of this
// size per kQueriesPerStep queries up to kMaxSplitRows, a property of the
// row's own sequence).  Rows of 2 KB or more
// (a K row with rope plus a separate V row) get 512-row splits, which keep
// the number of partials to merge low; lighter rows (1 KB bf16 rows with
// V = K, packed rows) get 256-row splits, which keep each workgroup's serial
// chain of tiles short (measured on the six workloads of the benchmark).
// params.split_rows, when nonzero, overrides the rule.
int split_rows(const sfmla_params& p) {
  if (p.split_rows) return p.split_rows;
  const bool packed = p.kv_dtype == SFMLA_KV_INT8_PACKED || p.kv_dtype == SFMLA_KV_FP8_E4M3_PACKED;
  const int row_bytes = packed ? 512 + 2 * p.rope_head_dim + 16
                               : 2 * (512 + p.rope_head_dim) + (p.has_separate_v ? 1024 : 0);
  // (packed rows with a value tensor add 512 code bytes: still below 2 KB)
  const int base = row_bytes >= 2048 ? 512 : 256;
  // Where the parameters alone bound the list (TopK slot counts, a window
  // open on both sides), the longest list is cut into even splits of at most
  // `base` rows, so its last split is not a short tail
  int64_t n = 0;
  if (p.ori_topk > 0) n = (int64_t)p.ori_topk * p.ori_sparse_block_size;
  else if (p.ori_mask_mode == SFMLA_MASK_BAND && p.ori_win_left >= 0 && p.ori_win_right >= 0)
    n = (int64_t)p.ori_win_left + p.ori_win_right + 1;
  else return base;
  if (p.has_cmp_kv) {
    if (p.cmp_topk <= 0) return base;                    // all visible rows: data-dependent
    n += p.cmp_topk;
  }
  if (n <= base) return base;
  const int64_t s = (n + base - 1) / base;
  const int64_t even = ((n + s - 1) / s + sfmla::kTile - 1) / sfmla::kTile * sfmla::kTile;
  return (int)even;
}

int max_splits(const sfmla_params& p) {
  const int64_t n = max_list(p);
  const int64_t s = (n + split_rows(p) - 1) / split_rows(p);
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, 4096));
}

// Query tiles.  Rows per tile that the waves of one workgroup hold: the 16-head
// blocks of a row, rounded up to a power of two, times the rows fill the 8
// waves (1: a row's heads need every wave).
int tile_limit(const sfmla_params& p) {
  const int blocks = (p.num_heads_q + 15) / 16;
  int pw = 1;
  while (pw < blocks) pw *= 2;
  return 8 / pw;
}

// Tiles need rule lists (a tile's rows then share most of their rows: the
// windows of consecutive rows overlap, the visible compressed rows of one
// row include the earlier row's) and 16-bit rows (the eight-wave kernel).
bool tile_eligible(const sfmla_params& p) {
  return (p.kv_dtype == SFMLA_KV_BF16 || p.kv_dtype == SFMLA_KV_FP16) && p.ori_topk == 0 &&
         p.cmp_topk == 0 && tile_limit(p) >= 2;
}

// Rows the four-wave kernel with two workgroups per CU takes where the
// launch fills the GPU: 16-bit, no rope, V = K nope, at most 64 heads.  It
// was measured faster than query tiles on every prefill shape (hca_prefill
// 94.3 vs 97.6 us, swa_prefill 27.2 vs 33.0, 16 heads 14.5 vs 20.5), so
// tiles are not the rule there.
bool four_wave_rows(const sfmla_params& p) {
  return (p.kv_dtype == SFMLA_KV_BF16 || p.kv_dtype == SFMLA_KV_FP16) && !p.has_separate_v &&
         p.rope_head_dim == 0 && p.num_heads_q <= 64;
}

// Most query rows per tile of this call (1: no tiles).  By rule: the most
// the waves hold, where a sequence may be long enough to be a prefill.
// Which sequences are tiled, and by rule with how many rows, is decided on
// the device from each sequence's own lengths (at least kMinTileQueries
// valid queries by rule, any number when forced, and a tile's union list
// within one split).
int query_tile(const sfmla_params& p) {
  if (p.query_tile == 1) return 1;
  if (p.query_tile > 1) return p.query_tile;        // validated
  if (!tile_eligible(p) || p.max_seqlen_q < sfmla::kMinTileQueries || four_wave_rows(p)) return 1;
  return tile_limit(p);
}

// Tile descriptors of a tiled call: at least the tiles any batch of these
// parameters has (sum over sequences of ceil(len / tq) <= (q_t + b (tq - 1)) / tq
// with the fewest rows per tile, and at most one per query row), rounded up
// to a multiple of 8 so that the rows of untiled sequences that follow the
// tiles in the grid start on XCD 0.
int64_t tile_bound(const sfmla_params& p) {
  if (query_tile(p) <= 1) return 0;
  const int tq = p.query_tile > 1 ? p.query_tile : 2;
  const int64_t n = std::min<int64_t>(((int64_t)p.q_t + (int64_t)p.batch_size * (tq - 1)) / tq,
                                      p.q_t);
  return (n + 7) / 8 * 8;
}

size_t tile_off(const sfmla_params& p) {
  return (size_t)sfmla::kHeaderInts +
         (size_t)(sfmla::kRecInts + sfmla::kCounterInts) * (size_t)p.q_t;
}

size_t metadata_ints(const sfmla_params& p) {
  return tile_off(p) + (size_t)sfmla::kTileDescInts * (size_t)tile_bound(p);
}

// Longest wait (us) of a split that merges the partials of its row's other
// splits for them (the splits of a row end within a few us of each other;
// past this bound it hands the merge to the last split to arrive).
constexpr int kMergeWaitUs = 40;

// Workgroups below which a launch spreads a row's heads over several groups,
// and the most it spreads them to: one workgroup per CU of the eight-wave
// kernels, a single round (a grouping past it runs its workgroups in two
// rounds: packed decode with 6 splits of 8 rows, 384 workgroups of one wave
// pair each, took 54 us against 31 for 192 of two pairs).
constexpr int64_t kMinGroups = 256;

// Split partials: normalised bf16 partial O for every (row, split, padded
// head), laid out per wave in MFMA fragment order, then the log2-domain LSEs.
struct WsLayout {
  size_t o_bytes, lse_bytes, total;
  int heads;   // heads per row as laid out (padded to whole waves)
};

WsLayout workspace_layout(const sfmla_params& p) {
  WsLayout L{0, 0, 0, p.num_heads_q};
  const int s = max_splits(p);
  if (s <= 1) return L;
  int nw, groups, bpg;
  choose_groups(p, &nw, &groups, &bpg);
  L.heads = groups * nw * heads_per_wave(p);
  const size_t slots = (size_t)p.q_t * s * L.heads;
  L.o_bytes = (slots * 512 * 2 + 255) / 256 * 256;
  L.lse_bytes = (slots * sizeof(float) + 255) / 256 * 256;
  L.total = L.o_bytes + L.lse_bytes;
  return L;
}

size_t workspace_bytes(const sfmla_params& p) { return workspace_layout(p).total; }

// Wave pairs: any call without query tiles (16-bit or packed rows).
bool pair_eligible(const sfmla_params& p) { return query_tile(p) <= 1; }

// Workgroup shape: nw waves; the heads of a query row are cut into `groups`
// head groups of bpg 16-head blocks (bpg <= nw), one block per wave, and the
// waves past bpg only help gather.  All heads of a query row share one
// workgroup (the KV rows are gathered once) unless the grid would have too
// few workgroups to spread over the chip; then the heads are spread over
// more groups, each re-gathering the row's KV (mostly from L2).  The shape
// never changes a result: every head is computed the same way in any group.
void choose_groups(const sfmla_params& p, int* nw, int* groups, int* bpg, bool* pair) {
  if (pair) *pair = false;
  if (query_tile(p) > 1) {
    // with query tiles, an untiled sequence's rows take every head in one
    // workgroup (tiles keep the grid full)
    *nw = 8;
    *groups = 1;
    *bpg = 8;
    return;
  }
  const int64_t units = (int64_t)p.q_t * max_splits(p);
  // Wave pairs: eight waves, bpg pairs of 16 heads per head group (every
  // wave's partial is 16 heads x 256 columns).  By rule only where even
  // four pairs per group keep the launch within one round (packed rows, 40
  // rows of 4 splits, 128 heads: 320 workgroups of pairs took 67 us, 160
  // without pairs 54)
  const int64_t pair_groups = ((p.num_heads_q + 15) / 16 + 3) / 4;
  const bool pairs = p.wave_pairs == 2 ||
                     (p.wave_pairs == 0 && pair_eligible(p) && p.head_blocks_per_group == 0 &&
                      units < kMinGroups && units * pair_groups <= kMinGroups);
  if (pairs) {
    if (pair) *pair = true;
    *nw = 8;
    const int pblocks = (p.num_heads_q + 15) / 16;
    int per = p.head_blocks_per_group ? std::min(p.head_blocks_per_group, 4) : 4;
    per = std::min(per, pblocks);
    if (per == 3) per = 2;
    if (!p.head_blocks_per_group)
      while (per > 1 && units * ((pblocks + per - 1) / per) < kMinGroups &&
             units * ((pblocks + per / 2 - 1) / (per / 2)) <= kMinGroups)
        per /= 2;
    *bpg = per;
    *groups = (pblocks + per - 1) / per;
    return;
  }
  const int blocks = (p.num_heads_q + 15) / 16;       // 16-head blocks of one wave each
  const bool packed = p.kv_dtype == SFMLA_KV_INT8_PACKED || p.kv_dtype == SFMLA_KV_FP8_E4M3_PACKED;
  // Packed rows: eight waves, two per SIMD, the decode and the gather of a
  // tile spread over all of them (a four-wave kernel with one wave per SIMD
  // and the whole register file measured slower at every size:
  // c8_packed_int8_q32 470 vs 280 us, c8_packed_int8 39.3 vs 37.6).
  int wmax = 8;
  // 16-bit rows without rope whose V is the K nope, at most 64 heads, in a
  // launch that fills the GPU: four waves, two workgroups per CU (every
  // SIMD then has two waves in the products; eight waves with four holding
  // heads leave one per SIMD): csa_prefill 74.5 -> 61.0 us
  if (four_wave_rows(p) && units >= kMinGroups && p.head_blocks_per_group == 0) wmax = 4;
  *nw = wmax;
  // params.head_blocks_per_group, when nonzero, overrides the rule
  if (p.head_blocks_per_group) {
    *bpg = std::min(p.head_blocks_per_group, wmax);
    *groups = (blocks + *bpg - 1) / *bpg;
    return;
  }
  int per = 1;                                         // blocks per group: 1, 2, 4 or 8
  while (per < wmax && per < blocks) per *= 2;
  while (per > 1 && units * ((blocks + per - 1) / per) < kMinGroups &&
         units * ((blocks + per / 2 - 1) / (per / 2)) <= kMinGroups)
    per /= 2;
  *bpg = per;
  *groups = (blocks + per - 1) / per;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15) == 0; }

sfmla_status fill_fwd_args(const sfmla_params& p, const sfmla_tensors* t, const int32_t* meta,
                           size_t n_ints, float scale, sfmla::FwdArgs* a) {
  REQUIRE(t != nullptr, "tensors is NULL");
  REQUIRE(meta != nullptr, "metadata is NULL");
  REQUIRE(aligned16(meta), "metadata must be 16-byte aligned");
  if (n_ints < metadata_ints(p))
    return fail(SFMLA_ERR_BUFFER_TOO_SMALL, "metadata holds %zu int32, needs %zu", n_ints,
                metadata_ints(p));
  REQUIRE(std::isfinite(scale), "softmax_scale must be finite");
  REQUIRE(t->q && aligned16(t->q), "q must be a 16-byte aligned device pointer");
  REQUIRE(!t->q_rope || (p.rope_head_dim == 64 && aligned16(t->q_rope)),
          "q_rope needs rope_head_dim 64 and a 16-byte aligned device pointer");
  REQUIRE(t->ori_kv && aligned16(t->ori_kv), "ori_kv must be a 16-byte aligned device pointer");
  const bool packed = p.kv_dtype == SFMLA_KV_INT8_PACKED || p.kv_dtype == SFMLA_KV_FP8_E4M3_PACKED;
  const int64_t need_row = packed ? 512 + 2 * p.rope_head_dim + 16
                                  : (p.rope_head_dim && !t->ori_rope ? 1152 : 1024);
  constexpr int64_t kMaxStride = ((int64_t)1 << 31) - 16;   // device row offsets are 32 x 32 bit
  REQUIRE(t->ori_kv_stride <= kMaxStride && t->ori_rope_stride <= kMaxStride &&
              t->ori_v_stride <= kMaxStride && t->cmp_kv_stride <= kMaxStride &&
              t->cmp_rope_stride <= kMaxStride,
          "row strides must be < 2^31 bytes");
  REQUIRE(t->ori_kv_stride >= need_row && t->ori_kv_stride % 16 == 0,
          "ori_kv_stride must be >= %lld bytes and a multiple of 16", (long long)need_row);
  if (t->ori_rope) {
    REQUIRE(!packed && p.rope_head_dim == 64, "ori_rope is only used with bf16 KV and rope 64");
    REQUIRE(aligned16(t->ori_rope) && t->ori_rope_stride >= 128 && t->ori_rope_stride % 16 == 0,
            "ori_rope must be 16-byte aligned with a stride >= 128, multiple of 16");
  }
  REQUIRE((p.has_separate_v != 0) == (t->ori_v != nullptr), "has_separate_v must match ori_v");
  if (t->ori_v) {
    // 16-bit V rows (512 values), or packed KV's value codes (512 bytes)
    const int64_t vmin = packed ? 512 : 1024;
    REQUIRE(aligned16(t->ori_v) && t->ori_v_stride >= vmin && t->ori_v_stride % 16 == 0,
            "ori_v must be 16-byte aligned with a stride >= %lld, multiple of 16", (long long)vmin);
  }
  if (p.has_cmp_kv) {
    REQUIRE(t->cmp_kv && aligned16(t->cmp_kv), "cmp_kv must be a 16-byte aligned device pointer");
    const int64_t need_c = packed ? 512 + 2 * p.rope_head_dim + 16
                                  : (p.rope_head_dim && !t->cmp_rope ? 1152 : 1024);
    REQUIRE(t->cmp_kv_stride >= need_c && t->cmp_kv_stride % 16 == 0,
            "cmp_kv_stride must be >= %lld bytes and a multiple of 16", (long long)need_c);
    if (t->cmp_rope)
      REQUIRE(!packed && p.rope_head_dim == 64 && aligned16(t->cmp_rope) &&
                  t->cmp_rope_stride >= 128 && t->cmp_rope_stride % 16 == 0,
              "cmp_rope needs bf16 KV, rope 64, 16-byte alignment and stride >= 128");
  } else {
    REQUIRE(t->cmp_kv == nullptr, "cmp_kv given but has_cmp_kv is 0");
  }
  if (p.layout_kv == SFMLA_LAYOUT_PA_BSND) {
    REQUIRE(t->ori_block_table, "PA needs ori_block_table");
    if (p.has_cmp_kv) REQUIRE(t->cmp_block_table, "PA needs cmp_block_table");
  }
  REQUIRE((p.ori_topk > 0) == (t->ori_sparse_indices != nullptr),
          "ori_sparse_indices must be given exactly when ori_topk > 0");
  REQUIRE((p.cmp_topk > 0) == (t->cmp_sparse_indices != nullptr),
          "cmp_sparse_indices must be given exactly when cmp_topk > 0 (CSA) and not for HCA");
  REQUIRE((p.has_sinks != 0) == (t->sinks != nullptr), "has_sinks must match sinks");
  REQUIRE((p.return_softmax_lse != 0) == (t->softmax_lse != nullptr),
          "return_softmax_lse must match softmax_lse");
  REQUIRE(t->attention_out && ((uintptr_t)t->attention_out & 7) == 0,
          "attention_out must be an 8-byte aligned device pointer");

  sfmla::FwdArgs& f = *a;
  std::memset(&f, 0, sizeof f);
  f.qn = p.num_heads_q;
  f.q_t = p.q_t;
  f.layout_kv = p.layout_kv;
  f.rope = p.rope_head_dim;
  f.ori_bs = p.ori_block_size;
  f.cmp_bs = p.cmp_block_size;
  f.ori_bt_cols = p.ori_block_table_cols;
  f.cmp_bt_cols = p.cmp_block_table_cols;
  f.ori_rows = p.ori_kv_rows;
  f.cmp_rows = p.cmp_kv_rows;
  f.ori_topk = p.ori_topk;
  f.ori_sbs_log2 = __builtin_ctz((unsigned)p.ori_sparse_block_size);   // a power of two
  f.cmp_topk = p.cmp_topk;
  f.ori_mode = p.ori_mask_mode;
  f.win_l = p.ori_win_left;
  f.win_r = p.ori_win_right;
  f.has_cmp = p.has_cmp_kv;
  f.max_splits = max_splits(p);
  f.split_rows = split_rows(p);
  f.has_sinks = p.has_sinks;
  f.fingerprint = fingerprint(p);
  f.scale_log2 = scale * 1.4426950408889634f;
  f.meta = meta;
  f.q = (const uint16_t*)t->q;
  f.q_rope = (const uint16_t*)t->q_rope;
  f.q_stride = t->q_rope ? 512u : (uint32_t)(512 + p.rope_head_dim);
  f.ori_kv = (const char*)t->ori_kv;
  f.ori_stride = (uint32_t)t->ori_kv_stride;
  f.ori_rope = (const char*)t->ori_rope;
  f.ori_rope_stride = (uint32_t)t->ori_rope_stride;
  f.ori_v = (const char*)t->ori_v;
  f.ori_v_stride = (uint32_t)t->ori_v_stride;
  f.cmp_kv = (const char*)t->cmp_kv;
  f.cmp_stride = (uint32_t)t->cmp_kv_stride;
  f.cmp_rope = (const char*)t->cmp_rope;
  f.cmp_rope_stride = (uint32_t)t->cmp_rope_stride;
  // The kernel takes every row address as base + row * stride: a V that is
  // the K nope and a rope stored after the nope become bases of their own.
  if (!f.ori_v) { f.ori_v = f.ori_kv; f.ori_v_stride = f.ori_stride; }
  if (!f.ori_rope) { f.ori_rope = f.ori_kv + 1024; f.ori_rope_stride = f.ori_stride; }
  if (!f.cmp_kv) { f.cmp_kv = f.ori_kv; f.cmp_stride = f.ori_stride; }
  if (!f.cmp_rope) { f.cmp_rope = f.cmp_kv + 1024; f.cmp_rope_stride = f.cmp_stride; }
  f.ori_bt = t->ori_block_table;
  f.cmp_bt = t->cmp_block_table;
  f.ori_idx = t->ori_sparse_indices;
  f.cmp_idx = t->cmp_sparse_indices;
  f.sinks = t->sinks;
  f.out = (uint16_t*)t->attention_out;
  f.lse = t->softmax_lse;
  f.status = t->status;
  return ok();
}

}  // namespace

extern "C" {

sfmla_status sfmla_time_next_forward(void* start_event, void* stop_event) {
  g_time_start = start_event;
  g_time_stop = stop_event;
  return ok();
}

const char* sfmla_last_error(void) { return g_err.c_str(); }

const char* sfmla_version(void) { return SFMLA_VERSION; }

sfmla_status sfmla_metadata_size(const sfmla_params* params, size_t* n_ints) {
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  REQUIRE(n_ints != nullptr, "n_ints is NULL");
  *n_ints = metadata_ints(*params);
  return ok();
}

sfmla_status sfmla_workspace_size(const sfmla_params* params, size_t* bytes) {
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = workspace_bytes(*params);
  return ok();
}

sfmla_status sfmla_metadata(const sfmla_params* params, const sfmla_lengths* len,
                            int32_t* metadata, size_t n_ints, void* stream) {
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  const sfmla_params& p = *params;
  REQUIRE(len != nullptr, "lengths is NULL");
  REQUIRE(metadata != nullptr, "metadata is NULL");
  REQUIRE(aligned16(metadata), "metadata must be 16-byte aligned");
  if (n_ints < metadata_ints(p))
    return fail(SFMLA_ERR_BUFFER_TOO_SMALL, "metadata holds %zu int32, needs %zu", n_ints,
                metadata_ints(p));
  REQUIRE((p.layout_q == SFMLA_LAYOUT_TND) == (len->cu_seqlens_q != nullptr),
          "cu_seqlens_q is required for TND q and not accepted otherwise");
  REQUIRE((p.layout_kv == SFMLA_LAYOUT_TND) == (len->cu_seqlens_ori_kv != nullptr),
          "cu_seqlens_ori_kv is required for TND kv and not accepted otherwise");
  REQUIRE((p.layout_kv == SFMLA_LAYOUT_TND && p.has_cmp_kv) == (len->cu_seqlens_cmp_kv != nullptr),
          "cu_seqlens_cmp_kv is required for TND cmp_kv and not accepted otherwise");
  REQUIRE((p.has_seqused_q != 0) == (len->seqused_q != nullptr), "has_seqused_q must match");
  REQUIRE((p.has_seqused_ori_kv != 0) == (len->seqused_ori_kv != nullptr),
          "has_seqused_ori_kv must match");
  REQUIRE((p.has_seqused_cmp_kv != 0) == (len->seqused_cmp_kv != nullptr),
          "has_seqused_cmp_kv must match");
  REQUIRE((p.has_cmp_residual_kv != 0) == (len->cmp_residual_kv != nullptr),
          "has_cmp_residual_kv must match");
  REQUIRE(!(p.has_seqused_cmp_kv && !p.has_cmp_kv), "seqused_cmp_kv given without cmp_kv");
  sfmla::PlanArgs a;
  a.p = p;
  a.len = *len;
  a.meta = metadata;
  a.fingerprint = fingerprint(p);
  a.max_splits = max_splits(p);
  a.split_rows = split_rows(p);
  a.split_rows_long = std::max(a.split_rows, sfmla::kMaxSplitRows);
  a.tq = query_tile(p);
  a.tile_auto = p.query_tile > 1 ? 0 : 1;
  a.tile_min_queries = p.query_tile > 1 ? 1 : sfmla::kMinTileQueries;
  a.tile_bound = (int32_t)tile_bound(p);
  a.tile_off = (int64_t)tile_off(p);
  hipError_t e = sfmla::launch_plan(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SFMLA_ERR_LAUNCH, "plan launch: %s", hipGetErrorString(e));
  return ok();
}

sfmla_status sfmla_forward_static_workspace(const sfmla_params* params, const sfmla_tensors* t,
                                            int32_t* metadata, size_t n_ints,
                                            float softmax_scale, void* stream) {
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  const size_t need = workspace_bytes(*params);
  if (need > sfmla::kStaticWorkspaceBytes)
    return fail(SFMLA_ERR_BUFFER_TOO_SMALL,
                "these parameters need %zu bytes of split workspace; the library-owned one "
                "holds %zu (use sfmla_forward with a caller workspace)",
                need, (size_t)sfmla::kStaticWorkspaceBytes);
  void* ws = nullptr;
  if (need) {
    const hipError_t e = sfmla::static_workspace(&ws);
    if (e != hipSuccess)
      return fail(SFMLA_ERR_LAUNCH, "library workspace address: %s", hipGetErrorString(e));
  }
  return sfmla_forward(params, t, metadata, n_ints, softmax_scale, ws, need ? need : 0, stream);
}

sfmla_status sfmla_forward(const sfmla_params* params, const sfmla_tensors* t,
                           int32_t* metadata, size_t n_ints, float softmax_scale,
                           void* workspace, size_t ws_bytes, void* stream) {
  // events asked for by sfmla_time_next_forward serve this call only
  const hipEvent_t t0 = (hipEvent_t)g_time_start, t1 = (hipEvent_t)g_time_stop;
  g_time_start = g_time_stop = nullptr;
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  const sfmla_params& p = *params;
  sfmla::FwdArgs a;
  s = fill_fwd_args(p, t, metadata, n_ints, softmax_scale, &a);
  if (s != SFMLA_OK) return s;
  const size_t need = workspace_bytes(p);
  if (need) {
    if (!workspace || ws_bytes < need)
      return fail(SFMLA_ERR_BUFFER_TOO_SMALL, "workspace holds %zu bytes, needs %zu", ws_bytes,
                  need);
    REQUIRE(((uintptr_t)workspace & 255) == 0, "workspace must be 256-byte aligned");
    const WsLayout L = workspace_layout(p);
    a.ws_ob = (uint16_t*)workspace;
    a.ws_lse = (float*)((char*)workspace + L.o_bytes);
  }
  a.counters = metadata + sfmla::kHeaderInts + (size_t)sfmla::kRecInts * p.q_t;
  const int dqk = 512 + p.rope_head_dim;
  const int vmode = p.has_separate_v ? 1 : 0;
  const int tq = query_tile(p);
  if (tq > 1) {
    a.tq = tq;
    a.nb = (p.num_heads_q + 15) / 16;
    a.tile_off = (int64_t)tile_off(p);
    a.tile_units = (int32_t)tile_bound(p);
    hipError_t e = sfmla::launch_forward_tiled(a, dqk, vmode, p.kv_dtype, (hipStream_t)stream,
                                               t0, t1);
    if (e != hipSuccess) return fail(SFMLA_ERR_LAUNCH, "forward launch: %s", hipGetErrorString(e));
    return ok();
  }
  int nw, groups, bpg;
  bool pair = false;
  choose_groups(p, &nw, &groups, &bpg, &pair);
  a.bpg = bpg;
  // the owned split merge waits at most this long for the row's other
  // splits (when the launch's workgroups are all resident at once)
  const int merge_wait_us = p.merge_wait_us == 0 ? kMergeWaitUs : std::max(0, p.merge_wait_us);
  hipError_t e = sfmla::launch_forward(a, nw, pair, dqk, vmode, p.kv_dtype, groups,
                                       merge_wait_us, (hipStream_t)stream, t0, t1);
  if (e != hipSuccess) return fail(SFMLA_ERR_LAUNCH, "forward launch: %s", hipGetErrorString(e));
  return ok();
}

sfmla_status sfmla_combine(int32_t n_parts, const float* part_o, const float* part_lse,
                           const float* sinks, void* out, float* lse_out, int32_t rows,
                           int32_t heads, int32_t dv, void* stream) {
  REQUIRE(n_parts >= 1, "n_parts must be >= 1");
  REQUIRE(rows >= 1 && heads >= 1, "rows and heads must be >= 1");
  REQUIRE(dv >= 4 && dv <= 4096 && dv % 4 == 0, "dv must be a multiple of 4 in 4..4096");
  REQUIRE(part_o && aligned16(part_o) && part_lse, "part_o (16-byte aligned) and part_lse are required");
  REQUIRE(out && ((uintptr_t)out & 7) == 0, "out must be an 8-byte aligned device pointer");
  REQUIRE(heads <= 65535, "heads must be <= 65535");
  REQUIRE((int64_t)n_parts * rows * heads * dv < ((int64_t)1 << 40), "partials too large");
  sfmla::CombineArgs c;
  std::memset(&c, 0, sizeof c);
  c.rows = rows;
  c.heads = heads;
  c.dv = dv;
  c.n_parts = n_parts;
  c.o_part_stride = (int64_t)rows * heads * dv;
  c.o_row_stride = (int64_t)heads * dv;
  c.lse_part_stride = (int64_t)rows * heads;
  c.lse_row_stride = heads;
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.sinks = sinks;
  c.out = (uint16_t*)out;
  c.lse_out = lse_out;
  hipError_t e = sfmla::launch_combine(c, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SFMLA_ERR_LAUNCH, "combine launch: %s", hipGetErrorString(e));
  return ok();
}

sfmla_status sfmla_debug_resolve(const sfmla_params* params, const sfmla_tensors* t,
                                 const int32_t* metadata, size_t n_ints, int64_t* rows_out,
                                 int32_t max_rows, int32_t* counts_out, void* stream) {
  sfmla_status s = validate(params);
  if (s != SFMLA_OK) return s;
  sfmla::FwdArgs a;
  s = fill_fwd_args(*params, t, metadata, n_ints, 1.0f, &a);
  if (s != SFMLA_OK) return s;
  REQUIRE(rows_out && counts_out && max_rows > 0, "rows_out, counts_out and max_rows > 0 required");
  a.dbg_rows = rows_out;
  a.dbg_counts = counts_out;
  a.dbg_max_rows = max_rows;
  hipError_t e = sfmla::launch_debug_resolve(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(SFMLA_ERR_LAUNCH, "resolve launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
