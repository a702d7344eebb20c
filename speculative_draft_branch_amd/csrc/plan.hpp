// Execution plan of one packed batch: host-side structure plus the layout of
// the metadata blob the kernels read from the workspace.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "branch_attn.h"

namespace ba {

// Rows per query tile in MFMA rows (base rows x q heads of one kv group).
constexpr int kTileRows = 128;
// Keys per backward key tile: 256, except for the bf16 d = 64 dK/dV kernel,
// whose twelve waves of 32 keys (three per SIMD) take 384.
constexpr int kBwdKeys = 256;
constexpr int kBwdKeys64 = 384;
inline int bwd_keys(int dtype, int d) { return dtype == BA_BF16 && d == 64 ? kBwdKeys64 : kBwdKeys; }
// Per-query-tile block of row ends the dq kernel stages: 128 prefix ends,
// then the tile's smallest end, largest end and valid MFMA rows (padded to 3 x 64
// words for whole-wave LDS copies).
constexpr int kTileMetaWords = 192;
// Longest branch the branch-local kernels handle.
constexpr int kMaxBranch = 32;

// One forward/backward query tile: rows [row_begin, row_begin + nrows) of the
// tile row list, all in one sequence, sorted by prefix end.
struct QTile {
  int32_t row_begin;  // index into tile_row_id / tile_row_end
  int32_t nrows;      // base rows used (<= rows_per_tile)
  int32_t kv_lo;      // first main key: the sequence start
  int32_t end_min;    // smallest prefix end (inclusive) of the tile's rows
  int32_t end_max;    // largest prefix end (inclusive)
  int32_t seq;        // sequence index
  int32_t pad0, pad1;
};
static_assert(sizeof(QTile) == 32, "QTile layout");

// One backward key tile: main keys [key_lo, key_hi) of one sequence and the
// range of query tiles (in sequence order) whose rows may see them.
struct KTile {
  int32_t key_lo, key_hi;
  int32_t qt_begin, qt_end;
};
static_assert(sizeof(KTile) == 16, "KTile layout");

// Byte offsets of each array inside the device metadata blob.
struct BlobLayout {
  size_t group_heads;   // int32 [Hkv * G]: q heads of each kv group
  size_t qtiles;        // QTile [n_qtiles], sequence order
  size_t fwd_order;     // int32 [n_qtiles]: longest-first launch order
  size_t fwd_pairs;     // int32 [n_fwd_pairs][2]: tiles sharing a forward workgroup (-1 = none), longest first
  size_t fwd_triples;   // int32 [n_fwd_triples][3]: the same in threes (the d = 64 forward), longest first
  size_t tile_row_id;   // int32 [n_qtiles * rows_per_tile]: combined row id, -1 = padding
  size_t tile_row_end;  // int32 [n_qtiles * rows_per_tile]: prefix end of that row
  size_t row_lo;        // int32 [Nq + Rb]: first visible main key of each combined row
  size_t row_hi;        // int32 [Nq + Rb]: last visible main key (inclusive)
  size_t cu_branch;     // int32 [A + 1]
  size_t mode;          // int32 [A]
  size_t ktiles;        // KTile [n_ktiles]
  size_t bwd_order;     // int32 [n_ktiles]: longest-first launch order
  size_t vt_tiles;      // int32 [n_vt_tiles][2]: main keys [lo, hi) of each transposed V tile (lo + 64 > hi allowed)
  size_t vt_base;       // int32 [S]: first transposed V tile of each sequence
  size_t brow_lo;       // int32 [Rb]: first branch key (branch row index) a branch row sees
  size_t brow_hi;       // int32 [Rb]: last branch key it sees (inclusive)
  size_t fwd_pair_bk;   // int32 [n_fwd_pairs][2]: branch keys [lo, hi) the rows of a forward pair see
  size_t fwd_triple_bk; // int32 [n_fwd_triples][2]: the same for the threes
  size_t fwd_unit_bt;   // int32 [units of the bf16 forward]: first branch V^T tile of each unit
  size_t vbt_start;     // int32 [n_vbt_tiles]: first branch key of each branch V^T tile
  size_t total;
};

}  // namespace ba

struct ba_plan {
  ba_dtype_t dtype;
  int32_t hq, hkv, d, G;
  float scale;
  int32_t S;
  int64_t N, Nq, A, Rb;
  std::vector<int32_t> kv_head_of, group_heads;
  std::vector<int32_t> cu, q_pos, anchors, cu_branch;
  std::vector<uint8_t> mode;
  int32_t rows_per_tile;  // base rows per query tile
  int32_t max_branch;     // longest branch (rows of one anchor)
  int32_t n_qtiles, n_ktiles, n_fwd_pairs, n_vt_tiles, n_fwd_triples;
  int32_t n_vbt_tiles;  // 64-key transposed tiles of the branch V (bf16 forward), per unit from its first branch key
  int64_t pairs[3];
  ba::BlobLayout layout;
  std::vector<uint8_t> blob;  // host copy of the device metadata
  size_t ws_split, ws_fwd, ws_bwd;
  // workspace regions (byte offsets)
  size_t off_queue;  // int32 [2][Hkv]: work counters of the forward or dQ kernel, then of the dK/dV kernel
  size_t off_vt;                                          // forward, bf16: V^T tiles [n_vt_tiles][Hkv][d][64]
  size_t off_vbt;                                         // forward, bf16: branch V^T tiles [n_vbt_tiles][Hkv][d][64]
  size_t off_o_pre, off_lse_pre, off_o_loc, off_lse_loc;  // forward
  size_t off_delta, off_dq_acc;                           // backward
  // backward, query-tile order per kv head: Q and dO rows [n_qtiles][Hkv][128][d],
  // LSE*log2(e) and D [n_qtiles][Hkv][128], row-end blocks [n_qtiles][kTileMetaWords]
  size_t off_qt, off_dot, off_lt, off_dt, off_et;
  // backward, bf16, when some key tile's query range is split in two: float32
  // dK and dV accumulators [N][Hkv][d] each (0 when nothing is split)
  size_t off_dkv_acc;
  bool dkv_split;
};

namespace ba {
ba_status_t set_error(ba_status_t st, const std::string &msg);
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace ba
