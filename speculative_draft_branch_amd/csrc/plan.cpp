// Plan construction: validation, per-row key ranges, query tiles, backward key
// tiles and longest-first launch orders. Pure host code.
//
// Which keys a row sees (rcap.io explainer, paragraph on branch attention under
// context parallelism; cere-bro wiki, "Mechanism"): a main row at packed
// position t sees main keys cu[s]..t of its sequence s; every query of a branch
// anchored at a sees main keys cu[s]..a. Rows whose prefix end is the same see
// the same main keys, so the plan groups rows by prefix end: the main row at a
// position, the branch rows anchored there and the q heads of one kv group all
// share one K/V stream.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <numeric>

#include "plan.hpp"

namespace ba {

namespace {
thread_local std::string g_last_error;
}

ba_status_t set_error(ba_status_t st, const std::string &msg) {
  g_last_error = msg;
  return st;
}

const char *last_error() { return g_last_error.c_str(); }

}  // namespace ba

using namespace ba;

namespace {

ba_status_t validate_and_copy(const ba_problem_t *p, ba_plan *pl) {
  if (!p) return set_error(BA_EINVAL, "problem is NULL");
  if (p->dtype != BA_F32 && p->dtype != BA_BF16) return set_error(BA_EINVAL, "dtype must be BA_F32 or BA_BF16");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1) return set_error(BA_EINVAL, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return set_error(BA_EINVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim != 64 && p->head_dim != 128)
    return set_error(BA_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (!(p->softmax_scale >= 0.0f) || std::isinf(p->softmax_scale))
    return set_error(BA_EINVAL, "softmax_scale must be finite and >= 0");
  pl->dtype = p->dtype;
  pl->hq = p->num_q_heads;
  pl->hkv = p->num_kv_heads;
  pl->d = p->head_dim;
  pl->G = pl->hq / pl->hkv;
  if (pl->G > kTileRows) return set_error(BA_EUNSUPPORTED, "more than 128 q heads per kv head");
  pl->scale = p->softmax_scale > 0.0f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);

  pl->kv_head_of.resize(pl->hq);
  for (int h = 0; h < pl->hq; ++h) pl->kv_head_of[h] = p->kv_head_of ? p->kv_head_of[h] : h / pl->G;
  pl->group_heads.assign((size_t)pl->hkv * pl->G, -1);
  std::vector<int> fill(pl->hkv, 0);
  for (int h = 0; h < pl->hq; ++h) {
    int g = pl->kv_head_of[h];
    if (g < 0 || g >= pl->hkv) return set_error(BA_EINVAL, "kv_head_of entry out of range");
    if (fill[g] >= pl->G) return set_error(BA_EINVAL, "kv_head_of must give every kv head Hq/Hkv q heads");
    pl->group_heads[(size_t)g * pl->G + fill[g]++] = h;
  }

  if (p->num_seqs < 1 || !p->cu_seqlens) return set_error(BA_EINVAL, "need num_seqs >= 1 and cu_seqlens");
  pl->S = p->num_seqs;
  pl->cu.assign(p->cu_seqlens, p->cu_seqlens + pl->S + 1);
  if (pl->cu[0] != 0) return set_error(BA_EINVAL, "cu_seqlens[0] must be 0");
  for (int s = 0; s < pl->S; ++s)
    if (pl->cu[s + 1] < pl->cu[s]) return set_error(BA_EINVAL, "cu_seqlens must be non-decreasing");
  pl->N = pl->cu[pl->S];

  if (p->q_pos) {
    if (p->num_q < 0) return set_error(BA_EINVAL, "num_q must be >= 0");
    pl->q_pos.assign(p->q_pos, p->q_pos + p->num_q);
    for (int64_t i = 0; i < p->num_q; ++i) {
      if (pl->q_pos[i] < 0 || pl->q_pos[i] >= pl->N) return set_error(BA_EINVAL, "q_pos out of [0, N)");
      if (i && pl->q_pos[i] <= pl->q_pos[i - 1]) return set_error(BA_EINVAL, "q_pos must be strictly increasing");
    }
  } else {
    pl->q_pos.resize(pl->N);
    std::iota(pl->q_pos.begin(), pl->q_pos.end(), 0);
  }
  pl->Nq = (int64_t)pl->q_pos.size();

  if (p->num_anchors < 0) return set_error(BA_EINVAL, "num_anchors must be >= 0");
  pl->A = p->num_anchors;
  if (pl->A > 0 && !p->anchors) return set_error(BA_EINVAL, "anchors is NULL");
  pl->anchors.assign(p->anchors, p->anchors + pl->A);
  for (int64_t m = 0; m < pl->A; ++m) {
    if (pl->anchors[m] < 0 || pl->anchors[m] >= pl->N) return set_error(BA_EINVAL, "anchor out of [0, N)");
    if (m && pl->anchors[m] <= pl->anchors[m - 1]) return set_error(BA_EINVAL, "anchors must be strictly increasing");
  }
  pl->cu_branch.resize(pl->A + 1);
  if (p->cu_branch) {
    pl->cu_branch.assign(p->cu_branch, p->cu_branch + pl->A + 1);
    if (pl->cu_branch[0] != 0) return set_error(BA_EINVAL, "cu_branch[0] must be 0");
  } else {
    if (p->branch_len < 0) return set_error(BA_EINVAL, "branch_len must be >= 0");
    for (int64_t m = 0; m <= pl->A; ++m) {
      int64_t v = m * (int64_t)p->branch_len;
      if (v > INT32_MAX) return set_error(BA_EINVAL, "too many branch rows");
      pl->cu_branch[m] = (int32_t)v;
    }
  }
  pl->max_branch = 0;
  for (int64_t m = 0; m < pl->A; ++m) {
    int32_t L = pl->cu_branch[m + 1] - pl->cu_branch[m];
    if (L < 0) return set_error(BA_EINVAL, "cu_branch must be non-decreasing");
    if (L > kMaxBranch) return set_error(BA_EINVAL, "a branch has more than 32 rows");
    pl->max_branch = std::max(pl->max_branch, L);
  }
  pl->Rb = pl->cu_branch[pl->A];
  pl->mode.resize(pl->A);
  for (int64_t m = 0; m < pl->A; ++m) {
    int md = p->mode ? (int)p->mode[m] : (int)p->uniform_mode;
    if (md != BA_TTT && md != BA_BLOCK) return set_error(BA_EINVAL, "mode must be BA_TTT or BA_BLOCK");
    pl->mode[m] = (uint8_t)md;
  }
  if (pl->Nq + pl->Rb > INT32_MAX / 2) return set_error(BA_EINVAL, "too many rows");
  return BA_OK;
}

template <class T>
size_t put(std::vector<uint8_t> &blob, size_t &cur, const std::vector<T> &v) {
  size_t off = cur;
  size_t bytes = v.size() * sizeof(T);
  cur = align_up(cur + bytes, 256);
  if (blob.size() < cur) blob.resize(cur, 0);
  if (bytes) std::memcpy(blob.data() + off, v.data(), bytes);
  return off;
}

void build(ba_plan *pl) {
  const int64_t Nq = pl->Nq, Rb = pl->Rb, R = Nq + Rb;
  // Per combined row: visible main key range [lo, hi].
  std::vector<int32_t> row_lo(R), row_hi(R);
  auto seq_of = [&](int32_t pos) {
    return (int32_t)(std::upper_bound(pl->cu.begin(), pl->cu.end(), pos) - pl->cu.begin() - 1);
  };
  for (int64_t i = 0; i < Nq; ++i) {
    int32_t t = pl->q_pos[i];
    row_lo[i] = pl->cu[seq_of(t)];
    row_hi[i] = t;
  }
  for (int64_t m = 0; m < pl->A; ++m) {
    int32_t a = pl->anchors[m], lo = pl->cu[seq_of(a)];
    for (int32_t b = pl->cu_branch[m]; b < pl->cu_branch[m + 1]; ++b) {
      row_lo[Nq + b] = lo;
      row_hi[Nq + b] = a;
    }
  }
  // Pair counts per q head.
  pl->pairs[0] = pl->pairs[1] = pl->pairs[2] = 0;
  for (int64_t i = 0; i < Nq; ++i) pl->pairs[0] += (int64_t)row_hi[i] - row_lo[i] + 1;
  for (int64_t b = 0; b < Rb; ++b) pl->pairs[1] += (int64_t)row_hi[Nq + b] - row_lo[Nq + b] + 1;
  for (int64_t m = 0; m < pl->A; ++m) {
    int64_t L = pl->cu_branch[m + 1] - pl->cu_branch[m];
    pl->pairs[2] += pl->mode[m] == BA_BLOCK ? L * L : L * (L + 1) / 2;
  }

  // Query tiles: per sequence, rows sorted by prefix end (main row first on a tie).
  const int RT = std::max(1, kTileRows / pl->G);
  pl->rows_per_tile = RT;
  std::vector<QTile> qt;
  std::vector<int32_t> trow_id, trow_end;
  std::vector<int32_t> seq_qt_begin(pl->S + 1, 0);
  int64_t qi = 0, mi = 0;
  for (int32_t s = 0; s < pl->S; ++s) {
    seq_qt_begin[s] = (int32_t)qt.size();
    const int32_t hi_pos = pl->cu[s + 1];
    std::vector<int32_t> rows;
    while (qi < Nq || mi < pl->A) {
      bool take_main = qi < Nq && pl->q_pos[qi] < hi_pos &&
                       (mi >= pl->A || pl->anchors[mi] >= hi_pos || pl->q_pos[qi] <= pl->anchors[mi]);
      if (take_main) {
        rows.push_back((int32_t)qi++);
      } else if (mi < pl->A && pl->anchors[mi] < hi_pos) {
        for (int32_t b = pl->cu_branch[mi]; b < pl->cu_branch[mi + 1]; ++b) rows.push_back((int32_t)(Nq + b));
        ++mi;
      } else {
        break;
      }
    }
    for (size_t r0 = 0; r0 < rows.size(); r0 += RT) {
      size_t n = std::min(rows.size() - r0, (size_t)RT);
      QTile t{};
      t.row_begin = (int32_t)trow_id.size();
      t.nrows = (int32_t)n;
      t.kv_lo = pl->cu[s];
      t.end_min = row_hi[rows[r0]];
      t.end_max = row_hi[rows[r0 + n - 1]];
      t.seq = s;
      for (size_t i = 0; i < (size_t)RT; ++i) {
        bool ok = i < n;
        trow_id.push_back(ok ? rows[r0 + i] : -1);
        trow_end.push_back(ok ? row_hi[rows[r0 + i]] : -1);
      }
      qt.push_back(t);
    }
  }
  seq_qt_begin[pl->S] = (int32_t)qt.size();
  pl->n_qtiles = (int32_t)qt.size();

  std::vector<int32_t> fwd_order(qt.size());
  std::iota(fwd_order.begin(), fwd_order.end(), 0);
  std::stable_sort(fwd_order.begin(), fwd_order.end(), [&](int32_t a, int32_t b) {
    int64_t ca = (int64_t)(qt[a].end_max - qt[a].kv_lo + 1) * qt[a].nrows;
    int64_t cb = (int64_t)(qt[b].end_max - qt[b].kv_lo + 1) * qt[b].nrows;
    return ca > cb;
  });

  // Forward workgroups take U consecutive tiles of one sequence (their prefix
  // ends are adjacent in the sorted order, so they share almost every K/V tile;
  // -1 where the sequence runs out); cost is the longest key range among them.
  // Units are listed longest first. Pairs serve the d = 128 forward and the dQ
  // kernel, threes the d = 64 forward.
  auto fwd_units = [&](int32_t U, int32_t &n_units) {
    std::vector<int32_t> units;
    std::vector<int64_t> cost;
    for (int32_t s = 0; s < pl->S; ++s) {
      for (int32_t a = seq_qt_begin[s]; a < seq_qt_begin[s + 1]; a += U) {
        int32_t e = qt[a].end_max;
        for (int32_t u = 0; u < U; ++u) {
          const int32_t t = a + u < seq_qt_begin[s + 1] ? a + u : -1;
          units.push_back(t);
          if (t >= 0) e = std::max(e, qt[t].end_max);
        }
        cost.push_back((int64_t)e - qt[a].kv_lo + 1);
      }
    }
    n_units = (int32_t)cost.size();
    std::vector<int32_t> ord(cost.size());
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return cost[x] > cost[y]; });
    std::vector<int32_t> sorted(units.size());
    for (size_t i = 0; i < ord.size(); ++i)
      for (int32_t u = 0; u < U; ++u) sorted[U * i + u] = units[U * (size_t)ord[i] + u];
    return sorted;
  };
  std::vector<int32_t> fwd_pairs = fwd_units(2, pl->n_fwd_pairs);
  std::vector<int32_t> fwd_triples = fwd_units(3, pl->n_fwd_triples);

  // Branch keys each branch row sees (branch row indices, inclusive): from its
  // anchor's first branch row to itself (TTT) or to the anchor's last (block).
  std::vector<int32_t> brow_lo(Rb), brow_hi(Rb);
  for (int64_t m = 0; m < pl->A; ++m)
    for (int32_t b = pl->cu_branch[m]; b < pl->cu_branch[m + 1]; ++b) {
      brow_lo[b] = pl->cu_branch[m];
      brow_hi[b] = pl->mode[m] == BA_BLOCK ? pl->cu_branch[m + 1] - 1 : b;
    }
  // The branch keys a forward unit's rows see, [lo, hi) (lo = hi = 0: none).
  // Branch rows of consecutive tiles belong to consecutive anchors, so the
  // range is contiguous and spans little more than the unit's branch rows.
  auto unit_branch_keys = [&](const std::vector<int32_t> &units, int32_t U) {
    std::vector<int32_t> out(2 * (units.size() / U), 0);
    for (size_t i = 0; i < units.size() / U; ++i) {
      int32_t lo = INT32_MAX, hi = 0;
      for (int32_t u = 0; u < U; ++u) {
        const int32_t t = units[U * i + u];
        if (t < 0) continue;
        for (int32_t r = 0; r < qt[t].nrows; ++r) {
          const int32_t row = trow_id[(size_t)qt[t].row_begin + r];
          if (row < Nq) continue;
          lo = std::min(lo, brow_lo[row - Nq]);
          hi = std::max(hi, brow_hi[row - Nq] + 1);
        }
      }
      if (hi > 0) {
        out[2 * i] = lo;
        out[2 * i + 1] = hi;
      }
    }
    return out;
  };
  std::vector<int32_t> fwd_pair_bk = unit_branch_keys(fwd_pairs, 2);
  std::vector<int32_t> fwd_triple_bk = unit_branch_keys(fwd_triples, 3);
  // Branch V^T tiles of the bf16 forward (pairs at d = 128, threes at d = 64):
  // each unit's branch keys in 64-key tiles from its first one, so a unit
  // whose branch keys fit in 64 takes one tile wherever they start.
  const std::vector<int32_t> &unit_bk = pl->d == 64 ? fwd_triple_bk : fwd_pair_bk;
  std::vector<int32_t> fwd_unit_bt(unit_bk.size() / 2), vbt_start;
  for (size_t u = 0; u < fwd_unit_bt.size(); ++u) {
    fwd_unit_bt[u] = (int32_t)vbt_start.size();
    for (int32_t b = unit_bk[2 * u]; b < unit_bk[2 * u + 1]; b += 64) vbt_start.push_back(b);
  }
  pl->n_vbt_tiles = (int32_t)vbt_start.size();

  // Backward key tiles: per sequence, bwd_keys() main keys each; the query
  // tiles that see a key tile are the sequence's tiles whose largest end
  // reaches it.
  const int32_t bk = bwd_keys(pl->dtype, pl->d);
  std::vector<KTile> kt;
  std::vector<int64_t> kt_cost;
  std::vector<int64_t> rows_prefix(qt.size() + 1, 0);
  for (size_t i = 0; i < qt.size(); ++i) rows_prefix[i + 1] = rows_prefix[i] + qt[i].nrows;
  for (int32_t s = 0; s < pl->S; ++s) {
    int32_t b0 = seq_qt_begin[s], b1 = seq_qt_begin[s + 1];
    for (int32_t k0 = pl->cu[s]; k0 < pl->cu[s + 1]; k0 += bk) {
      KTile t{};
      t.key_lo = k0;
      t.key_hi = std::min(k0 + bk, pl->cu[s + 1]);
      int32_t lo = b0, hi = b1;  // first tile with end_max >= k0
      while (lo < hi) {
        int32_t mid = (lo + hi) / 2;
        if (qt[mid].end_max >= k0) hi = mid; else lo = mid + 1;
      }
      t.qt_begin = lo;
      t.qt_end = b1;
      kt.push_back(t);
      kt_cost.push_back(rows_prefix[b1] - rows_prefix[lo]);
    }
  }
  // A key tile whose query range costs more than a compute unit's share of the
  // whole (Hkv workgroups per tile over 256 compute units) would set the
  // kernel's end by itself: its range is split in two halves of equal rows,
  // and then every dK/dV workgroup adds its float32 result into a zeroed
  // accumulator (one add for a whole tile, two for a split one, exact in either
  // order, so the result stays deterministic) that one pass converts to bf16.
  pl->dkv_split = false;
  if (pl->dtype == BA_BF16 && !kt.empty()) {
    int64_t total = 0;
    for (int64_t c : kt_cost) total += c;
    const double share = (double)total * pl->hkv / 256.0;
    std::vector<KTile> kt2;
    std::vector<int64_t> cost2;
    for (size_t i = 0; i < kt.size(); ++i) {
      const KTile t = kt[i];
      if ((double)kt_cost[i] > share && t.qt_end - t.qt_begin >= 2) {
        const int64_t half = (rows_prefix[t.qt_begin] + rows_prefix[t.qt_end]) / 2;
        int32_t mid = t.qt_begin + 1;
        while (mid < t.qt_end - 1 && rows_prefix[mid] < half) ++mid;
        KTile a = t, b = t;
        a.qt_end = mid;
        b.qt_begin = mid;
        kt2.push_back(a);
        cost2.push_back(rows_prefix[mid] - rows_prefix[t.qt_begin]);
        kt2.push_back(b);
        cost2.push_back(rows_prefix[t.qt_end] - rows_prefix[mid]);
        pl->dkv_split = true;
      } else {
        kt2.push_back(t);
        cost2.push_back(kt_cost[i]);
      }
    }
    kt.swap(kt2);
    kt_cost.swap(cost2);
  }
  pl->n_ktiles = (int32_t)kt.size();
  std::vector<int32_t> bwd_order(kt.size());
  std::iota(bwd_order.begin(), bwd_order.end(), 0);
  std::stable_sort(bwd_order.begin(), bwd_order.end(),
                   [&](int32_t a, int32_t b) { return kt_cost[a] > kt_cost[b]; });

  // Transposed V tiles for the bf16 forward: 64 keys each, aligned to each
  // sequence's start like the forward's K/V tiles.
  std::vector<int32_t> vt_tiles, vt_base(pl->S, 0);
  for (int32_t s = 0; s < pl->S; ++s) {
    vt_base[s] = (int32_t)(vt_tiles.size() / 2);
    for (int32_t k0 = pl->cu[s]; k0 < pl->cu[s + 1]; k0 += 64) {
      vt_tiles.push_back(k0);
      vt_tiles.push_back(pl->cu[s + 1]);
    }
  }
  pl->n_vt_tiles = (int32_t)(vt_tiles.size() / 2);

  // Device metadata blob.
  std::vector<int32_t> mode32(pl->mode.begin(), pl->mode.end());
  std::vector<uint8_t> &blob = pl->blob;
  blob.clear();
  size_t cur = 0;
  BlobLayout &L = pl->layout;
  L.group_heads = put(blob, cur, pl->group_heads);
  L.qtiles = put(blob, cur, qt);
  L.fwd_order = put(blob, cur, fwd_order);
  L.fwd_pairs = put(blob, cur, fwd_pairs);
  L.fwd_triples = put(blob, cur, fwd_triples);
  L.tile_row_id = put(blob, cur, trow_id);
  L.tile_row_end = put(blob, cur, trow_end);
  L.row_lo = put(blob, cur, row_lo);
  L.row_hi = put(blob, cur, row_hi);
  L.cu_branch = put(blob, cur, pl->cu_branch);
  L.mode = put(blob, cur, mode32);
  L.ktiles = put(blob, cur, kt);
  L.bwd_order = put(blob, cur, bwd_order);
  L.vt_tiles = put(blob, cur, vt_tiles);
  L.vt_base = put(blob, cur, vt_base);
  L.brow_lo = put(blob, cur, brow_lo);
  L.brow_hi = put(blob, cur, brow_hi);
  L.fwd_pair_bk = put(blob, cur, fwd_pair_bk);
  L.fwd_triple_bk = put(blob, cur, fwd_triple_bk);
  L.fwd_unit_bt = put(blob, cur, fwd_unit_bt);
  L.vbt_start = put(blob, cur, vbt_start);
  L.total = cur;
  blob.resize(std::max<size_t>(cur, 256));

  // Workspace layouts.
  const size_t f32 = sizeof(float);
  size_t base = align_up(blob.size(), 256);
  pl->off_queue = base;
  base += align_up((size_t)2 * pl->hkv * sizeof(int32_t), 256);
  pl->off_vt = base;
  const size_t vt_bytes =
      pl->dtype == BA_BF16 ? align_up((size_t)pl->n_vt_tiles * pl->hkv * pl->d * 64 * sizeof(uint16_t), 256) : 0;
  pl->ws_split = base + vt_bytes;
  // bf16 forward: the branch V^T tiles follow the main ones (the split-path
  // entry points do not use them)
  pl->off_vbt = pl->ws_split;
  const size_t vbt_bytes =
      pl->dtype == BA_BF16 ? align_up((size_t)pl->n_vbt_tiles * pl->hkv * pl->d * 64 * sizeof(uint16_t), 256) : 0;
  size_t o_bytes = align_up((size_t)Rb * pl->hq * pl->d * f32, 256);
  size_t l_bytes = align_up((size_t)Rb * pl->hq * f32, 256);
  pl->off_o_pre = pl->ws_split;
  pl->off_lse_pre = pl->off_o_pre + o_bytes;
  pl->off_o_loc = pl->off_lse_pre + l_bytes;
  pl->off_lse_loc = pl->off_o_loc + o_bytes;
  // bf16: the main kernel takes the branch keys as its last key tiles and
  // writes every row's final output, so the forward needs no partials.
  pl->ws_fwd = pl->dtype == BA_BF16 ? pl->off_vbt + vbt_bytes : pl->off_lse_loc + l_bytes;
  pl->off_delta = base;
  size_t d_bytes = align_up((size_t)R * pl->hq * f32, 256);
  pl->off_dq_acc = pl->off_delta + d_bytes;
  // float32 dQ accumulator: float32 plans only (the bf16 dq kernel sums a row's
  // whole dQ in registers and writes it once)
  size_t cur_b = pl->off_dq_acc + (pl->dtype == BA_F32 ? align_up((size_t)R * pl->hq * pl->d * f32, 256) : 0);
  const size_t tiles_g = (size_t)pl->n_qtiles * pl->hkv;
  if (pl->dtype == BA_BF16) {
    const size_t row_bytes = align_up(tiles_g * kTileRows * pl->d * 2, 256);
    const size_t scal_bytes = align_up(tiles_g * kTileRows * f32, 256);
    pl->off_qt = cur_b;
    pl->off_dot = pl->off_qt + row_bytes;
    pl->off_lt = pl->off_dot + row_bytes;
    pl->off_dt = pl->off_lt + scal_bytes;
    pl->off_et = pl->off_dt + scal_bytes;
    cur_b = pl->off_et + align_up((size_t)pl->n_qtiles * kTileMetaWords * 4, 256);
  } else {
    pl->off_qt = pl->off_dot = pl->off_lt = pl->off_dt = pl->off_et = cur_b;
  }
  pl->off_dkv_acc = 0;
  if (pl->dkv_split) {
    pl->off_dkv_acc = cur_b;
    cur_b += 2 * align_up((size_t)pl->N * pl->hkv * pl->d * f32, 256);
  }
  pl->ws_bwd = cur_b;
}

}  // namespace

extern "C" {

ba_status_t ba_plan_create(const ba_problem_t *problem, ba_plan_t **out) {
  if (!out) return set_error(BA_EINVAL, "out is NULL");
  *out = nullptr;
  ba_plan *pl = new (std::nothrow) ba_plan();
  if (!pl) return set_error(BA_EINVAL, "out of host memory");
  ba_status_t st;
  try {
    st = validate_and_copy(problem, pl);
    if (st == BA_OK) build(pl);
  } catch (const std::bad_alloc &) {
    st = set_error(BA_EINVAL, "out of host memory while building the plan");
  }
  if (st != BA_OK) {
    delete pl;
    return st;
  }
  *out = pl;
  return BA_OK;
}

void ba_plan_destroy(ba_plan_t *plan) { delete plan; }

size_t ba_workspace_bytes(const ba_plan_t *plan, int pass) {
  if (!plan) return 0;
  switch (pass) {
    case 0: return plan->ws_fwd;
    case 1: return plan->ws_bwd;
    case 2: return plan->ws_split;
    default: return 0;
  }
}

ba_status_t ba_plan_sizes(const ba_plan_t *plan, int64_t out[5]) {
  if (!plan || !out) return set_error(BA_EINVAL, "NULL argument");
  out[0] = plan->N;
  out[1] = plan->Nq;
  out[2] = plan->Rb;
  out[3] = plan->n_qtiles;
  out[4] = plan->n_ktiles;
  return BA_OK;
}

ba_status_t ba_plan_pairs(const ba_plan_t *plan, int64_t out[3]) {
  if (!plan || !out) return set_error(BA_EINVAL, "NULL argument");
  for (int i = 0; i < 3; ++i) out[i] = plan->pairs[i];
  return BA_OK;
}

const char *ba_status_str(ba_status_t st) {
  switch (st) {
    case BA_OK: return "BA_OK";
    case BA_EINVAL: return "BA_EINVAL";
    case BA_EUNSUPPORTED: return "BA_EUNSUPPORTED";
    case BA_EWORKSPACE: return "BA_EWORKSPACE";
    case BA_EHIP: return "BA_EHIP";
  }
  return "unknown status";
}

const char *ba_last_error(void) { return ba::last_error(); }

int ba_abi_version(void) { return BA_ABI_VERSION; }

}  // extern "C"
