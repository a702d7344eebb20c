// Main-sequence backward on bf16 MFMA (gfx950): gradients of every row's
// attention over its causal main prefix, taken through the row's final (merged)
// LSE, so the log-sum-exp merge needs no backward of its own:
//   P = exp(S - LSE),  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// (Decomposition and merge: evolve.pub review, "Scope & Claims", section 3.2 and
// Eq. 2; the merged result is one softmax over the union of keys, rcap.io
// explainer, paragraph on branch attention under context parallelism.)
//
// Two kernels. Every gradient element has one writer, except in plans whose
// backward key tiles are split (small plans only): there each dK/dV element
// gets one or two float32 atomic adds into a zeroed accumulator, a sum of at
// most two terms, so the result does not depend on their order.
//  * dq: query-tile major, the forward's work unit (query tile x its key range,
//    64-key LDS tiles). S^T = K Q^T and dP^T = V dO^T put one query row on each
//    lane (dP^T starts from -D of that row, which the kernel takes from the
//    row's dO and O itself); dQ^T += K^T dS^T takes K through the transposing
//    LDS read and dS^T straight from registers. The unit's
//    branch keys (rows of kb, vb) follow its main keys as the last tiles, each
//    row masked to its own branch's keys, so every row's whole dQ is summed in
//    registers and written once, in bf16.
//  * dkdv: key-tile major: 256 main keys of one kv head (eight waves of 32
//    keys, sharing every staged query tile) against every query tile whose rows
//    may see them; each wave keeps its keys' dK, dV in registers across all
//    query tiles, written once, summed over the group's q heads. The dq kernel
//    stages Q scaled by scale * log2(e) and -LSE * log2(e), -D per row, so the
//    S and dP MFMAs (started from those) deliver the exponent of P and dP - D.
//    S = Q K^T puts the key on the lane, so P and dS are directly the A
//    operands of dV += P^T dO and dK += dS^T Q (dO and Q via the transposing
//    LDS read).
#include <climits>

#include "launch.hpp"

namespace ba {

// ---------------------------------------------------------------------------
namespace {

template <int HD>
struct DqState {
  static constexpr int KS = HD / 16;
  static constexpr int DT = HD / 32;
  bf16x8 qf[KS], of[KS];
  f32x16 acc[DT];
  float l2;
  f32x16 nd;  // -D of the lane's row in every element: the start value of dP^T
  int end, wmin;
  int grp, in_j, in_q, lane;
};

// One 64-key tile [k0, k0 + 64) of the wave's 32 rows against LDS tiles sK, sV.
constexpr int kDqRing = 4;
// K^T operands in flight in the dQ product pipeline.
constexpr int kDqKRing = 4;

// MASK: some key of the tile lies past some row's prefix end (a wave-uniform
// condition, so the unmasked tiles carry no per-element selects). BR: a tile
// of branch keys (branch row indices k0..); the row sees keys [br->x, br->y]
// of it, read from LDS where they are used (the kernel has no register to keep
// them in).
template <int HD, bool MASK, bool BR = false>
__device__ __forceinline__ void dq_tile(DqState<HD> &st, const bf16 *sK, const bf16 *sV, int k0, float sl2,
                                        const int2 *br = nullptr) {
  constexpr int KS = DqState<HD>::KS, DT = DqState<HD>::DT;
  const int lane = st.lane;
  // One 32-key block at a time: S^T, dP^T, dS^T, then its two dQ k-steps.
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 s = f32x16{}, dp = f32x16{};
    const int r = kb * 32 + (lane & 31);
    // S^T and dP^T as one software pipeline of (LDS read, MFMA) steps, step
    // 2ks reading K and 2ks+1 reading V, with kDqRing operands in flight; the
    // scheduling barriers keep the compiler from sinking each read next to its
    // MFMA and waiting for it there.
    auto rd = [&](int i) {
      const int off = r * HD + (((2 * (i >> 1) + (lane >> 5)) ^ swz<HD>(r)) << 3);
      return *reinterpret_cast<const bf16x8 *>(((i & 1) ? sV : sK) + off);
    };
    bf16x8 ring[kDqRing];
    __builtin_amdgcn_s_setprio(1);  // a wave in an MFMA stretch wins issue; the other wave's VALU fills in
#pragma unroll
    for (int i = 0; i < kDqRing; ++i) ring[i] = rd(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {
      if (i & 1) dp = mfma32(ring[i % kDqRing], st.of[i >> 1], i == 1 ? st.nd : dp);
      else s = mfma32(ring[i % kDqRing], st.qf[i >> 1], s);
      if (i + kDqRing < 2 * KS) ring[i % kDqRing] = rd(i + kDqRing);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    // dQ^T += K^T dS^T in 2*DT steps n = (h2, dt), K^T through the transposing
    // LDS read; slot 8*half + 4c + j <-> key 16kk + 8c + 4*half + j. Operands are
    // requested kDqKRing steps ahead of their MFMA.
    auto rdk = [&](int n) {
      const int kk = kb * 2 + n / DT, dt = n % DT;
      const int key0 = kk * 16 + 4 * (st.grp >> 1) + st.in_j;
      const int d = dt * 32 + (st.grp & 1) * 16 + 4 * st.in_q;
      return join(lds_read_tr(sK + lds_off<HD>(key0, d)), lds_read_tr(sK + lds_off<HD>(key0 + 8, d)));
    };
    bf16x8 db[2];  // dS^T operands of the block's two 16-key k-steps
    int2 bkr = {0, 0};
    if constexpr (BR) {
      const int2 *bp = br;
      asm volatile("" : "+v"(bp));  // read where used, not held across the tile
      bkr = *bp;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = fast_exp2(fmaf(s[i], sl2, -st.l2));
      if constexpr (BR) {
        const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (key < bkr.x || key > bkr.y) p = 0.0f;
      } else if constexpr (MASK) {
        const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (key > st.end) p = 0.0f;
      }
      db[i >> 3][i & 7] = (bf16)(p * dp[i]);
    }
    bf16x8 kr[kDqKRing];
#pragma unroll
    for (int i = 0; i < kDqKRing; ++i) kr[i] = rdk(i);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(2);  // above an S/dP stretch: a wave that has its products ready goes first
#pragma unroll
    for (int n = 0; n < 2 * DT; ++n) {
      st.acc[n % DT] = mfma32(kr[n % kDqKRing], db[n / DT], st.acc[n % DT]);
      if (n + kDqKRing < 2 * DT) kr[n % kDqKRing] = rdk(n + kDqKRing);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

}  // namespace

// NG: groups of four waves, one query tile each (the forward's work unit): two
// at d = 128, three at d = 64, where three waves per SIMD fit in the registers
// and the vector work of one wave's tile meets the MFMAs of two others.
// The unit's branch keys [bk_lo, bk_hi) (the forward's ranges) follow its main
// keys in 64-key tiles of kb, vb; dQ of every row goes to dq / dqb in bf16.
template <int HD, int NG>
__global__ __launch_bounds__(256 * NG, 1) void main_bwd_dq_bf16_kernel(Meta mt, const bf16 *__restrict__ q,
                                                               const bf16 *__restrict__ qb,
                                                               const bf16 *__restrict__ k,
                                                               const bf16 *__restrict__ v,
                                                               const bf16 *__restrict__ d_o,
                                                               const bf16 *__restrict__ d_ob,
                                                               const float *__restrict__ lse,
                                                               const float *__restrict__ lseb,
                                                               const bf16 *__restrict__ o,
                                                               const bf16 *__restrict__ ob,
                                                               const bf16 *__restrict__ kb,
                                                               const bf16 *__restrict__ vb,
                                                               bf16 *__restrict__ dq, bf16 *__restrict__ dqb,
                                                               BwdStage sg) {
  constexpr int BN = 64;
  constexpr int KS = HD / 16, DT = HD / 32;
  // K and V of one buffer share an array (one address for both reads).
  __shared__ __attribute__((aligned(16))) bf16 sKV0[2 * BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sKV1[2 * BN * HD];
  bf16 *const sK0 = sKV0, *const sV0 = sKV0 + BN * HD;
  bf16 *const sK1 = sKV1, *const sV1 = sKV1 + BN * HD;
  // per MFMA row of each group: the branch keys [x, y] the row sees (x > y: none)
  __shared__ int2 sBr[NG * 128];
  // per MFMA row of each group: (row * Hq + h) of a main row, -2 - ((row - Nq) *
  // Hq + h) of a branch row, -1 for padding (the row copies below)
  __shared__ int64_t sRowIdx[NG * 128];

  // Work unit: the forward's pair of adjacent query tiles of one sequence
  // (waves 0-3 the first, 4-7 the second) against the union of their key
  // ranges; every K/V tile in LDS serves both, which halves the K/V streams an
  // XCD's L2 has to hold.
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = mt.hkv, G = mt.G;
  __shared__ int sItem;
  const int item = workgroup_item(mt.queue_units, NG == 2 ? mt.n_fwd_pairs : mt.n_fwd_triples, hkv, &sItem);
  if (item < 0) return;  // every unit is taken (the whole workgroup)
  const int g = item % hkv;
  const int unit = item / hkv;
  int tl[NG];
#pragma unroll
  for (int u = 0; u < NG; ++u) tl[u] = uni(NG == 2 ? mt.fwd_pairs[2 * unit + u] : mt.fwd_triples[NG * unit + u]);
  const QTile tile_a = load_qtile(mt.qtiles + tl[0]);
  int end_b = -1;
#pragma unroll
  for (int u = 1; u < NG; ++u)
    if (tl[u] >= 0) end_b = max(end_b, uni(mt.qtiles[tl[u]].end_max));
  // With NG = 3 the DMA of a 64 x 64 tile (eight 1 KB blocks) is issued by waves 0-7.
  const bool dma_wave = NG == 2 || wave < 8;
  const int64_t R = mt.Nq + mt.Rb;
  const int kv_lo = tile_a.kv_lo, kv_end = max(tile_a.end_max, end_b);
  const int ntiles = (kv_end - kv_lo + BN) / BN;
  const int *bkr = NG == 2 ? mt.fwd_pair_bk : mt.fwd_triple_bk;
  const int bk_lo = uni(bkr[2 * unit]), bk_hi = uni(bkr[2 * unit + 1]);
  const int nbt = (bk_hi - bk_lo + BN - 1) / BN;  // 64-key tiles from bk_lo on (0 when none)
  AsyncTile<HD, BN, 512> kvt;
  kvt.init(hkv * HD, tid);
  const bf16 *kg = k + (int64_t)g * HD, *vg = v + (int64_t)g * HD;
  if (dma_wave) {
    kvt.load(sK0, kg, kv_lo, kv_end);
    kvt.load(sV0, vg, kv_lo, kv_end);
  }

  DqState<HD> st;
  const int mrow = (wave & 3) * 32 + (lane & 31);
  const int bi = mrow / G, hj = mrow - bi * G;
  int row = -1;
  st.end = -1;
  const int grpi = wave >> 2;
  const int my_tile = grpi == 0 ? tl[0] : grpi == 1 ? tl[1] : tl[NG - 1];
  QTile tile{};
  if (my_tile >= 0) {
    tile = load_qtile(mt.qtiles + my_tile);
    if (bi < tile.nrows) {
      row = mt.tile_row_id[tile.row_begin + bi];
      st.end = mt.tile_row_end[tile.row_begin + bi];
    }
  }
  const int h = mt.group_heads[g * G + hj];
  const bool is_main = row >= 0 && row < mt.Nq;
  const int64_t roff = row < 0 ? 0
                       : is_main ? ((int64_t)row * mt.hq + h) * HD
                                 : ((int64_t)(row - mt.Nq) * mt.hq + h) * HD;
  if (lane < 32)
    sRowIdx[grpi * 128 + mrow] = row < 0     ? -1
                                 : is_main ? (int64_t)row * mt.hq + h
                                           : -2 - ((int64_t)(row - mt.Nq) * mt.hq + h);
  __syncthreads();  // the table is complete (every wave of the workgroup)
  // The row's LSE and branch keys, loaded without a branch (a row that has
  // none reads a word of the staging area instead, and the value is dropped).
  const float *lp = row < 0 ? sg.lt : is_main ? lse + (int64_t)h * mt.Nq + row : lseb + (int64_t)h * mt.Rb + (row - mt.Nq);
  const bool has_br = row >= mt.Nq;
  const int *blp = has_br ? mt.brow_lo + (row - mt.Nq) : sg.et;
  const int *bhp = has_br ? mt.brow_hi + (row - mt.Nq) : sg.et;
  const float lrow = *lp;
  const int br_lo = *blp, br_hi = *bhp;
  const int2 br = has_br ? int2{br_lo, br_hi} : int2{INT_MAX, -1};
  // The Q and dO rows of the group's tile for the dK/dV kernel (stored further
  // down), read by the group's 256 threads as a stream of their own (LPR lanes
  // per row, whole 16-byte chunks; each row's source from the table above),
  // not stored from the registers that hold Q and dO: such a store makes the
  // compiler allocate the main loop's registers differently and serialise its
  // exponentials (measured 2.4% slower). A padding row reads a chunk of the
  // staging area instead (dropped).
  constexpr int LPR = HD / 8, RPP = 256 / LPR, NP = kTileRows / RPP;
  uint4 cq[NP], cdo[NP];
  {
    const int gt = tid & 255, ch = gt % LPR;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int64_t ri = sRowIdx[grpi * 128 + p * RPP + gt / LPR];
      const bool pad = ri == -1, mn = ri >= 0;
      const int64_t off = (mn ? ri : -2 - ri) * HD;
      const bf16 *xs = pad ? sg.qt : (mn ? q : qb) + off;
      const bf16 *ys = pad ? sg.dot : (mn ? d_o : d_ob) + off;
      uint4 x = reinterpret_cast<const uint4 *>(xs)[ch];
      uint4 y = reinterpret_cast<const uint4 *>(ys)[ch];
      if (pad) x = y = uint4{0u, 0u, 0u, 0u};
      cq[p] = x;
      cdo[p] = y;
    }
  }
  // Q, dO and O of the lane's half row (one batch of loads; O only for D).
  bf16x8 orow[KS];
  {
    const bf16 *qp = (is_main ? q : qb) + roff + 8 * (lane >> 5);
    const bf16 *op = (is_main ? d_o : d_ob) + roff + 8 * (lane >> 5);
    const bf16 *fp = (is_main ? o : ob) + roff + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row >= 0) {
        st.qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
        st.of[ks] = *reinterpret_cast<const bf16x8 *>(op + 16 * ks);
        orow[ks] = *reinterpret_cast<const bf16x8 *>(fp + 16 * ks);
      } else {
        st.qf[ks] = bf16x8{};
        st.of[ks] = bf16x8{};
        orow[ks] = bf16x8{};
      }
    }
  }
  st.l2 = row >= 0 ? lrow * kLog2e : INFINITY;  // padding rows: P = 0
  // D = rowsum(dO * O): lanes l and l + 32 hold the two halves of a row.
  float dd = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) dd = fmaf((float)st.of[ks][e], (float)orow[ks][e], dd);
  dd += __shfl_xor(dd, 32, 64);
#pragma unroll
  for (int i = 0; i < 16; ++i) st.nd[i] = -dd;
  const float sl2 = mt.scale * kLog2e;
  // What the dK/dV kernel streams, in its query-tile order: the tile's 128
  // MFMA rows with Q scaled by scale * log2(e) (rounded to bf16), dO,
  // -LSE * log2(e) and -D (the start values of its S and dP accumulators) and
  // (kv head 0) the row ends and the tile's end range; also D in [Hq, rows]
  // for the branch-local backward. Padding rows: zero rows, P = 0.
  if (my_tile >= 0) {
    const int64_t trow = ((int64_t)my_tile * hkv + g) * kTileRows + mrow;
    {
      const int gt = tid & 255, ch = gt % LPR;
      const int64_t tbase = ((int64_t)my_tile * hkv + g) * kTileRows;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int m = p * RPP + gt / LPR;
        const bf16x8 xb = __builtin_bit_cast(bf16x8, cq[p]);
        bf16x8 sq;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq[e] = (bf16)((float)xb[e] * sl2);
        reinterpret_cast<uint4 *>(sg.qt + (tbase + m) * HD)[ch] = __builtin_bit_cast(uint4, sq);
        reinterpret_cast<uint4 *>(sg.dot + (tbase + m) * HD)[ch] = cdo[p];
      }
    }
    if (lane < 32) {
      sg.lt[trow] = -st.l2;
      sg.dtt[trow] = row >= 0 ? -dd : 0.0f;
      if (row >= 0) sg.delta[(int64_t)h * R + row] = dd;
      if (g == 0) sg.et[(int64_t)my_tile * kTileMetaWords + mrow] = st.end;
    }
    if (g == 0 && (wave & 3) == 0 && lane < kTileMetaWords - kTileRows)
      sg.et[(int64_t)my_tile * kTileMetaWords + kTileRows + lane] =
          lane == 0 ? tile.end_min : lane == 1 ? tile.end_max : lane == 2 ? tile.nrows * G : 0;
  }
  st.wmin = wave_min(row >= 0 ? st.end : INT_MAX);
  const int wmax = wave_max(st.end);
  const int wbmin = uni(wave_min(br.x)), wbmax = uni(wave_max(br.y));
  int2 *const sBrw = sBr + grpi * 128 + (wave & 3) * 32;  // this wave's 32 rows
  if (lane < 32) sBrw[lane] = br;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
  st.lane = lane;
  st.grp = lane >> 4;
  st.in_j = (lane & 15) >> 2;
  st.in_q = lane & 3;

  for (int j = 0; j < ntiles; j += 2) {
    const int k0 = kv_lo + j * BN;
    dma_barrier<0>();  // tile j is in buffer 0; every wave is done with buffer 1
    if (j + 1 < ntiles && dma_wave) {
      kvt.load(sK1, kg, k0 + BN, kv_end);
      kvt.load(sV1, vg, k0 + BN, kv_end);
    }
    if (k0 <= wmax) {
      if (k0 + 63 > st.wmin) dq_tile<HD, true>(st, sK0, sV0, k0, sl2);
      else dq_tile<HD, false>(st, sK0, sV0, k0, sl2);
    }
    if (j + 1 >= ntiles) break;
    dma_barrier<0>();  // tile j+1 is in buffer 1; every wave is done with buffer 0
    if (j + 2 < ntiles && dma_wave) {
      kvt.load(sK0, kg, k0 + 2 * BN, kv_end);
      kvt.load(sV0, vg, k0 + 2 * BN, kv_end);
    }
    if (k0 + BN <= wmax) {
      if (k0 + BN + 63 > st.wmin) dq_tile<HD, true>(st, sK1, sV1, k0 + BN, sl2);
      else dq_tile<HD, false>(st, sK1, sV1, k0 + BN, sl2);
    }
  }
  // Branch tiles after the main loop (a few per unit, starting at the unit's
  // first branch key, so a unit whose branch keys fit in 64 takes one), one at
  // a time in buffer 0, masked to each row's own branch keys.
  const bf16 *kbg = kb + (int64_t)g * HD, *vbg = vb + (int64_t)g * HD;
  for (int jb = 0; jb < nbt; ++jb) {
    const int b0 = bk_lo + jb * BN;
    dma_barrier<0>();  // every wave is done with buffer 0
    if (dma_wave) {
      kvt.load(sK0, kbg, b0, (int)mt.Rb - 1);
      kvt.load(sV0, vbg, b0, (int)mt.Rb - 1);
    }
    dma_barrier<0>();  // the tile is in buffer 0
    if (b0 <= wbmax && b0 + BN - 1 >= wbmin) dq_tile<HD, true, true>(st, sK0, sV0, b0, sl2, sBrw + (lane & 31));
  }
  // The row's offset again from the LDS table, so that none of the row's
  // addressing is kept in registers across the key loops.
  const int64_t ridx = sRowIdx[uni(threadIdx.x >> 6) * 32 + (lane_id_here() & 31)];
  if (ridx != -1) {
    bf16 *dst = (ridx >= 0 ? dq + ridx * HD : dqb + (-2 - ridx) * HD);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + q4 * 8 + (lane >> 5) * 4;
        const bf16x4 val = {(bf16)(mt.scale * st.acc[dt][q4 * 4 + 0]), (bf16)(mt.scale * st.acc[dt][q4 * 4 + 1]),
                            (bf16)(mt.scale * st.acc[dt][q4 * 4 + 2]), (bf16)(mt.scale * st.acc[dt][q4 * 4 + 3])};
        *reinterpret_cast<bf16x4 *>(dst + d) = val;
      }
  }
}

namespace {

// Keys per wave: KB blocks of 32. At d = 128 eight waves of one block each
// give two waves per SIMD within the 256-register budget (K, V fragments and
// the dK, dV accumulators alone hold 192 registers); at d = 64 a wave needs
// about 164, so twelve waves (three per SIMD, 384 keys) fit, and each wave's
// elementwise work has two other waves' MFMAs beside it.
constexpr int kDkdvBlocks = 1;
// Operands in flight in the dV/dK product stretch (a ring of single operands).
constexpr int kDkdvRing = 4;
constexpr int dkdv_threads(int hd) { return 64 * (hd == 64 ? kBwdKeys64 : kBwdKeys) / (32 * kDkdvBlocks); }

template <int HD, int KB>
struct DkdvState {
  static constexpr int KS = HD / 16;
  static constexpr int DT = HD / 32;
  bf16x8 kf[KB][KS], vf[KB][KS];
  f32x16 adk[KB][DT], adv[KB][DT];
  int my_key[KB];
  int wkey_lo, key_hi;
  int lane;
  uint32_t r_base;  // padded-tile row reads of Q, dO (A operands of S, dP)
  uint32_t t_base;  // padded-tile transposing reads of dO, Q (B operands of dV, dK)
};

// Rows of one staged query tile against the wave's 32*KB keys; MASK when some
// row's prefix end or the key range cuts through the wave's keys.
template <int HD, int KB, bool MASK>
__device__ __forceinline__ void dkdv_rows(DkdvState<HD, KB> &st, const bf16 *sQ, const bf16 *sdO, const float *sL2,
                                          const float *sD, const int *sEnd) {
  constexpr int BM = kTileRows;
  constexpr int KS = DkdvState<HD, KB>::KS, DT = DkdvState<HD, KB>::DT;
  // dO follows Q in the same array; the second buffer starts beyond the reach
  // of an LDS read's 16-bit offset, so with the addresses left to constant
  // folding every read of it took an add of its own. Instead each row block
  // forms its two Q addresses (row and transposing reads: tile, lane offset,
  // row block) once, kept opaque, and every read is one of them plus an
  // immediate (dO at a fixed distance).
  constexpr uint32_t kOff = BM * kPadRowBytes<HD>;  // dO - Q, bytes
  uint32_t a_r = st.r_base, a_t = st.t_base;
  asm volatile("" : "+v"(a_r), "+v"(a_t));  // formed here, not hoisted out of the tile loop and spilled
  a_r += (uint32_t)(uintptr_t)sQ;
  a_t += (uint32_t)(uintptr_t)sQ;
  (void)sdO;
#pragma unroll 1
  for (int rb = 0; rb < BM / 32; ++rb) {
    const int lane = lane_id_here();
    uint32_t q_r = a_r + rb * 32 * kPadRowBytes<HD>, q_t = a_t + rb * 32 * kPadRowBytes<HD>;
    asm volatile("" : "+v"(q_r), "+v"(q_t));
    // Rows 32rb..32rb+31. element i: row rb*32 + (i/4)*8 + 4*(lane/32) + i%4,
    // key my_key[b].
    bf16x8 pa[KB][2], dsa[KB][2];
    // Operands of dV += P^T dO and dK += dS^T Q (transposing reads of dO, Q):
    // step i < NS is dV step i, step NS + n is dK step n; n = (kh, dt).
    // Operand slot 8*half + 4c + j <-> row 32rb + 16kh + 8c + 4*half + j.
    constexpr int NS = 2 * DT;
    auto rd = [&](int i) {
      const int n = i % NS, kk = n / DT, dt = n % DT;
      const uint32_t t = i < NS ? q_t + kOff : q_t;
      return join(pad_tr_read_at<HD>(t, 0, kk, dt), pad_tr_read_at<HD>(t, 1, kk, dt));
    };
    bf16x8 ring[kDkdvRing];
    {
      // S and dP of these rows, then P and dS element by element from the fp32
      // values (P rounded to bf16 once, for the dV product). The dP accumulator
      // starts at -D of its rows (staged per tile), so the MFMAs deliver dP - D.
      // Likewise S starts at -LSE * log2(e) of its rows and Q is staged scaled
      // by scale * log2(e), so the S MFMAs deliver the exponent of P.
      f32x16 sc[KB], dp[KB];
      f32x16 nd, nl;
      // the row block's -D and -LSE entries, from two opaque addresses plus
      // immediates (these arrays too lie beyond the reads' offset reach)
      uint32_t a_d = (uint32_t)(uintptr_t)sD + rb * 128 + 16 * (lane >> 5);
      uint32_t a_l = (uint32_t)(uintptr_t)sL2 + rb * 128 + 16 * (lane >> 5);
      asm volatile("" : "+v"(a_d), "+v"(a_l));
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 x = *(const __attribute__((address_space(3))) f32x4 *)(uintptr_t)(a_d + i4 * 32);
        const f32x4 y = *(const __attribute__((address_space(3))) f32x4 *)(uintptr_t)(a_l + i4 * 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nd[i4 * 4 + e] = x[e];
          nl[i4 * 4 + e] = y[e];
        }
      }
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        sc[b] = nl;
        dp[b] = nd;
      }
      __builtin_amdgcn_s_setprio(1);  // a wave in an MFMA stretch wins issue; the other wave's VALU fills in
      // The operands of step ks + 1 are read while step ks multiplies.
      bf16x8 aq[2], ao[2];
      aq[0] = pad_row_read_at<HD>(q_r, 0);
      ao[0] = pad_row_read_at<HD>(q_r + kOff, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 1 < KS) {
          aq[(ks + 1) & 1] = pad_row_read_at<HD>(q_r, ks + 1);
          ao[(ks + 1) & 1] = pad_row_read_at<HD>(q_r + kOff, ks + 1);
        }
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          sc[b] = mfma32(aq[ks & 1], st.kf[b][ks], sc[b]);
          dp[b] = mfma32(ao[ks & 1], st.vf[b][ks], dp[b]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // The first product operands do not depend on the elementwise step:
      // their reads are issued before it, so its vector work covers them.
#pragma unroll
      for (int i = 0; i < kDkdvRing - 1; ++i) ring[i] = rd(i);
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r0 = rb * 32 + i4 * 8 + 4 * (lane >> 5);
        int4 ends = {0, 0, 0, 0};
        if constexpr (MASK) ends = *reinterpret_cast<const int4 *>(sEnd + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = i4 * 4 + e;
#pragma unroll
          for (int b = 0; b < KB; ++b) {
            float p = fast_exp2(sc[b][i]);
            if (MASK && (ends[e] < st.my_key[b] || st.my_key[b] >= st.key_hi)) p = 0.0f;
            pa[b][i >> 3][i & 7] = (bf16)p;
            dsa[b][i >> 3][i & 7] = (bf16)(p * dp[b][i]);
          }
        }
      }
    }
    // dV += P^T dO, dK += dS^T Q over these 32 rows (two 16-row k-steps): all
    // dV steps, then all dK steps, through one ring of kDkdvRing operands, a
    // read issued kDkdvRing - 1 MFMAs before its use.
    __builtin_amdgcn_s_setprio(2);  // above an S/dP stretch of the other wave
    {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NS; ++i) {
        if (i + kDkdvRing - 1 < 2 * NS) ring[(i + kDkdvRing - 1) % kDkdvRing] = rd(i + kDkdvRing - 1);
        const int n = i % NS;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          if (i < NS) st.adv[b][n % DT] = mfma32(pa[b][n / DT], ring[i % kDkdvRing], st.adv[b][n % DT]);
          else st.adk[b][n % DT] = mfma32(dsa[b][n / DT], ring[i % kDkdvRing], st.adk[b][n % DT]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

// One query tile (128 MFMA rows staged in LDS) against the wave's 32*KB keys.
template <int HD, int KB>
__device__ __forceinline__ void dkdv_tile(DkdvState<HD, KB> &st, const bf16 *sQ, const bf16 *sdO, const float *sL2,
                                          const float *sD, const int *sEnd) {
  constexpr int BM = kTileRows;
  constexpr int WK = 32 * KB;  // keys of this wave
  const int end_min = uni(sEnd[BM]), end_max = uni(sEnd[BM + 1]), valid_rows = uni(sEnd[BM + 2]);
  if (end_max < st.wkey_lo || st.wkey_lo >= st.key_hi) return;  // no row of this tile sees the wave's keys
  if (end_min < st.wkey_lo + WK - 1 || st.wkey_lo + WK - 1 >= st.key_hi || valid_rows < BM)
    dkdv_rows<HD, KB, true>(st, sQ, sdO, sL2, sD, sEnd);
  else
    dkdv_rows<HD, KB, false>(st, sQ, sdO, sL2, sD, sEnd);
}

}  // namespace

template <int HD>
__global__ __launch_bounds__(dkdv_threads(HD), 1) void main_bwd_dkdv_bf16_kernel(Meta mt, const bf16 *__restrict__ k,
                                                                          const bf16 *__restrict__ v,
                                                                          const bf16 *__restrict__ qt_rows,
                                                                          const bf16 *__restrict__ do_rows,
                                                                          const float *__restrict__ lt,
                                                                          const float *__restrict__ dtt,
                                                                          const int *__restrict__ et,
                                                                          bf16 *__restrict__ dk, bf16 *__restrict__ dv,
                                                                          float *__restrict__ dkv_acc) {
  constexpr int BM = kTileRows;  // 128 MFMA rows per query tile
  constexpr int KB = kDkdvBlocks, NT = dkdv_threads(HD);
  constexpr int KS = HD / 16, DT = HD / 32;
  static_assert((HD == 64 ? kBwdKeys64 : kBwdKeys) == 32 * KB * (NT / 64) && BM == 128, "tile shape");
  constexpr int NSW = 8;  // waves that stage the Q and dO rows (128 rows split evenly)
  // Padded tiles (see stage_padded_async). Q and dO of one buffer share an
  // array, so a read of either is one address plus a constant offset.
  constexpr int TILE = BM * kPadRowBytes<HD> / 2;  // elements per padded tile
  __shared__ __attribute__((aligned(16))) bf16 sQO0[2 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 sQO1[2 * TILE];
  bf16 *const sQ0 = sQO0, *const sO0 = sQO0 + TILE;
  bf16 *const sQ1 = sQO1, *const sO1 = sQO1 + TILE;
  __shared__ __attribute__((aligned(16))) float sL0[BM], sD0[BM], sL1[BM], sD1[BM];
  __shared__ __attribute__((aligned(16))) int sE0[kTileMetaWords], sE1[kTileMetaWords];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = mt.hkv;
  __shared__ int sItem;
  const int item = workgroup_item(mt.queue_ktiles, mt.n_ktiles, hkv, &sItem);
  if (item < 0) return;  // every key tile is taken (the whole workgroup)
  const int g = item % hkv;
  const KTile kt = load_ktile(mt.ktiles + uni(mt.bwd_order[item / hkv]));

  // Query tile qi, kv head g -> one LDS buffer (all asynchronous; the next tile
  // barrier waits for it): the row metadata (-LSE, -D, row ends) by waves 0-2,
  // the Q and dO rows by the NSW staging waves.
  auto prefetch = [&](int qi, bf16 *sQ, bf16 *sO, float *sL, float *sD, int *sE) {
    const int64_t tb = ((int64_t)qi * hkv + g) * BM;
    const int lane = lane_id_here();  // per-lane source addresses formed here, not kept across the tile loop
    if (wave == 0) stage_words_async<BM / 64>(sL, lt + tb, lane);
    else if (wave == 1) stage_words_async<BM / 64>(sD, dtt + tb, lane);
    else if (wave == 2) stage_words_async<kTileMetaWords / 64>(sE, et + (int64_t)qi * kTileMetaWords, lane);
    if (NT / 64 == NSW || wave < NSW) {
      stage_padded_async<HD, BM, NSW>(sQ, qt_rows + tb * HD, wave, lane);
      stage_padded_async<HD, BM, NSW>(sO, do_rows + tb * HD, wave, lane);
    }
  };
  if (kt.qt_begin < kt.qt_end) prefetch(kt.qt_begin, sQ0, sO0, sL0, sD0, sE0);

  // The wave's own K and V as B operands: in key block b, lane holds key
  // 32*(KB*wave + b) + lane%32, d = 16*ks + 8*(lane/32) + 0..7.
  DkdvState<HD, KB> st;
  st.wkey_lo = kt.key_lo + wave * 32 * KB;
  st.key_hi = kt.key_hi;
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    st.my_key[b] = st.wkey_lo + 32 * b + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (st.my_key[b] < kt.key_hi) {
        const int64_t src = ((int64_t)st.my_key[b] * hkv + g) * HD + 16 * ks + 8 * (lane >> 5);
        st.kf[b][ks] = *reinterpret_cast<const bf16x8 *>(k + src);
        st.vf[b][ks] = *reinterpret_cast<const bf16x8 *>(v + src);
      } else {
        st.kf[b][ks] = bf16x8{};
        st.vf[b][ks] = bf16x8{};
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      st.adk[b][dt] = f32x16{};
      st.adv[b][dt] = f32x16{};
    }
  }
  st.lane = lane;
  st.r_base = pad_row_base<HD>(lane);
  st.t_base = pad_tr_base<HD>(lane);

  // Waves 0-3 (the older wave of each SIMD, which wins issue ties and would
  // otherwise run ahead, then wait at the next barrier) start each tile about
  // 128 cycles after the others.
  const bool delay = uni(wave) < 4;
  for (int qi = kt.qt_begin; qi < kt.qt_end; qi += 2) {
    dma_barrier<0>();  // tile qi is in buffer 0; every wave is done with buffer 1
    if (qi + 1 < kt.qt_end) prefetch(qi + 1, sQ1, sO1, sL1, sD1, sE1);
    if (delay) __builtin_amdgcn_s_sleep(2);
    dkdv_tile<HD, KB>(st, sQ0, sO0, sL0, sD0, sE0);
    if (qi + 1 >= kt.qt_end) break;
    dma_barrier<0>();  // tile qi+1 is in buffer 1; every wave is done with buffer 0
    if (qi + 2 < kt.qt_end) prefetch(qi + 2, sQ0, sO0, sL0, sD0, sE0);
    if (delay) __builtin_amdgcn_s_sleep(2);
    dkdv_tile<HD, KB>(st, sQ1, sO1, sL1, sD1, sE1);
  }

  // dK, dV of the wave's keys: element i of block (b, dt) is key wkey_lo +
  // 32b + (i/4)*8 + 4*(lane/32) + i%4, d = 32dt + lane%32. The staged Q rows
  // carry scale * log2(e), so dK = scale * dS^T Q = ln(2) * dS^T Q_staged.
  // With split key tiles the float32 results are added into the accumulators
  // (dK at dkv_acc, dV N * Hkv * d further on) instead.
  const int64_t acc_v = (int64_t)mt.N * hkv * HD;
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = st.wkey_lo + 32 * b + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
      if (key < kt.key_hi) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int64_t dst = ((int64_t)key * hkv + g) * HD + dt * 32 + (lane & 31);
          if (dkv_acc) {
            atomicAdd(dkv_acc + dst, kLn2 * st.adk[b][dt][i]);
            atomicAdd(dkv_acc + acc_v + dst, st.adv[b][dt][i]);
          } else {
            dk[dst] = (bf16)(kLn2 * st.adk[b][dt][i]);
            dv[dst] = (bf16)st.adv[b][dt][i];
          }
        }
      }
    }
}

hipError_t launch_main_bwd_dq_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *v,
                                   const bf16 *d_o, const bf16 *d_ob, const float *lse, const float *lseb,
                                   const bf16 *o, const bf16 *ob, const bf16 *kb, const bf16 *vb, bf16 *dq,
                                   bf16 *dqb, const BwdStage &sg, hipStream_t st) {
  if (mt.n_fwd_pairs == 0) return hipSuccess;
  if (mt.d == 128)
    main_bwd_dq_bf16_kernel<128, 2><<<queue_grid((int64_t)mt.n_fwd_pairs * mt.hkv, mt.queue_units), 512, 0, st>>>(
        mt, q, qb, k, v, d_o, d_ob, lse, lseb, o, ob, kb, vb, dq, dqb, sg);
  else
    main_bwd_dq_bf16_kernel<64, 3><<<queue_grid((int64_t)mt.n_fwd_triples * mt.hkv, mt.queue_units), 768, 0, st>>>(
        mt, q, qb, k, v, d_o, d_ob, lse, lseb, o, ob, kb, vb, dq, dqb, sg);
  return hipGetLastError();
}

hipError_t launch_main_bwd_dkdv_bf16(const Meta &mt, const bf16 *k, const bf16 *v, const bf16 *qt, const bf16 *dot,
                                     const float *lt, const float *dtt, const int *et, bf16 *dk, bf16 *dv,
                                     float *dkv_acc, hipStream_t st) {
  if (mt.n_ktiles == 0) return hipSuccess;
  const unsigned grid = queue_grid((int64_t)mt.n_ktiles * mt.hkv, mt.queue_ktiles);
  if (mt.d == 128)
    main_bwd_dkdv_bf16_kernel<128><<<grid, dkdv_threads(128), 0, st>>>(mt, k, v, qt, dot, lt, dtt, et, dk, dv,
                                                                        dkv_acc);
  else
    main_bwd_dkdv_bf16_kernel<64><<<grid, dkdv_threads(64), 0, st>>>(mt, k, v, qt, dot, lt, dtt, et, dk, dv,
                                                                      dkv_acc);
  return hipGetLastError();
}

}  // namespace ba
