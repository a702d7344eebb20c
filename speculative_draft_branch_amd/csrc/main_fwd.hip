// Main-sequence forward on bf16 MFMA (gfx950): every query row -- main rows and
// draft-branch rows alike -- attends its causal main prefix in its own packed
// sequence, with an online softmax. In the merged forward (FUSED) the branch
// rows then take their own branch's keys as the last key tiles of the same
// softmax, which is the log-sum-exp merge of the main-prefix and branch-local
// parts taken inside one pass (evolve.pub review, "Scope & Claims", section 3.2
// and Eq. 2; rcap.io explainer, paragraph on branch attention under context
// parallelism; cere-bro wiki, "Mechanism"); branch K/V still never join the
// main-key tiles, and every row's final output is written once. The split-path
// instantiation instead leaves branch rows a float32 partial (O_pre, LSE_pre)
// for lse_merge.
//
// Work unit: two query tiles of one sequence that are adjacent in prefix-end
// order (each up to 128 MFMA rows = base rows x q heads of one kv group, sorted
// by prefix end) against their key range [sequence start, largest prefix end],
// streamed in 64-key K/V tiles through LDS. Rows that share a prefix end (a main
// row, the branch rows anchored at the same token, and the q heads of the kv
// group) share every K/V tile, and so do the two query tiles. The grid is
// longest-first; blockIdx % Hkv selects the kv head, so with 8 kv heads each
// XCD streams one kv head's keys.
//
// Eight waves in two groups of four, one group per query tile, two waves per
// SIMD. Each group alternates a matrix phase (P V of the previous K/V tile, then
// S of the current one) with a softmax phase, and the groups start each tile
// one phase apart (group 0 on its matrix phase, group 1 on its softmax phase):
// while one group's exponentials occupy the vector ALUs the other group's MFMAs
// keep the matrix cores busy. One workgroup barrier per tile; within the tile
// each group moves on to its second phase as soon as its first is done. K and
// V tiles are double-buffered and written straight into LDS by
// global_load_lds; a tile is requested two phases before its first use.
//
// Per wave (32 query rows): S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so each
// lane owns one query row (lane % 32) and row max/sum need a single exchange
// between the two wave halves; P^T feeds O^T += V^T P^T straight from
// registers. V is transposed once per call into 64-key tiles [d][key] whose
// keys sit in the MFMA operand-slot order, so its operand is a plain 16-byte
// row read (the transposing LDS read runs at about half that rate). The
// softmax reference is each row's max over the wave's first tile and is only
// raised when a row sum would pass 2^64, so no per-tile max is taken.
#include <climits>

#include "launch.hpp"

namespace ba {

namespace {


template <int HD>
struct FwdState {
  static constexpr int KS = HD / 16;
  static constexpr int DT = HD / 32;
  bf16x8 qf[KS];
  f32x16 acc[DT];
  float m_run, l_run;
  bool started;  // the running max has been set (wave-uniform)
  int end, wmin, wmax;
  int klo;  // ring step: first key of the window (keys below it are masked)
  int blo, bhi;      // branch keys (branch row indices) this row sees: [blo, bhi]; none for main rows
  int wbmin, wbmax;  // smallest blo and largest bhi of the wave
  int lane;
  uint32_t k_base, k_t;  // K row reads
  uint32_t v_base, v_t;  // V^T row reads
  // the swizzled byte offset of each k-step's K and V^T read, formed once, so a
  // read is a register plus an immediate (no XOR and add per read)
  uint32_t k_off[KS], v_off[4];
};

// Matrix phase: O^T += V^T P^T for the previous K/V tile (PV), then the raw
// scores S^T[key][row] of the current tile in two 32-key blocks (S). PV k-step
// kk covers tile keys 16kk..16kk+15; operand slot 8*half + 4c + j <-> key
// 16kk + 8c + 4*half + j on both operands, which is the order the V^T tile
// stores them in, so lane (d, half) reads 8 consecutive elements of row d.
//
// The phase is one software pipeline of (LDS read, MFMA) steps: the operands
// of the next ring steps are always in flight, so LDS latency is paid about
// once per phase rather than once per k-step. Six at d = 128; three at d = 64,
// where three waves per SIMD leave 168 registers a wave: with six the kernel
// spilled, and reloaded the spilled DMA addresses inside the tile loop (4.8%
// slower).
constexpr int fwd_ring(int hd) { return hd == 64 ? 3 : 6; }

template <int HD, bool PV, bool S>
__device__ __forceinline__ void fwd_mphase(FwdState<HD> &st, const bf16 *sVt, const bf16 *sK, const bf16x8 (&pb)[4],
                                           f32x16 (&s)[2]) {
  constexpr int KS = FwdState<HD>::KS, DT = FwdState<HD>::DT;
  constexpr int NPV = PV ? 4 * DT : 0;  // step i < NPV: kk = i / DT, dt = i % DT
  constexpr int NS = S ? 2 * KS : 0;    // then step NPV + j: ks = j / 2, kb = j % 2
  constexpr int N = NPV + NS;
  constexpr int R = fwd_ring(HD) < N ? fwd_ring(HD) : N;
  auto rd = [&](int i) -> bf16x8 {
    if (i < NPV)
      return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(sVt) + st.v_off[i / DT] +
                                               (i % DT) * 32 * 64 * 2);
    const int j = i - NPV;
    return *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(sK) + st.k_off[j / 2] +
                                             (j % 2) * 32 * HD * 2);
  };
  if constexpr (S) {
    s[0] = f32x16{};
    s[1] = f32x16{};
  }
  // The scheduling barriers pin this order; left alone, the compiler sinks
  // every read next to its MFMA and waits for each one in turn.
  bf16x8 ring[R];
#pragma unroll
  for (int i = 0; i < R; ++i) ring[i] = rd(i);
  // The S steps, whose scores the wave's own next softmax phase waits for,
  // run at priority 2, the P V steps at the caller's 1.
  if (!PV) __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (PV && S && i == NPV) __builtin_amdgcn_s_setprio(2);
    if (i < NPV) {
      st.acc[i % DT] = mfma32(ring[i % R], pb[i / DT], st.acc[i % DT]);
    } else {
      const int j = i - NPV;
      s[j % 2] = mfma32(ring[i % R], st.qf[j / 2], s[j % 2]);
    }
    if (i + R < N) ring[i % R] = rd(i + R);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Softmax phase for the tile [k0, k0 + 64): mask keys past each row's prefix
// end and form P^T = exp2(S * scale * log2(e) - m) in bf16. The reference m is
// the row max of the wave's first tile and is not re-derived per tile: a later
// score above it only makes P larger than 1, which bf16 and the fp32 sums hold
// exactly in relative terms. Only when a lane's partial row sum passes 2^64 is
// the tile's true max taken, O and l rescaled to it and P formed again.
template <int HD>
__device__ __forceinline__ float tile_row_max(const f32x16 (&s)[2], float sl2) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  return half_max(mx) * sl2;
}

// P^T in bf16 against the current reference; returns this lane's partial row sum.
template <int HD>
__device__ __forceinline__ float fwd_form_p(const FwdState<HD> &st, const f32x16 (&s)[2], float sl2,
                                            bf16x8 (&pb)[4]) {
  const float m_use = (st.m_run == -INFINITY) ? 0.0f : st.m_run;  // padding rows stay at -inf
  float rs = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[kb][i], sl2, -m_use));
      rs += p;
      pb[kb * 2 + (i >> 3)][i & 7] = (bf16)p;
    }
  return rs;
}

template <int HD, bool RING, bool BRANCH>
__device__ __forceinline__ void fwd_softmax(FwdState<HD> &st, f32x16 (&s)[2], int k0, float sl2, bf16x8 (&pb)[4]) {
  constexpr int DT = FwdState<HD>::DT;
  const int lane = st.lane;
  if constexpr (BRANCH) {  // a tile of branch keys: each row sees its own branch's keys only
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (key < st.blo || key > st.bhi) s[kb][i] = -INFINITY;
      }
  } else if (k0 + 63 > st.wmin || (RING && k0 < st.klo)) {
    // some key of this tile lies past some row's prefix end (or, in a ring step, before the window)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (key > st.end || (RING && key < st.klo)) s[kb][i] = -INFINITY;
      }
  }
  if (!st.started) {  // the wave's first tile holds every row's first visible key
    st.m_run = tile_row_max<HD>(s, sl2);
    st.started = true;
  }
  float rs = fwd_form_p<HD>(st, s, sl2, pb);
  if (__any(rs > 0x1p64f)) {  // rare: raise the reference to this tile's max and form P again
    const float m_new = fmaxf(st.m_run, tile_row_max<HD>(s, sl2));
    const float alpha = fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
    st.m_run = m_new;
    rs = fwd_form_p<HD>(st, s, sl2, pb);
  }
  st.l_run += rs;
}


// K tile of keys [key0, key0 + 64): rows past `last` read row `last`; in a ring
// step the buffer starts at position kb0 and rows before `first` read `first`.
template <bool RING, class Tile>
__device__ __forceinline__ void load_k_tile(const Tile &kt, bf16 *dst, const bf16 *kg, int key0, int kb0, int first,
                                            int last) {
  if constexpr (RING) kt.load_window(dst, kg, key0 - kb0, first - kb0, last - kb0);
  else kt.load(dst, kg, key0, last);
}

}  // namespace

// RING: one step of a context-parallel ring. Only the main keys in the window
// [win_lo, win_hi) are attended; k holds exactly those rows (row 0 = position
// win_lo) and vt their V^T tiles; every row's partial is merged into the
// running float32 (o_run [Nq+Rb][Hq][d], lse_run [Hq][Nq+Rb]) in the epilogue.
// FUSED: after its main keys the unit takes the branch keys its branch rows
// see -- the contiguous range [bk_lo, bk_hi) of branch rows, in 64-key tiles
// from bk_lo on (rows of kb; the unit's own tiles of vbt, the branch V
// transposed like vt, so a range that fits in 64 keys is one tile wherever
// it starts) -- as further key tiles of the
// same online softmax, each row masked to its own branch's keys (a TTT query j
// sees keys 1..j of its branch, a block query the whole block). The softmax
// then covers the union of the row's keys, which is the merged result of the
// main-prefix and branch-local parts (the log-sum-exp merge, taken inside the
// pass), so every row's final output goes straight to o / ob (bf16) and lse /
// lseb, with no partial in HBM. Otherwise branch rows leave a float32 partial
// of their main prefix in o_pre / lse_pre.
// NG: groups of four waves, one query tile each. With NG = 3 (the d = 64
// forward, whose softmax phase is twice its matrix phase) two groups run their
// softmax beside the third group's MFMAs, which gives the vector units of a
// SIMD a third more throughput than one softmax wave gets there.
template <int HD, bool RING, int NG, bool FUSED>
__global__ __launch_bounds__(256 * NG, 1) void main_fwd_bf16_kernel(Meta mt, const bf16 *__restrict__ q,
                                                            const bf16 *__restrict__ qb,
                                                            const bf16 *__restrict__ k,
                                                            const bf16 *__restrict__ vt, bf16 *__restrict__ o,
                                                            float *__restrict__ lse, float *__restrict__ o_pre,
                                                            float *__restrict__ lse_pre, int win_lo, int win_hi,
                                                            float *__restrict__ o_run, float *__restrict__ lse_run,
                                                            const bf16 *__restrict__ kb, const bf16 *__restrict__ vbt,
                                                            bf16 *__restrict__ ob, float *__restrict__ lseb) {
  constexpr int BN = 64;  // keys per K/V tile
  constexpr int KS = HD / 16, DT = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV1[BN * HD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grpi = wave >> 2;  // group: 0 runs one phase ahead of the others
  const int gp = grpi == 0 ? 0 : 1;  // the phase order of the wave's group
  const int hkv = mt.hkv, G = mt.G;
  __shared__ int sItem;
  // At d = 128 the workgroups loop over items while the counters hand them out
  // (one workgroup per compute unit); at d = 64 (the loop there costs spills)
  // and with no counters, one item per workgroup.
  for (;;) {
    const int item = workgroup_item(mt.queue_units, NG == 2 ? mt.n_fwd_pairs : mt.n_fwd_triples, hkv, &sItem);
    if (item < 0) return;  // every unit is taken (the whole workgroup)
    const int g = item % hkv;
    const int unit = item / hkv;
    int tl[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) tl[u] = uni(NG == 2 ? mt.fwd_pairs[2 * unit + u] : mt.fwd_triples[NG * unit + u]);
    const int ta = tl[0];
    const QTile tile_a = load_qtile(mt.qtiles + ta);
    int end_b = -1;
#pragma unroll
    for (int u = 1; u < NG; ++u)
      if (tl[u] >= 0) end_b = max(end_b, uni(mt.qtiles[tl[u]].end_max));
    // With NG = 3 the DMA of a 64 x 64 tile (eight 1 KB blocks) is issued by waves 0-7.
    const bool dma_wave = NG == 2 || wave < 8;
    // Keys [k_first + 64j, ...) for j < ntiles; k_first is the sequence start, or
    // in a ring step the start of the sequence's 64-key tile holding the window
    // start (tile t0 of the sequence), and keys before klo are masked.
    const int kv_lo = tile_a.kv_lo;
    int kv_end = max(tile_a.end_max, end_b), klo = kv_lo, t0 = 0;
    if constexpr (RING) {
      klo = max(kv_lo, win_lo);
      t0 = (klo - kv_lo) / BN;
      kv_end = min(kv_end, win_hi - 1);
    }
    const int k_first = kv_lo + t0 * BN;
    const int ntiles = kv_end >= klo ? (kv_end - k_first + BN) / BN : 0;
    // Fused: nbt branch tiles follow the main tiles, 64 branch keys each from
    // the unit's first branch key b_first; their V^T tiles from vbt tile bt0 on.
    int b_first = 0, bt0 = 0, nbt = 0;
    if constexpr (FUSED) {
      const int *bk = NG == 2 ? mt.fwd_pair_bk : mt.fwd_triple_bk;
      const int bk_lo = uni(bk[2 * unit]), bk_hi = uni(bk[2 * unit + 1]);
      b_first = bk_lo;
      bt0 = uni(mt.fwd_unit_bt[unit]);
      nbt = (bk_hi - bk_lo + BN - 1) / BN;
    }

    // This lane's query row: MFMA row 32*(wave%4) + lane%32 = base row * G + head
    // of the group's tile.
    FwdState<HD> st;
    const int mrow = (wave & 3) * 32 + (lane & 31);
    const int bi = mrow / G, hj = mrow - bi * G;
    int row = -1;
    st.end = -1;
    const int my_tile = grpi == 0 ? tl[0] : grpi == 1 ? tl[1] : tl[NG - 1];
    if (my_tile >= 0) {
      const QTile tile = load_qtile(mt.qtiles + my_tile);
      if (bi < tile.nrows) {
        row = mt.tile_row_id[tile.row_begin + bi];
        st.end = mt.tile_row_end[tile.row_begin + bi];
        if constexpr (RING) st.end = min(st.end, win_hi - 1);  // may fall below klo: the row sees no key
      }
    }
    const int h = mt.group_heads[g * G + hj];
    const bool is_main = row >= 0 && row < mt.Nq;
    const int64_t roff = row < 0 ? 0
                         : is_main ? ((int64_t)row * mt.hq + h) * HD
                                   : ((int64_t)(row - mt.Nq) * mt.hq + h) * HD;
    // Q as the B operand: lane holds row lane%32, d = 16*ks + 8*(lane/32) + 0..7.
    {
      const bf16 *qp = (is_main ? q : qb) + roff + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (row >= 0) st.qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
        else st.qf[ks] = bf16x8{};
      }
    }
    st.wmin = wave_min(row >= 0 ? st.end : INT_MAX);
    st.wmax = wave_max(st.end);
    if constexpr (FUSED) {
      st.blo = INT_MAX;
      st.bhi = -1;
      if (row >= mt.Nq) {
        st.blo = mt.brow_lo[row - mt.Nq];
        st.bhi = mt.brow_hi[row - mt.Nq];
      }
      st.wbmin = uni(wave_min(st.blo));
      st.wbmax = uni(wave_max(st.bhi));
    }
    st.klo = klo;
    st.m_run = -INFINITY;
    st.l_run = 0.0f;
    st.started = false;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
    st.lane = lane;
    row_read_init<HD>(lane & 31, lane, st.k_base, st.k_t);
    row_read_init<64>(lane & 31, lane, st.v_base, st.v_t);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) st.k_off[ks] = st.k_base + (((uint32_t)ks << 5) ^ st.k_t);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) st.v_off[kk] = st.v_base + (((uint32_t)kk << 5) ^ st.v_t);
    const float sl2 = mt.scale * kLog2e;

    // K tiles: 64 keys x d from the [N][Hkv][d] tensor; V^T tiles: d rows x 64
    // keys, whole tiles of this sequence's transposed copy.
    AsyncTile<HD, BN, 512> kt;
    kt.init(hkv * HD, tid);
    AsyncTile<64, HD, 512> vtt;
    vtt.init(64, tid);
    const bf16 *kg = k + (int64_t)g * HD;
    const bf16 *vtg = vt + ((int64_t)(mt.vt_base[tile_a.seq] + t0) * hkv + g) * (HD * 64);
    const int64_t vt_stride = (int64_t)hkv * HD * 64;  // between consecutive V^T tiles
    // K rows are addressed relative to the buffer's first position (the window
    // start in a ring step); a ring step's first tile may begin before it.
    const int kb0 = RING ? win_lo : 0;
    if (ntiles > 0 && dma_wave) load_k_tile<RING>(kt, sK0, kg, k_first, kb0, klo, kv_end);
    dma_barrier<0>();

    // Phase slots: slot t runs, for group grpi, local phase u = t - grpi; even u
    // is the matrix phase of tile j = u/2 (P V of tile j-1, S of tile j), odd u
    // the softmax of tile (u-1)/2. Tile j's K is in buffer j%2 from slot 2j, its
    // V in buffer j%2 from slot 2j+2; both are requested at slot 2j-2 and 2j
    // respectively, so every DMA has two phases to land. The loop is unrolled
    // over the tile parity, so every buffer address is a constant.
    f32x16 s[2];
    bf16x8 pb[4];
    const int nslots = 2 * ntiles + 2;
    for (int j = 0;; j += 2) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int jj = j + par;  // tile whose matrix phase falls in these two slots
        bf16 *const sKc = par ? sK1 : sK0, *const sKn = par ? sK0 : sK1;
        bf16 *const sVc = par ? sV1 : sV0, *const sVp = par ? sV0 : sV1;
        // slot 2jj: requests, then group 0 matrix phase of jj, group 1 softmax of jj-1
        if (2 * jj >= nslots) goto done;
        if (jj + 1 < ntiles && dma_wave) load_k_tile<RING>(kt, sKn, kg, k_first + (jj + 1) * BN, kb0, klo, kv_end);
        if (jj < ntiles && dma_wave) vtt.load(sVc, vtg + jj * vt_stride, 0, HD - 1);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          if (h2 == 1 && 2 * jj + 1 >= nslots) goto done;
          if (gp == h2) {  // matrix phase of tile jj
            const bool do_pv = jj >= 1 && jj <= ntiles && k_first + (jj - 1) * BN <= st.wmax;
            const bool do_s = jj < ntiles && k_first + jj * BN <= st.wmax;
            __builtin_amdgcn_s_setprio(1);  // the matrix wave wins issue arbitration over the softmax wave
            if (do_pv && do_s) fwd_mphase<HD, true, true>(st, sVp, sKc, pb, s);
            else if (do_s) fwd_mphase<HD, false, true>(st, sVp, sKc, pb, s);
            else if (do_pv) fwd_mphase<HD, true, false>(st, sVp, sKc, pb, s);
            __builtin_amdgcn_s_setprio(0);
          } else {  // softmax of tile jj - 1 (group 1 at h2 = 0) or jj (group 0 at h2 = 1)
            const int js = jj - 1 + h2;
            if (js >= 0 && js < ntiles && k_first + js * BN <= st.wmax)
              fwd_softmax<HD, RING, false>(st, s, k_first + js * BN, sl2, pb);
          }
          // Only the end of the tile needs a barrier (the next requests reuse
          // buffers read in this tile); a second one between the phases, which
          // only kept the groups in step, cost 1.2%.
          if (h2 == 1) dma_barrier<0>();
        }
      }
    }
  done:
    if constexpr (FUSED) {
      // The branch keys, one 64-key tile at a time after the main loop (a few
      // tiles per unit): S, the softmax masked to each row's own branch keys,
      // then P V, all in each wave, with no phase offset between the groups.
      const bf16 *kbg = kb + (int64_t)g * HD;
      const bf16 *vbtg = vbt + (int64_t)g * (HD * 64);
      for (int jb = 0; jb < nbt; ++jb) {
        const int b0 = b_first + jb * BN;
        dma_barrier<0>();  // every wave is done with buffer 0
        if (dma_wave) {
          kt.load(sK0, kbg, b0, (int)mt.Rb - 1);
          vtt.load(sV0, vbtg + (int64_t)(bt0 + jb) * vt_stride, 0, HD - 1);
        }
        dma_barrier<0>();  // the tile is in buffer 0
        if (b0 <= st.wbmax && b0 + BN - 1 >= st.wbmin) {
          fwd_mphase<HD, false, true>(st, sV0, sK0, pb, s);
          __builtin_amdgcn_s_setprio(0);  // the S steps raised it; no phase offset here
          fwd_softmax<HD, false, true>(st, s, b0, sl2, pb);
          fwd_mphase<HD, true, false>(st, sV0, sK0, pb, s);
        }
      }
    }

    const float l_tot = half_sum(st.l_run);
    if constexpr (RING) {
      // Merge this window's partial into the running (O, LSE) of the row (Eq. 2);
      // a row that saw no key of the window leaves it unchanged.
      if (row >= 0 && l_tot > 0.0f) {
        const int64_t R = mt.Nq + mt.Rb;
        float *orow = o_run + ((int64_t)row * mt.hq + h) * HD;
        const float lp = (st.m_run + __log2f(l_tot)) * kLn2;
        const float la = lse_run[(int64_t)h * R + row];
        const float M = fmaxf(la, lp);
        const float wa = __expf(la - M), wb = __expf(lp - M);
        const float tot = wa + wb;
        const float fa = wa / tot, fb = wb / (tot * l_tot);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d = dt * 32 + q4 * 8 + (lane >> 5) * 4;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(orow + d);
            const f32x4 val = {fa * x[0] + fb * st.acc[dt][q4 * 4 + 0], fa * x[1] + fb * st.acc[dt][q4 * 4 + 1],
                               fa * x[2] + fb * st.acc[dt][q4 * 4 + 2], fa * x[3] + fb * st.acc[dt][q4 * 4 + 3]};
            *reinterpret_cast<f32x4 *>(orow + d) = val;
          }
        if (lane < 32) lse_run[(int64_t)h * R + row] = M + __logf(tot);
      }
      return;
    }
    if (row >= 0) {
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = dt * 32 + q4 * 8 + (lane >> 5) * 4;
          const f32x4 val = {st.acc[dt][q4 * 4 + 0] * inv, st.acc[dt][q4 * 4 + 1] * inv,
                             st.acc[dt][q4 * 4 + 2] * inv, st.acc[dt][q4 * 4 + 3] * inv};
          if (is_main || FUSED) {
            const bf16x4 b = {(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
            *reinterpret_cast<bf16x4 *>((is_main ? o : ob) + roff + d) = b;
          } else {
            *reinterpret_cast<f32x4 *>(o_pre + roff + d) = val;
          }
        }
      if (lane < 32) {
        const float lv = (st.m_run + __log2f(l_tot)) * kLn2;
        if (is_main) lse[(int64_t)h * mt.Nq + row] = lv;
        else (FUSED ? lseb : lse_pre)[(int64_t)h * mt.Rb + (row - mt.Nq)] = lv;
      }
    }
    if (NG != 2 || !mt.queue_units) break;
  }
}

// V^T tile: 64 keys of one sequence (zero past its end) x d, written as d rows
// of 64 keys with bits 2 and 3 of the key index swapped inside each 16-key
// group (stored position 8h + 4c + j holds key 8c + 4h + j).
// Ring step (win_lo < win_hi): only tiles that meet the window are written, v
// holds the window's rows (row 0 = position win_lo) and keys outside the window
// are zero. rows_hi >= 0: the rows of v are branch keys, tile ti holds rows
// [vbt_start[ti], vbt_start[ti] + 64), zero from rows_hi on.
template <int HD>
__global__ __launch_bounds__(256) void vt_transpose_bf16_kernel(Meta mt, const bf16 *__restrict__ v,
                                                                bf16 *__restrict__ vt, int win_lo, int win_hi,
                                                                int rows_hi) {
  constexpr int NCH = HD / 8;
  constexpr int LD = HD + 2;  // padded LDS row (elements) against bank conflicts on the column reads
  __shared__ __attribute__((aligned(16))) bf16 t[64 * LD];
  const int hkv = mt.hkv, g = blockIdx.x % hkv, ti = blockIdx.x / hkv;
  const int key_lo = rows_hi >= 0 ? mt.vbt_start[ti] : mt.vt_tiles[2 * ti];
  int lo = key_lo, hi = rows_hi >= 0 ? rows_hi : mt.vt_tiles[2 * ti + 1], base = 0;
  if (win_lo < win_hi) {
    lo = max(lo, win_lo);
    hi = min(hi, win_hi);
    base = win_lo;
    if (lo >= hi) return;  // the whole workgroup
  }
  for (int c = threadIdx.x; c < 64 * NCH; c += 256) {
    const int r = c / NCH, ch = c % NCH;
    const int key = key_lo + r;
    uint4 x = {0u, 0u, 0u, 0u};
    if (key >= lo && key < hi) x = *reinterpret_cast<const uint4 *>(v + ((int64_t)(key - base) * hkv + g) * HD + ch * 8);
    uint32_t *d32 = reinterpret_cast<uint32_t *>(t + r * LD + ch * 8);
    d32[0] = x.x;
    d32[1] = x.y;
    d32[2] = x.z;
    d32[3] = x.w;
  }
  __syncthreads();
  bf16 *dst = vt + ((int64_t)ti * hkv + g) * (HD * 64);
  for (int c = threadIdx.x; c < HD * 8; c += 256) {
    const int d = c >> 3, p8 = c & 7;
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int p = 8 * p8 + e;
      const int key = (p & ~15) | (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1);
      out[e] = t[key * LD + d];
    }
    *reinterpret_cast<bf16x8 *>(dst + d * 64 + 8 * p8) = out;
  }
}

// Every variant is instantiated explicitly: with two values of the bool
// parameter launched from this file, this hipcc emitted the host launch stubs
// of only one of them (the other launch then referenced an undefined stub).
#define BA_FWD_INSTANCE(HD, RING, NG, FUSED)                                                                     \
  template __global__ void main_fwd_bf16_kernel<HD, RING, NG, FUSED>(                                           \
      Meta, const bf16 *, const bf16 *, const bf16 *, const bf16 *, bf16 *, float *, float *, float *, int, int,  \
      float *, float *, const bf16 *, const bf16 *, bf16 *, float *)
BA_FWD_INSTANCE(128, false, 2, false);
BA_FWD_INSTANCE(64, false, 3, false);
BA_FWD_INSTANCE(128, false, 2, true);
BA_FWD_INSTANCE(64, false, 3, true);
BA_FWD_INSTANCE(128, true, 2, false);
BA_FWD_INSTANCE(64, true, 2, false);
#undef BA_FWD_INSTANCE

hipError_t launch_vt_transpose_bf16(const Meta &mt, const bf16 *v, bf16 *vt, hipStream_t st, int win_lo,
                                    int win_hi) {
  if (mt.n_vt_tiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)mt.n_vt_tiles * mt.hkv);
  if (mt.d == 128)
    vt_transpose_bf16_kernel<128><<<grid, 256, 0, st>>>(mt, v, vt, win_lo, win_hi, -1);
  else
    vt_transpose_bf16_kernel<64><<<grid, 256, 0, st>>>(mt, v, vt, win_lo, win_hi, -1);
  return hipGetLastError();
}

hipError_t launch_vbt_transpose_bf16(const Meta &mt, const bf16 *vb, bf16 *vbt, hipStream_t st) {
  if (mt.n_vbt_tiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)mt.n_vbt_tiles * mt.hkv);
  if (mt.d == 128)
    vt_transpose_bf16_kernel<128><<<grid, 256, 0, st>>>(mt, vb, vbt, 0, 0, (int)mt.Rb);
  else
    vt_transpose_bf16_kernel<64><<<grid, 256, 0, st>>>(mt, vb, vbt, 0, 0, (int)mt.Rb);
  return hipGetLastError();
}

hipError_t launch_main_fwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *vt,
                                bf16 *o, float *lse, float *o_pre, float *lse_pre, hipStream_t st) {
  if (mt.n_fwd_pairs == 0) return hipSuccess;
  if (mt.d == 128)
    main_fwd_bf16_kernel<128, false, 2, false><<<(unsigned)((int64_t)mt.n_fwd_pairs * mt.hkv), 512, 0, st>>>(
        mt, q, qb, k, vt, o, lse, o_pre, lse_pre, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  else
    main_fwd_bf16_kernel<64, false, 3, false><<<(unsigned)((int64_t)mt.n_fwd_triples * mt.hkv), 768, 0, st>>>(
        mt, q, qb, k, vt, o, lse, o_pre, lse_pre, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_main_fwd_fused_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *vt,
                                      const bf16 *kb, const bf16 *vbt, bf16 *o, float *lse, bf16 *ob, float *lseb,
                                      hipStream_t st) {
  if (mt.n_fwd_pairs == 0) return hipSuccess;
  if (mt.d == 128)
    main_fwd_bf16_kernel<128, false, 2, true>
        <<<persistent_grid((int64_t)mt.n_fwd_pairs * mt.hkv, mt.queue_units), 512, 0, st>>>(
            mt, q, qb, k, vt, o, lse, nullptr, nullptr, 0, 0, nullptr, nullptr, kb, vbt, ob, lseb);
  else
    main_fwd_bf16_kernel<64, false, 3, true>
        <<<queue_grid((int64_t)mt.n_fwd_triples * mt.hkv, mt.queue_units), 768, 0, st>>>(
            mt, q, qb, k, vt, o, lse, nullptr, nullptr, 0, 0, nullptr, nullptr, kb, vbt, ob, lseb);
  return hipGetLastError();
}

hipError_t launch_ring_fwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k_win, const bf16 *vt,
                                int win_lo, int win_hi, float *o_run, float *lse_run, hipStream_t st) {
  if (mt.n_fwd_pairs == 0 || win_lo >= win_hi) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)mt.n_fwd_pairs * mt.hkv);
  if (mt.d == 128)
    main_fwd_bf16_kernel<128, true, 2, false><<<grid, 512, 0, st>>>(mt, q, qb, k_win, vt, nullptr, nullptr, nullptr,
                                                                 nullptr, win_lo, win_hi, o_run, lse_run, nullptr,
                                                                 nullptr, nullptr, nullptr);
  else
    main_fwd_bf16_kernel<64, true, 2, false><<<grid, 512, 0, st>>>(mt, q, qb, k_win, vt, nullptr, nullptr, nullptr,
                                                                nullptr, win_lo, win_hi, o_run, lse_run, nullptr,
                                                                nullptr, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace ba
