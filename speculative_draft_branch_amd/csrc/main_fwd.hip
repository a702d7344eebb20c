// Main-sequence forward on bf16 MFMA (gfx950): every query row -- main rows and
// draft-branch rows alike -- attends its causal main prefix in its own packed
// sequence, with an online softmax; main rows get their final output and LSE,
// branch rows a float32 partial (O_pre, LSE_pre) that is merged later with the
// branch-local partial by the log-sum-exp reduction (evolve.pub review,
// "Scope & Claims", section 3.2 and Eq. 2; rcap.io explainer, paragraph on
// branch attention under context parallelism). Branch K/V never enter these
// tiles.
//
// Work unit: one query tile (up to 128 MFMA rows = base rows x q heads of one
// kv group, all rows sharing a sequence and sorted by prefix end) against the
// tile's key range [sequence start, largest prefix end], streamed in 64-key
// tiles through LDS. Rows that share a prefix end (a main row, the branch rows
// anchored at the same token, and the q heads of the kv group) share every K/V
// tile. The grid is longest-first; blockIdx % Hkv selects the kv head, so with
// 8 kv heads each XCD streams one kv head's keys.
//
// K/V tiles are double-buffered: global_load_lds writes the next tile straight
// into LDS while the current one is consumed; one barrier per tile.
//
// Per wave (32 query rows): S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so each
// lane owns one query row (lane % 32) and row max/sum need a single exchange
// between the two wave halves; P^T feeds O^T += V^T P^T straight from
// registers, with V read from LDS by the transposing ds_read_b64_tr_b16. The
// running max is only raised (and O, l rescaled) when a row's max grows by more
// than 2^8, which keeps P <= 256 and skips almost every rescale.
#include <climits>

#include "launch.hpp"

namespace ba {

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int HD>
struct FwdState {
  static constexpr int KS = HD / 16;
  static constexpr int DT = HD / 32;
  bf16x8 qf[KS];
  f32x16 acc[DT];
  float m_run, l_run;
  int end, wmin, wmax;
  int grp, in_j, in_q, lane;
};

// One 64-key tile [k0, k0 + 64) of the wave's 32 rows against LDS tiles sK, sV.
template <int HD>
__device__ __forceinline__ void fwd_tile(FwdState<HD> &st, const bf16 *sK, const bf16 *sV, int k0, float sl2) {
  constexpr int KS = FwdState<HD>::KS, DT = FwdState<HD>::DT;
  const int lane = st.lane;
  // S^T[key][row] for two 32-key blocks.
  f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int r = kb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = 2 * ks + (lane >> 5);
      const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sK + r * HD + ((ch ^ swz<HD>(r)) << 3));
      s[kb] = mfma32(a, st.qf[ks], s[kb]);
    }
  }
  if (k0 + 63 > st.wmin) {  // some key of this tile lies past some row's prefix end
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (key > st.end) s[kb][i] = -INFINITY;
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
  const float mt = half_max(mx) * sl2;
  if (__any(mt > st.m_run + kRescaleSlack)) {
    const float m_new = fmaxf(st.m_run, mt);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2(st.m_run - m_new);
    st.l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] *= alpha;
    st.m_run = m_new;
  }
  const float m_use = (st.m_run == -INFINITY) ? 0.0f : st.m_run;
  float rs = 0.0f;
  bf16x8 pb[4];  // P^T operands of the four 16-key k-steps
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[kb][i], sl2, -m_use));
      rs += p;
      pb[kb * 2 + (i >> 3)][i & 7] = (bf16)p;
    }
  st.l_run += rs;
  // O^T += V^T P^T. k-step kk covers tile keys 16kk..16kk+15; operand slot
  // 8*half + 4c + j <-> key 16kk + 8c + 4*half + j on both operands.
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int key0 = kk * 16 + 4 * (st.grp >> 1) + st.in_j;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 32 + (st.grp & 1) * 16 + 4 * st.in_q;
      const i16x4 t0 = lds_read_tr(sV + lds_off<HD>(key0, d));
      const i16x4 t1 = lds_read_tr(sV + lds_off<HD>(key0 + 8, d));
      st.acc[dt] = mfma32(join(t0, t1), pb[kk], st.acc[dt]);
    }
  }
}

}  // namespace

template <int HD>
__global__ __launch_bounds__(256, 2) void main_fwd_bf16_kernel(Meta mt, const bf16 *__restrict__ q,
                                                            const bf16 *__restrict__ qb,
                                                            const bf16 *__restrict__ k,
                                                            const bf16 *__restrict__ v, bf16 *__restrict__ o,
                                                            float *__restrict__ lse, float *__restrict__ o_pre,
                                                            float *__restrict__ lse_pre) {
  constexpr int BN = 64;  // keys per K/V tile
  constexpr int KS = HD / 16, DT = HD / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV1[BN * HD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = mt.hkv, G = mt.G;
  const int g = blockIdx.x % hkv;
  const QTile tile = load_qtile(mt.qtiles + uni(mt.fwd_order[blockIdx.x / hkv]));
  const int kv_lo = tile.kv_lo, kv_end = tile.end_max;
  const int ntiles = (kv_end - kv_lo + BN) / BN;

  // Start fetching the first K/V tile before anything else. K and V share the
  // layout, so one set of per-lane offsets serves both.
  AsyncTile<HD, BN, 256> kvt;
  kvt.init(hkv * HD, tid);
  const bf16 *kg = k + (int64_t)g * HD, *vg = v + (int64_t)g * HD;
  kvt.load(sK0, kg, kv_lo, kv_end);
  kvt.load(sV0, vg, kv_lo, kv_end);

  // This lane's query row: MFMA row 32*wave + lane%32 = base row * G + head.
  FwdState<HD> st;
  const int mrow = wave * 32 + (lane & 31);
  const int bi = mrow / G, hj = mrow - bi * G;
  int row = -1;
  st.end = -1;
  if (bi < tile.nrows) {
    row = mt.tile_row_id[tile.row_begin + bi];
    st.end = mt.tile_row_end[tile.row_begin + bi];
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
  st.m_run = -INFINITY;
  st.l_run = 0.0f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.acc[dt] = f32x16{};
  st.lane = lane;
  st.grp = lane >> 4;
  st.in_j = (lane & 15) >> 2;
  st.in_q = lane & 3;
  const float sl2 = mt.scale * kLog2e;

  // Tiles alternate between the two buffers; the loop is unrolled by two so
  // each buffer is a distinct LDS object.
  for (int j = 0; j < ntiles; j += 2) {
    const int k0 = kv_lo + j * BN;
    wait_async_loads();
    __syncthreads();  // tile j is in buffer 0; every wave is done with buffer 1
    if (j + 1 < ntiles) {
      kvt.load(sK1, kg, k0 + BN, kv_end);
      kvt.load(sV1, vg, k0 + BN, kv_end);
    }
    if (k0 <= st.wmax) fwd_tile<HD>(st, sK0, sV0, k0, sl2);
    if (j + 1 >= ntiles) break;
    wait_async_loads();
    __syncthreads();  // tile j+1 is in buffer 1; every wave is done with buffer 0
    if (j + 2 < ntiles) {
      kvt.load(sK0, kg, k0 + 2 * BN, kv_end);
      kvt.load(sV0, vg, k0 + 2 * BN, kv_end);
    }
    if (k0 + BN <= st.wmax) fwd_tile<HD>(st, sK1, sV1, k0 + BN, sl2);
  }

  const float l_tot = half_sum(st.l_run);
  if (row >= 0) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + q4 * 8 + (lane >> 5) * 4;
        const f32x4 val = {st.acc[dt][q4 * 4 + 0] * inv, st.acc[dt][q4 * 4 + 1] * inv,
                           st.acc[dt][q4 * 4 + 2] * inv, st.acc[dt][q4 * 4 + 3] * inv};
        if (is_main) {
          const bf16x4 b = {(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
          *reinterpret_cast<bf16x4 *>(o + roff + d) = b;
        } else {
          *reinterpret_cast<f32x4 *>(o_pre + roff + d) = val;
        }
      }
    if (lane < 32) {
      const float lv = (st.m_run + __log2f(l_tot)) * kLn2;
      if (is_main) lse[(int64_t)h * mt.Nq + row] = lv;
      else lse_pre[(int64_t)h * mt.Rb + (row - mt.Nq)] = lv;
    }
  }
}

hipError_t launch_main_fwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *v,
                                bf16 *o, float *lse, float *o_pre, float *lse_pre, hipStream_t st) {
  if (mt.n_qtiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)mt.n_qtiles * mt.hkv);
  if (mt.d == 128)
    main_fwd_bf16_kernel<128><<<grid, 256, 0, st>>>(mt, q, qb, k, v, o, lse, o_pre, lse_pre);
  else
    main_fwd_bf16_kernel<64><<<grid, 256, 0, st>>>(mt, q, qb, k, v, o, lse, o_pre, lse_pre);
  return hipGetLastError();
}

}  // namespace ba
