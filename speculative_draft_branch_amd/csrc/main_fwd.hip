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
// Per wave (32 query rows): S^T = K Q^T with v_mfma_f32_32x32x16_bf16 so each
// lane owns one query row (lane % 32) and row max/sum need a single exchange
// between the two wave halves; P^T feeds O^T += V^T P^T straight from
// registers, with V read from LDS by the transposing ds_read_b64_tr_b16.
#include <climits>

#include "launch.hpp"

namespace ba {

template <int HD>
__global__ __launch_bounds__(256) void main_fwd_bf16_kernel(Meta mt, const bf16 *__restrict__ q,
                                                            const bf16 *__restrict__ qb,
                                                            const bf16 *__restrict__ k,
                                                            const bf16 *__restrict__ v, bf16 *__restrict__ o,
                                                            float *__restrict__ lse, float *__restrict__ o_pre,
                                                            float *__restrict__ lse_pre) {
  constexpr int BN = 64;        // keys per K/V tile
  constexpr int NCH = HD / 8;   // 16-byte chunks per key row
  constexpr int KS = HD / 16;   // MFMA k-steps over head_dim
  constexpr int DT = HD / 32;   // 32-wide output blocks over head_dim
  __shared__ __attribute__((aligned(16))) bf16 sK[BN * HD];
  __shared__ __attribute__((aligned(16))) bf16 sV[BN * HD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = mt.hkv, G = mt.G;
  const int g = blockIdx.x % hkv;
  const QTile tile = mt.qtiles[mt.fwd_order[blockIdx.x / hkv]];

  // This lane's query row: MFMA row 32*wave + lane%32 = base row * G + head.
  const int mrow = wave * 32 + (lane & 31);
  const int bi = mrow / G, hj = mrow - bi * G;
  int row = -1, end = -1;
  if (bi < tile.nrows) {
    row = mt.tile_row_id[tile.row_begin + bi];
    end = mt.tile_row_end[tile.row_begin + bi];
  }
  const int h = mt.group_heads[g * G + hj];
  const bool is_main = row >= 0 && row < mt.Nq;
  const int64_t roff = row < 0 ? 0
                       : is_main ? ((int64_t)row * mt.hq + h) * HD
                                 : ((int64_t)(row - mt.Nq) * mt.hq + h) * HD;

  // Q as the B operand: lane holds row lane%32, d = 16*ks + 8*(lane/32) + 0..7.
  bf16x8 qf[KS];
  {
    const bf16 *qp = (is_main ? q : qb) + roff + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row >= 0) qf[ks] = *reinterpret_cast<const bf16x8 *>(qp + 16 * ks);
      else qf[ks] = bf16x8{};
    }
  }
  const int wmin = wave_min(row >= 0 ? end : INT_MAX);
  const int wmax = wave_max(end);

  const float sl2 = mt.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // transposed-read coordinates of this lane (as an input lane of its 16-lane group)
  const int grp = lane >> 4, in_j = (lane & 15) >> 2, in_q = lane & 3;

  const int kv_end = tile.end_max;
  for (int k0 = tile.kv_lo; k0 <= kv_end; k0 += BN) {
#pragma unroll
    for (int it = 0; it < BN * NCH / 256; ++it) {
      const int c = tid + it * 256;
      const int r = c / NCH, ch = c % NCH;
      const int key = k0 + r;
      uint4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (key <= kv_end) {
        const int64_t src = ((int64_t)key * hkv + g) * HD + ch * 8;
        kx = *reinterpret_cast<const uint4 *>(k + src);
        vx = *reinterpret_cast<const uint4 *>(v + src);
      }
      const int dst = r * HD + ((ch ^ swz<HD>(r)) << 3);
      *reinterpret_cast<uint4 *>(sK + dst) = kx;
      *reinterpret_cast<uint4 *>(sV + dst) = vx;
    }
    __syncthreads();
    if (k0 <= wmax) {
      // S^T[key][row] for two 32-key blocks.
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = kb * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = 2 * ks + (lane >> 5);
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(sK + r * HD + ((ch ^ swz<HD>(r)) << 3));
          s[kb] = mfma32(a, qf[ks], s[kb]);
        }
      }
      if (k0 + BN - 1 > wmin) {  // some key of this tile lies past some row's prefix end
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
            if (key > end) s[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx * sl2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
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
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      // O^T += V^T P^T. k-step kk covers tile keys 16kk..16kk+15; operand slot
      // 8*half + 4c + j <-> key 16kk + 8c + 4*half + j on both operands.
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key0 = kk * 16 + 4 * (grp >> 1) + in_j;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int d = dt * 32 + (grp & 1) * 16 + 4 * in_q;
          const i16x4 t0 = lds_read_tr(sV + lds_off<HD>(key0, d));
          const i16x4 t1 = lds_read_tr(sV + lds_off<HD>(key0 + 8, d));
          acc[dt] = mfma32(join(t0, t1), pb[kk], acc[dt]);
        }
      }
    }
    __syncthreads();
  }

  const float l_tot = half_sum(l_run);
  if (row >= 0) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + q4 * 8 + (lane >> 5) * 4;
        const f32x4 val = {acc[dt][q4 * 4 + 0] * inv, acc[dt][q4 * 4 + 1] * inv, acc[dt][q4 * 4 + 2] * inv,
                           acc[dt][q4 * 4 + 3] * inv};
        if (is_main) {
          const bf16x4 b = {(bf16)val[0], (bf16)val[1], (bf16)val[2], (bf16)val[3]};
          *reinterpret_cast<bf16x4 *>(o + roff + d) = b;
        } else {
          *reinterpret_cast<f32x4 *>(o_pre + roff + d) = val;
        }
      }
    if (lane < 32) {
      const float lv = (m_run + __log2f(l_tot)) * kLn2;
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
