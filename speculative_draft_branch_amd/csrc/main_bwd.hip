// Main-sequence backward on bf16 MFMA (gfx950): gradients of every row's
// attention over its causal main prefix, taken through the row's final (merged)
// LSE, so the log-sum-exp merge needs no backward of its own:
//   P = exp(S - LSE),  dP = dO V^T,  dS = P * (dP - D),  D = rowsum(dO * O),
//   dV += P^T dO,  dK += scale dS^T Q,  dQ += scale dS K.
// (Decomposition and merge: evolve.pub review, "Scope & Claims", section 3.2 and
// Eq. 2; the merged result is one softmax over the union of keys, rcap.io
// explainer, paragraph on branch attention under context parallelism.)
//
// Work unit: 128 main keys of one kv head (one backward key tile) against every
// query tile whose rows may see them; each of the 4 waves owns 32 keys and keeps
// their dK/dV in registers across all query tiles, so each key's gradient is
// written once, summed over the q heads of the group. dQ is accumulated with
// float32 atomics into a workspace buffer, once per workgroup per query tile,
// after the waves' dS blocks are exchanged through LDS.
//
// MFMA layouts (v_mfma_f32_32x32x16_bf16): S = Q K^T puts the key on the lane
// (lane % 32) and 16 query rows in the lane's registers, so P and dS are
// directly the A operand of the dV and dK products; dO and Q enter those
// products through the transposing LDS read.
#include <climits>

#include "launch.hpp"

namespace ba {

template <int HD>
__global__ __launch_bounds__(256) void main_bwd_bf16_kernel(Meta mt, const bf16 *__restrict__ q,
                                                            const bf16 *__restrict__ qb,
                                                            const bf16 *__restrict__ k,
                                                            const bf16 *__restrict__ v,
                                                            const bf16 *__restrict__ d_o,
                                                            const bf16 *__restrict__ d_ob,
                                                            const float *__restrict__ lse,
                                                            const float *__restrict__ lseb,
                                                            const float *__restrict__ delta,
                                                            float *__restrict__ dq_acc, bf16 *__restrict__ dk,
                                                            bf16 *__restrict__ dv) {
  constexpr int BK = kBwdKeys;  // 128 keys per workgroup, 32 per wave
  constexpr int BM = kTileRows; // 128 MFMA rows per query tile
  constexpr int NCH = HD / 8;
  constexpr int KS = HD / 16;
  constexpr int DT = HD / 32;
  static_assert(BK == 128 && BM == 128, "tile shape");
  __shared__ __attribute__((aligned(16))) bf16 sQ[BM * HD];
  __shared__ __attribute__((aligned(16))) bf16 sdO[BM * HD];
  __shared__ __attribute__((aligned(16))) bf16 sK[BK * HD];
  __shared__ __attribute__((aligned(16))) bf16 sdS[BK * BM];  // [key][row], 16-byte chunks swizzled
  __shared__ __attribute__((aligned(16))) float sL2[BM];  // LSE * log2(e); +inf for padding rows
  __shared__ __attribute__((aligned(16))) float sD[BM];
  __shared__ int sEnd[BM];       // prefix end; -1 for padding rows
  __shared__ int64_t sAcc[BM];   // dq_acc element offset of the row; -1 for padding

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hkv = mt.hkv, G = mt.G;
  const int g = blockIdx.x % hkv;
  const KTile kt = mt.ktiles[mt.bwd_order[blockIdx.x / hkv]];
  const int64_t R = mt.Nq + mt.Rb;
  const float sl2 = mt.scale * kLog2e;

  // Stage this workgroup's K tile in LDS (for the dQ product) and keep the
  // wave's own K and V as MFMA B operands: lane holds key 32*wave + lane%32,
  // d = 16*ks + 8*(lane/32) + 0..7.
#pragma unroll
  for (int it = 0; it < BK * NCH / 256; ++it) {
    const int c = tid + it * 256;
    const int r = c / NCH, ch = c % NCH;
    const int key = kt.key_lo + r;
    uint4 kx = {0u, 0u, 0u, 0u};
    if (key < kt.key_hi) kx = *reinterpret_cast<const uint4 *>(k + ((int64_t)key * hkv + g) * HD + ch * 8);
    *reinterpret_cast<uint4 *>(sK + r * HD + ((ch ^ swz<HD>(r)) << 3)) = kx;
  }
  const int my_key = kt.key_lo + wave * 32 + (lane & 31);
  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (my_key < kt.key_hi) {
      const int64_t src = ((int64_t)my_key * hkv + g) * HD + 16 * ks + 8 * (lane >> 5);
      kf[ks] = *reinterpret_cast<const bf16x8 *>(k + src);
      vf[ks] = *reinterpret_cast<const bf16x8 *>(v + src);
    } else {
      kf[ks] = bf16x8{};
      vf[ks] = bf16x8{};
    }
  }
  const int wkey_lo = kt.key_lo + wave * 32;  // first key of this wave

  f32x16 adk[DT], adv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    adk[dt] = f32x16{};
    adv[dt] = f32x16{};
  }
  const int grp = lane >> 4, in_j = (lane & 15) >> 2, in_q = lane & 3;

  for (int qi = kt.qt_begin; qi < kt.qt_end; ++qi) {
    const QTile qt = mt.qtiles[qi];
    __syncthreads();  // previous iteration's LDS reads are done
    {
      // Two threads per MFMA row: row metadata and half of its Q / dO row each.
      const int m = tid >> 1, half = tid & 1;
      const int bi = m / G, hj = m - bi * G;
      const bool ok = bi < qt.nrows;
      int row = -1;
      int64_t qoff = 0;
      if (ok) {
        row = mt.tile_row_id[qt.row_begin + bi];
        const int h = mt.group_heads[g * G + hj];
        const bool is_main = row < mt.Nq;
        qoff = is_main ? ((int64_t)row * mt.hq + h) * HD : ((int64_t)(row - mt.Nq) * mt.hq + h) * HD;
        if (half == 0) {
          const float l = is_main ? lse[(int64_t)h * mt.Nq + row] : lseb[(int64_t)h * mt.Rb + (row - mt.Nq)];
          sL2[m] = l * kLog2e;
          sD[m] = delta[(int64_t)h * R + row];
          sEnd[m] = mt.tile_row_end[qt.row_begin + bi];
          sAcc[m] = ((int64_t)row * mt.hq + h) * HD;
        }
        const bf16 *qp = (is_main ? q : qb) + qoff;
        const bf16 *dp = (is_main ? d_o : d_ob) + qoff;
#pragma unroll
        for (int c = 0; c < NCH / 2; ++c) {
          const int ch = half * (NCH / 2) + c;
          const int dst = m * HD + ((ch ^ swz<HD>(m)) << 3);
          *reinterpret_cast<uint4 *>(sQ + dst) = *reinterpret_cast<const uint4 *>(qp + ch * 8);
          *reinterpret_cast<uint4 *>(sdO + dst) = *reinterpret_cast<const uint4 *>(dp + ch * 8);
        }
      } else {
        if (half == 0) {
          sL2[m] = INFINITY;
          sD[m] = 0.0f;
          sEnd[m] = -1;
          sAcc[m] = -1;
        }
#pragma unroll
        for (int c = 0; c < NCH / 2; ++c) {
          const int ch = half * (NCH / 2) + c;
          const int dst = m * HD + ((ch ^ swz<HD>(m)) << 3);
          *reinterpret_cast<uint4 *>(sQ + dst) = uint4{0u, 0u, 0u, 0u};
          *reinterpret_cast<uint4 *>(sdO + dst) = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
    __syncthreads();

    // Does any row of this query tile end before one of this wave's keys?
    const bool need_mask = qt.end_min < wkey_lo + 31 || wkey_lo + 31 >= kt.key_hi || qt.nrows * G < BM;
    const bool any_visible = qt.end_max >= wkey_lo && wkey_lo < kt.key_hi;
    if (any_visible) {
#pragma unroll
      for (int rb = 0; rb < BM / 32; ++rb) {
        // S and dP for rows 32rb..32rb+31 x the wave's 32 keys.
        f32x16 s = f32x16{}, dp = f32x16{};
        const int ar = rb * 32 + (lane & 31);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = 2 * ks + (lane >> 5);
          const int off = ar * HD + ((ch ^ swz<HD>(ar)) << 3);
          s = mfma32(*reinterpret_cast<const bf16x8 *>(sQ + off), kf[ks], s);
          dp = mfma32(*reinterpret_cast<const bf16x8 *>(sdO + off), vf[ks], dp);
        }
        // element i: row rb*32 + (i/4)*8 + 4*(lane/32) + i%4, key my_key
        bf16x8 pa[2], dsa[2];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r0 = rb * 32 + i4 * 8 + 4 * (lane >> 5);
          const f32x4 l2 = *reinterpret_cast<const f32x4 *>(sL2 + r0);
          const f32x4 dd = *reinterpret_cast<const f32x4 *>(sD + r0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = i4 * 4 + e;
            float p = fast_exp2(fmaf(s[i], sl2, -l2[e]));
            if (need_mask && (sEnd[r0 + e] < my_key || my_key >= kt.key_hi)) p = 0.0f;
            const float ds = p * (dp[i] - dd[e]);
            pa[i >> 3][i & 7] = (bf16)p;
            dsa[i >> 3][i & 7] = (bf16)ds;
          }
        }
        // dV += P^T dO and dK += dS^T Q over these 32 rows (two 16-row k-steps).
        // Operand slot 8*half + 4c + j <-> row 32rb + 16kh + 8c + 4*half + j.
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const int row0 = rb * 32 + kh * 16 + 4 * (grp >> 1) + in_j;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const int d = dt * 32 + (grp & 1) * 16 + 4 * in_q;
            const bf16x8 bo = join(lds_read_tr(sdO + lds_off<HD>(row0, d)), lds_read_tr(sdO + lds_off<HD>(row0 + 8, d)));
            const bf16x8 bq = join(lds_read_tr(sQ + lds_off<HD>(row0, d)), lds_read_tr(sQ + lds_off<HD>(row0 + 8, d)));
            adv[dt] = mfma32(pa[kh], bo, adv[dt]);
            adk[dt] = mfma32(dsa[kh], bq, adk[dt]);
          }
        }
        // Stage dS for the dQ product: sdS[key][row], 4 consecutive rows per write.
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int kl = wave * 32 + (lane & 31);
          const int r0 = rb * 32 + i4 * 8 + 4 * (lane >> 5);
          const bf16x4 val = {dsa[i4 >> 1][(i4 & 1) * 4 + 0], dsa[i4 >> 1][(i4 & 1) * 4 + 1],
                              dsa[i4 >> 1][(i4 & 1) * 4 + 2], dsa[i4 >> 1][(i4 & 1) * 4 + 3]};
          *reinterpret_cast<bf16x4 *>(sdS + lds_off<BM>(kl, r0)) = val;
        }
      }
    } else {
      // No row of this tile sees the wave's keys: its dS block is zero.
#pragma unroll
      for (int rb = 0; rb < BM / 32; ++rb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int kl = wave * 32 + (lane & 31);
          const int r0 = rb * 32 + i4 * 8 + 4 * (lane >> 5);
          *reinterpret_cast<bf16x4 *>(sdS + lds_off<BM>(kl, r0)) = bf16x4{};
        }
    }
    __syncthreads();

    // dQ for rows 32*wave..32*wave+31 against all 128 keys: A = dS (rows x keys)
    // through the transposing read of sdS, B = K (keys x d) through that of sK.
    // Slot 8*half + 4c + j <-> key 16*ks + 8*half + 4c + j.
    // Two passes over halves of head_dim keep the dQ accumulator at DT/2 blocks.
    constexpr int DH = DT > 1 ? DT / 2 : 1;
    const int qrow = wave * 32 + (grp & 1) * 16 + 4 * in_q;
#pragma unroll
    for (int dpass = 0; dpass < DT / DH; ++dpass) {
      f32x16 aq[DH];
#pragma unroll
      for (int dt = 0; dt < DH; ++dt) aq[dt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < BK / 16; ++ks) {
        const int key0 = ks * 16 + 8 * (grp >> 1) + in_j;
        const bf16x8 a = join(lds_read_tr(sdS + lds_off<BM>(key0, qrow)), lds_read_tr(sdS + lds_off<BM>(key0 + 4, qrow)));
#pragma unroll
        for (int dt = 0; dt < DH; ++dt) {
          const int d = (dpass * DH + dt) * 32 + (grp & 1) * 16 + 4 * in_q;
          const bf16x8 b = join(lds_read_tr(sK + lds_off<HD>(key0, d)), lds_read_tr(sK + lds_off<HD>(key0 + 4, d)));
          aq[dt] = mfma32(a, b, aq[dt]);
        }
      }
      // element i of block dt: row 32*wave + (i/4)*8 + 4*(lane/32) + i%4, d = 32dt + lane%32
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = wave * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
        const int64_t base = sAcc[m];
        if (base >= 0) {
#pragma unroll
          for (int dt = 0; dt < DH; ++dt)
            atomicAdd(dq_acc + base + (dpass * DH + dt) * 32 + (lane & 31), mt.scale * aq[dt][i]);
        }
      }
    }
  }

  // dK, dV of the wave's keys: element i of block dt is key 32*wave +
  // (i/4)*8 + 4*(lane/32) + i%4, d = 32dt + lane%32.
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = kt.key_lo + wave * 32 + (i >> 2) * 8 + 4 * (lane >> 5) + (i & 3);
    if (key < kt.key_hi) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int64_t dst = ((int64_t)key * hkv + g) * HD + dt * 32 + (lane & 31);
        dk[dst] = (bf16)(mt.scale * adk[dt][i]);
        dv[dst] = (bf16)adv[dt][i];
      }
    }
  }
}

hipError_t launch_main_bwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *v,
                                const bf16 *d_o, const bf16 *d_ob, const float *lse, const float *lseb,
                                const float *delta, float *dq_acc, bf16 *dk, bf16 *dv, hipStream_t st) {
  if (mt.n_ktiles == 0) return hipSuccess;
  const unsigned grid = (unsigned)((int64_t)mt.n_ktiles * mt.hkv);
  if (mt.d == 128)
    main_bwd_bf16_kernel<128><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dq_acc, dk, dv);
  else
    main_bwd_bf16_kernel<64><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dq_acc, dk, dv);
  return hipGetLastError();
}

}  // namespace ba
