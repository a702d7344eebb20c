// Branch-local attention on bf16 MFMA (gfx950): every draft-branch query
// against the K/V of its own branch only (a TTT query at depth j sees branch
// keys 1..j, a block query sees the whole block). Branch K/V never leave their
// anchor and never join the main-sequence tiles (evolve.pub review,
// "Frequently asked questions"; rcap.io explainer, paragraph on branch
// attention under context parallelism).
//
// One wave (one workgroup) per (anchor, kv head): the anchor's L <= 32 keys
// and its L x G query vectors (branch row j, q head hj of the group, query
// index j*G + hj) in blocks of 16. The products are tiny, so they run on the
// 16x16 MFMA shapes: S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with K and Q rows
// loaded straight from HBM as operands (lane l: row l%16, d 8*(l/16)..+7 of a
// 32-wide d step), which leaves lane l holding query l%16 against keys
// 4*(l/16)..+3 of each 16-key block; the contractions over keys or queries use
// v_mfma_f32_16x16x16bf16_1k, whose transposed operands come from rows staged
// in LDS through the transposing LDS read.
//
// These kernels serve the split path: the forward writes the branch-local
// partial (O_loc, LSE_loc) that lse_merge joins with the main-prefix partial
// (Eq. 2 as named in the evolve.pub review, "Scope & Claims"); the merged
// forward of branch_attn_fwd instead takes the branch keys as the last key
// tiles of the main kernel. The backward gives the branch keys' dK and dV,
// summed over the anchor's queries; those queries' dQ, branch part included,
// comes from the main dq kernel, which takes the branch keys as its last key
// tiles.
#include <cmath>

#include "launch.hpp"

namespace ba {

namespace {

__device__ __forceinline__ f32x4 mfma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16k16(i16x4 a, i16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Transposed 16 x 16 operand from a row-major bf16 LDS block (row stride LD
// elements): lane l receives column c0 + l%16 of rows r0 + 4*(l/16) .. +3, the
// operand of a 16x16x16 MFMA whose k index runs along the LDS rows. Within each
// 16-lane group, input lane t addresses row r0 + 4*(l/16) + t/4, columns
// c0 + 4*(t%4) .. +3.
template <int LD>
__device__ __forceinline__ i16x4 tr16(const bf16 *tile, int r0, int c0, int lane) {
  const int t = lane & 15;
  const bf16 *p = tile + (r0 + 4 * (lane >> 4) + (t >> 2)) * LD + c0 + 4 * (t & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
}

__device__ __forceinline__ float xor16_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float xor16_sum(float x) {
  x += __shfl_xor(x, 16, 64);
  return x + __shfl_xor(x, 32, 64);
}

__device__ __forceinline__ i16x4 pack4(float a, float b, float c, float d) {
  const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  return __builtin_bit_cast(i16x4, v);
}

// The anchor/kv-head pair of this workgroup; false when the anchor belongs to
// the other key-block variant (KB = 1 takes L <= 16, KB = 2 takes 17..32) or
// has no rows.
template <int KB>
__device__ __forceinline__ bool branch_of(const Meta &mt, int64_t &m, int &g, int &b0, int &L) {
  m = (int64_t)blockIdx.x / mt.hkv;
  g = (int)((int64_t)blockIdx.x - m * mt.hkv);
  b0 = mt.cu_branch[m];
  L = mt.cu_branch[m + 1] - b0;
  return L > 0 && (KB == 2) == (L > 16);
}

// Row-major [KB*16][LD] copy of the anchor's rows of a [rows][Hkv][HD] tensor;
// rows past L are zero.
template <int HD, int KB, int LD>
__device__ __forceinline__ void stage_branch_rows(bf16 *dst, const bf16 *__restrict__ src, int b0, int L, int hkv, int g,
                                           int lane) {
  constexpr int CH = HD / 8;  // 16-byte chunks per row
#pragma unroll
  for (int c = lane; c < KB * 16 * CH; c += 64) {
    const int r = c / CH, e = (c - r * CH) * 8;
    bf16x8 v = {};
    if (r < L) v = *reinterpret_cast<const bf16x8 *>(src + ((int64_t)(b0 + r) * hkv + g) * HD + e);
    *reinterpret_cast<bf16x8 *>(dst + r * LD + e) = v;
  }
}

}  // namespace

// Forward: the branch-local partial (o_loc float32, lse_loc) of the split path.
template <int HD, int KB>
__global__ __launch_bounds__(64) void branch_fwd_bf16_kernel(Meta mt, const bf16 *__restrict__ qb,
                                                             const bf16 *__restrict__ kb, const bf16 *__restrict__ vb,
                                                             float *__restrict__ o_loc, float *__restrict__ lse_loc) {
  constexpr int LD = HD + 8;  // LDS row stride (elements): rows 16 bytes apart in bank order
  constexpr int KS = HD / 32, DT = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16 sV[KB * 16 * LD];
  const int lane = threadIdx.x;
  int64_t m;
  int g, b0, L;
  if (!branch_of<KB>(mt, m, g, b0, L)) return;  // the whole workgroup (one wave)
  const int G = mt.G, NQ = L * G, hq = mt.hq;
  const bool blk = mt.mode[m] == BA_BLOCK;
  const float sl2 = mt.scale * kLog2e;

  stage_branch_rows<HD, KB, LD>(sV, vb, b0, L, mt.hkv, g, lane);
  // K as the A operand of S^T: lane holds key kb*16 + lane%16, d 32*ks + 8*(lane/16) .. +7.
  bf16x8 kf[KB][KS];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int key = b * 16 + (lane & 15);
    const bf16 *kp = kb + ((int64_t)(b0 + key) * mt.hkv + g) * HD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kf[b][ks] = key < L ? *reinterpret_cast<const bf16x8 *>(kp + 32 * ks) : bf16x8{};
  }
  __syncthreads();

  for (int q0 = 0; q0 < NQ; q0 += 16) {
    const int qi = q0 + (lane & 15);
    const bool qv = qi < NQ;
    const int j = qv ? qi / G : 0, hj = qv ? qi - j * G : 0;
    const int h = mt.group_heads[g * G + hj];
    const int64_t row = b0 + j;
    const int64_t roff = (row * hq + h) * HD;
    f32x4 s[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) s[b] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qf = qv ? *reinterpret_cast<const bf16x8 *>(qb + roff + 32 * ks + 8 * (lane >> 4)) : bf16x8{};
#pragma unroll
      for (int b = 0; b < KB; ++b) s[b] = mfma16k32(kf[b][ks], qf, s[b]);
    }
    // lane: query qi against keys b*16 + 4*(lane/16) + i; softmax in base 2.
    float mx = -INFINITY;
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = b * 16 + 4 * (lane >> 4) + i;
        const bool vis = key < L && (blk || key <= j);
        s[b][i] = vis ? s[b][i] * sl2 : -INFINITY;
        mx = fmaxf(mx, s[b][i]);
      }
    mx = xor16_max(mx);  // finite: key 0 is visible to every query
    float sum = 0.0f;
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += fast_exp2(s[b][i] - mx);
    sum = xor16_sum(sum);
    const float lse2 = mx + __log2f(sum);
    i16x4 pk[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b)
      pk[b] = pack4(fast_exp2(s[b][0] - lse2), fast_exp2(s[b][1] - lse2), fast_exp2(s[b][2] - lse2),
                    fast_exp2(s[b][3] - lse2));
    const float lse_l = lse2 * kLn2;
    // O^T = V^T P^T per 16-wide d block: lane holds query qi, d = dt*16 + 4*(lane/16) .. +3.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      f32x4 o = {};
#pragma unroll
      for (int b = 0; b < KB; ++b) o = mfma16k16(tr16<LD>(sV, b * 16, dt * 16, lane), pk[b], o);
      const int64_t off = roff + dt * 16 + 4 * (lane >> 4);
      if (qv) *reinterpret_cast<f32x4 *>(o_loc + off) = o;
    }
    if (qv && lane < 16) lse_loc[(int64_t)h * mt.Rb + row] = lse_l;
  }
}

// Backward through the final (merged) LSE: P = exp(S - LSE), dS = P (dP - D);
// dKb = scale dS^T Q and dVb = P^T dO summed over the anchor's queries.
template <int HD, int KB>
__global__ __launch_bounds__(64) void branch_bwd_bf16_kernel(Meta mt, const bf16 *__restrict__ qb,
                                                             const bf16 *__restrict__ kb, const bf16 *__restrict__ vb,
                                                             const bf16 *__restrict__ dob,
                                                             const float *__restrict__ lseb,
                                                             const float *__restrict__ delta,
                                                             bf16 *__restrict__ dkb, bf16 *__restrict__ dvb) {
  constexpr int LD = HD + 8;
  constexpr int LP = KB * 16 + 4;  // row stride of the P and dS blocks
  constexpr int KS = HD / 32, DT = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16 sQ[16 * LD];
  __shared__ __attribute__((aligned(16))) bf16 sdO[16 * LD];
  __shared__ __attribute__((aligned(16))) bf16 sP[16 * LP];
  __shared__ __attribute__((aligned(16))) bf16 sdS[16 * LP];
  const int lane = threadIdx.x;
  int64_t m;
  int g, b0, L;
  if (!branch_of<KB>(mt, m, g, b0, L)) return;
  const int G = mt.G, NQ = L * G, hq = mt.hq;
  const bool blk = mt.mode[m] == BA_BLOCK;
  const float sl2 = mt.scale * kLog2e;
  const int64_t R = mt.Nq + mt.Rb;

  // K and V as A operands of S^T and dP^T (lane: key b*16 + lane%16, d 32*ks + 8*(lane/16) .. +7).
  bf16x8 kf[KB][KS], vf[KB][KS];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int key = b * 16 + (lane & 15);
    const int64_t off = ((int64_t)(b0 + key) * mt.hkv + g) * HD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[b][ks] = key < L ? *reinterpret_cast<const bf16x8 *>(kb + off + 32 * ks) : bf16x8{};
      vf[b][ks] = key < L ? *reinterpret_cast<const bf16x8 *>(vb + off + 32 * ks) : bf16x8{};
    }
  }
  // dK^T and dV^T accumulators: lane holds key b*16 + lane%16, d = dt*16 + 4*(lane/16) .. +3.
  f32x4 dk[KB][DT], dv[KB][DT];
#pragma unroll
  for (int b = 0; b < KB; ++b)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[b][dt] = f32x4{};
      dv[b][dt] = f32x4{};
    }

  for (int q0 = 0; q0 < NQ; q0 += 16) {
    const int qi = q0 + (lane & 15);
    const bool qv = qi < NQ;
    const int j = qv ? qi / G : 0, hj = qv ? qi - j * G : 0;
    const int h = mt.group_heads[g * G + hj];
    const int64_t row = b0 + j;
    const int64_t roff = (row * hq + h) * HD;
    __syncthreads();  // the previous block's LDS reads are done
    f32x4 s[KB], dp[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      s[b] = f32x4{};
      dp[b] = f32x4{};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int e = 32 * ks + 8 * (lane >> 4);
      const bf16x8 qf = qv ? *reinterpret_cast<const bf16x8 *>(qb + roff + e) : bf16x8{};
      const bf16x8 df = qv ? *reinterpret_cast<const bf16x8 *>(dob + roff + e) : bf16x8{};
      *reinterpret_cast<bf16x8 *>(sQ + (lane & 15) * LD + e) = qf;
      *reinterpret_cast<bf16x8 *>(sdO + (lane & 15) * LD + e) = df;
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        s[b] = mfma16k32(kf[b][ks], qf, s[b]);
        dp[b] = mfma16k32(vf[b][ks], df, dp[b]);
      }
    }
    const float l2 = qv ? lseb[(int64_t)h * mt.Rb + row] * kLog2e : 0.0f;
    const float dd = qv ? delta[(int64_t)h * R + mt.Nq + row] : 0.0f;
    i16x4 pk[KB], dsk[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      float p[4], ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = b * 16 + 4 * (lane >> 4) + i;
        const bool vis = qv && key < L && (blk || key <= j);
        p[i] = vis ? fast_exp2(s[b][i] * sl2 - l2) : 0.0f;
        ds[i] = p[i] * (dp[b][i] - dd);
      }
      pk[b] = pack4(p[0], p[1], p[2], p[3]);
      dsk[b] = pack4(ds[0], ds[1], ds[2], ds[3]);
      *reinterpret_cast<i16x4 *>(sP + (lane & 15) * LP + b * 16 + 4 * (lane >> 4)) = pk[b];
      *reinterpret_cast<i16x4 *>(sdS + (lane & 15) * LP + b * 16 + 4 * (lane >> 4)) = dsk[b];
    }
    __syncthreads();  // this block's Q, dO, P and dS rows are in LDS
    // dV^T += dO^T P and dK^T += Q^T dS, contracted over the block's 16 queries.
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const i16x4 pb = tr16<LP>(sP, 0, b * 16, lane);
      const i16x4 db = tr16<LP>(sdS, 0, b * 16, lane);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dv[b][dt] = mfma16k16(tr16<LD>(sdO, 0, dt * 16, lane), pb, dv[b][dt]);
        dk[b][dt] = mfma16k16(tr16<LD>(sQ, 0, dt * 16, lane), db, dk[b][dt]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int key = b * 16 + (lane & 15);
    if (key < L) {
      const int64_t off = ((int64_t)(b0 + key) * mt.hkv + g) * HD + 4 * (lane >> 4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const f32x4 k4 = dk[b][dt] * mt.scale, v4 = dv[b][dt];
        const bf16x4 kk = {(bf16)k4[0], (bf16)k4[1], (bf16)k4[2], (bf16)k4[3]};
        const bf16x4 vv = {(bf16)v4[0], (bf16)v4[1], (bf16)v4[2], (bf16)v4[3]};
        *reinterpret_cast<bf16x4 *>(dkb + off + dt * 16) = kk;
        *reinterpret_cast<bf16x4 *>(dvb + off + dt * 16) = vv;
      }
    }
  }
}

hipError_t launch_branch_fwd_bf16(const Meta &mt, const bf16 *qb, const bf16 *kb, const bf16 *vb, float *o_loc,
                                  float *lse_loc, hipStream_t st) {
  if (mt.A == 0 || mt.Rb == 0) return hipSuccess;
  const unsigned grid = (unsigned)(mt.A * mt.hkv);
#define BA_LAUNCH(HD, KB) branch_fwd_bf16_kernel<HD, KB><<<grid, 64, 0, st>>>(mt, qb, kb, vb, o_loc, lse_loc)
  if (mt.d == 128) {
    BA_LAUNCH(128, 1);
    if (mt.max_branch > 16) BA_LAUNCH(128, 2);
  } else {
    BA_LAUNCH(64, 1);
    if (mt.max_branch > 16) BA_LAUNCH(64, 2);
  }
#undef BA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_branch_bwd_bf16(const Meta &mt, const bf16 *qb, const bf16 *kb, const bf16 *vb, const bf16 *dob,
                                  const float *lseb, const float *delta, bf16 *dkb, bf16 *dvb, hipStream_t st) {
  if (mt.A == 0 || mt.Rb == 0) return hipSuccess;
  const unsigned grid = (unsigned)(mt.A * mt.hkv);
#define BA_LAUNCH(HD, KB) \
  branch_bwd_bf16_kernel<HD, KB><<<grid, 64, 0, st>>>(mt, qb, kb, vb, dob, lseb, delta, dkb, dvb)
  if (mt.d == 128) {
    BA_LAUNCH(128, 1);
    if (mt.max_branch > 16) BA_LAUNCH(128, 2);
  } else {
    BA_LAUNCH(64, 1);
    if (mt.max_branch > 16) BA_LAUNCH(64, 2);
  }
#undef BA_LAUNCH
  return hipGetLastError();
}

}  // namespace ba
