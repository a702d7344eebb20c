// HBM-bound and small kernels of the branch-attention path: buffer fill, the
// log-sum-exp merge, the branch-local forward/backward, the backward
// preprocess D = rowsum(dO * O), fp32 -> output conversion, and the plain
// float32 main-sequence kernels used for the float32 element type.
#include <cmath>

#include "launch.hpp"

namespace ba {

namespace {

inline unsigned grid_for(int64_t threads, int block) {
  int64_t g = (threads + block - 1) / block;
  return (unsigned)(g < 1 ? 1 : g);
}

template <class T> struct Vec16;  // 16 bytes of T
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int n = 4; };
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int n = 8; };

}  // namespace

// ---------------------------------------------------------------------------
__global__ void fill_f32_kernel(float *__restrict__ p, int64_t n4, float v) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const f32x4 val = {v, v, v, v};
  for (; i < n4; i += stride) reinterpret_cast<f32x4 *>(p)[i] = val;
}

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // n is a multiple of 4 for every buffer the library fills (row sizes are multiples of 4)
  int64_t n4 = n / 4;
  unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 65536);
  fill_f32_kernel<<<grid, 256, 0, st>>>(p, n4, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of two partials (Eq. 2 as named in the evolve.pub review,
// "Scope & Claims"). One thread per 4 elements; the d/4 threads of one
// (row, head) are consecutive lanes of one wave, so every lane reads both LSEs
// before any lane stores the merged LSE (in-place on lse_a is safe).
template <class OutT>
__global__ void lse_merge_kernel(int64_t rows, int heads, int d, const float *oa,
                                 const float *la, const float *__restrict__ ob, const float *__restrict__ lb,
                                 OutT *oo, float *lo) {
  const int per = d >> 2;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t >= rows * heads * per) return;
  const int c = (int)(t % per);
  const int64_t rh = t / per;
  const int h = (int)(rh % heads);
  const int64_t r = rh / heads;
  const float a = la[h * rows + r], b = lb[h * rows + r];
  const float M = fmaxf(a, b);
  const float M0 = (M == -INFINITY) ? 0.0f : M;
  const float wa = expf(a - M0), wb = expf(b - M0);
  const float s = wa + wb;
  const float L = (s == 0.0f) ? -INFINITY : M0 + logf(s);
  const float fa = (s == 0.0f) ? 0.0f : wa / s;
  const float fb = (s == 0.0f) ? 0.0f : wb / s;
  const f32x4 x = reinterpret_cast<const f32x4 *>(oa)[rh * per + c];
  const f32x4 y = reinterpret_cast<const f32x4 *>(ob)[rh * per + c];
  const f32x4 z = fa * x + fb * y;
  OutT *dst = oo + (rh * per + c) * 4;
  if constexpr (sizeof(OutT) == 4) {
    *reinterpret_cast<f32x4 *>(dst) = z;
  } else {
    bf16x4 zb = {(bf16)z[0], (bf16)z[1], (bf16)z[2], (bf16)z[3]};
    *reinterpret_cast<bf16x4 *>(dst) = zb;
  }
  if (c == 0) lo[h * rows + r] = L;
}

hipError_t launch_lse_merge(int64_t rows, int heads, int d, const float *oa, const float *la, const float *ob,
                            const float *lb, void *oo, ba_dtype_t out_dtype, float *lo, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t threads = rows * heads * (d / 4);
  if (out_dtype == BA_F32)
    lse_merge_kernel<float><<<grid_for(threads, 256), 256, 0, st>>>(rows, heads, d, oa, la, ob, lb, (float *)oo, lo);
  else
    lse_merge_kernel<bf16><<<grid_for(threads, 256), 256, 0, st>>>(rows, heads, d, oa, la, ob, lb, (bf16 *)oo, lo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Branch-local forward: each branch query against the keys of its own branch
// only (TTT query j: keys 1..j; block query: the whole block). The branch's K/V
// never leave their anchor (evolve.pub review, "Frequently asked questions":
// branch K/V never communicate). One workgroup per (anchor, kv head); one
// thread per (branch row, q head of the group). Writes the float32 partial.
template <class T, int HD>
__global__ __launch_bounds__(256) void branch_local_fwd_kernel(Meta mt, const T *__restrict__ qb,
                                                               const T *__restrict__ kb,
                                                               const T *__restrict__ vb, float *__restrict__ o_loc,
                                                               float *__restrict__ lse_loc) {
  __shared__ float sK[kMaxBranch * HD];
  __shared__ float sV[kMaxBranch * HD];
  __shared__ float sP[256][kMaxBranch + 1];
  const int64_t m = blockIdx.x / mt.hkv;
  const int g = blockIdx.x % mt.hkv;
  const int b0 = mt.cu_branch[m];
  const int L = mt.cu_branch[m + 1] - b0;
  if (L == 0) return;
  const bool is_block = mt.mode[m] == BA_BLOCK;
  for (int i = threadIdx.x; i < L * HD; i += blockDim.x) {
    const int r = i / HD, e = i % HD;
    const int64_t src = ((int64_t)(b0 + r) * mt.hkv + g) * HD + e;
    sK[i] = to_f32(kb[src]);
    sV[i] = to_f32(vb[src]);
  }
  __syncthreads();
  for (int t0 = 0; t0 < L * mt.G; t0 += blockDim.x) {
    const int t = t0 + threadIdx.x;
    if (t < L * mt.G) {
      const int j = t / mt.G, hj = t % mt.G;
      const int h = mt.group_heads[g * mt.G + hj];
      const int64_t row = b0 + j;
      const T *qp = qb + (row * mt.hq + h) * HD;
      float qv[HD];
      for (int e = 0; e < HD; ++e) qv[e] = to_f32(qp[e]);
      const int nk = is_block ? L : j + 1;
      float mx = -INFINITY;
      for (int kk = 0; kk < nk; ++kk) {
        float s = 0.0f;
        for (int e = 0; e < HD; ++e) s = fmaf(qv[e], sK[kk * HD + e], s);
        s *= mt.scale;
        sP[threadIdx.x][kk] = s;
        mx = fmaxf(mx, s);
      }
      float sum = 0.0f;
      for (int kk = 0; kk < nk; ++kk) sum += expf(sP[threadIdx.x][kk] - mx);
      const float lse = mx + logf(sum);
      for (int kk = 0; kk < nk; ++kk) sP[threadIdx.x][kk] = expf(sP[threadIdx.x][kk] - lse);
      float *op = o_loc + (row * mt.hq + h) * HD;
      for (int e4 = 0; e4 < HD; e4 += 4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int kk = 0; kk < nk; ++kk) {
          const float p = sP[threadIdx.x][kk];
          acc[0] = fmaf(p, sV[kk * HD + e4 + 0], acc[0]);
          acc[1] = fmaf(p, sV[kk * HD + e4 + 1], acc[1]);
          acc[2] = fmaf(p, sV[kk * HD + e4 + 2], acc[2]);
          acc[3] = fmaf(p, sV[kk * HD + e4 + 3], acc[3]);
        }
        *reinterpret_cast<f32x4 *>(op + e4) = acc;
      }
      lse_loc[(int64_t)h * mt.Rb + row] = lse;
    }
  }
}

hipError_t launch_branch_local_fwd(const Meta &mt, ba_dtype_t dt, const void *qb, const void *kb, const void *vb,
                                   float *o_loc, float *lse_loc, hipStream_t st) {
  if (mt.A == 0 || mt.Rb == 0) return hipSuccess;
  const unsigned grid = (unsigned)(mt.A * mt.hkv);
#define BA_LAUNCH(T, HD) \
  branch_local_fwd_kernel<T, HD><<<grid, 256, 0, st>>>(mt, (const T *)qb, (const T *)kb, (const T *)vb, o_loc, lse_loc)
  if (dt == BA_F32) { if (mt.d == 128) BA_LAUNCH(float, 128); else BA_LAUNCH(float, 64); }
  else { if (mt.d == 128) BA_LAUNCH(bf16, 128); else BA_LAUNCH(bf16, 64); }
#undef BA_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Branch-local backward: gradients of the branch-local part through the final
// (merged) LSE, P = exp(S - LSE), dS = P * (dO.V - D). Adds the branch rows'
// local dQ into the float32 accumulator, writes dKb and dVb (only branch rows
// of the same anchor see a branch key). One workgroup per (anchor, kv head).
template <class T, int HD>
__global__ __launch_bounds__(256) void branch_local_bwd_kernel(
    Meta mt, const T *__restrict__ qb, const T *__restrict__ kb, const T *__restrict__ vb,
    const T *__restrict__ dob, const float *__restrict__ lseb, const float *__restrict__ delta,
    float *__restrict__ dq_acc, T *__restrict__ dkb, T *__restrict__ dvb) {
  __shared__ float sK[kMaxBranch * HD], sV[kMaxBranch * HD];
  __shared__ float sQ[kMaxBranch * HD], sdO[kMaxBranch * HD];
  __shared__ float sdK[kMaxBranch * HD], sdV[kMaxBranch * HD];
  __shared__ float sP[kMaxBranch][kMaxBranch + 1], sdS[kMaxBranch][kMaxBranch + 1];
  const int64_t m = blockIdx.x / mt.hkv;
  const int g = blockIdx.x % mt.hkv;
  const int b0 = mt.cu_branch[m];
  const int L = mt.cu_branch[m + 1] - b0;
  if (L == 0) return;
  const bool is_block = mt.mode[m] == BA_BLOCK;
  const int64_t R = mt.Nq + mt.Rb;
  for (int i = threadIdx.x; i < L * HD; i += blockDim.x) {
    const int r = i / HD, e = i % HD;
    const int64_t src = ((int64_t)(b0 + r) * mt.hkv + g) * HD + e;
    sK[i] = to_f32(kb[src]);
    sV[i] = to_f32(vb[src]);
    sdK[i] = 0.0f;
    sdV[i] = 0.0f;
  }
  for (int hj = 0; hj < mt.G; ++hj) {
    const int h = mt.group_heads[g * mt.G + hj];
    __syncthreads();
    for (int i = threadIdx.x; i < L * HD; i += blockDim.x) {
      const int r = i / HD, e = i % HD;
      const int64_t src = ((int64_t)(b0 + r) * mt.hq + h) * HD + e;
      sQ[i] = to_f32(qb[src]);
      sdO[i] = to_f32(dob[src]);
    }
    __syncthreads();
    for (int t = threadIdx.x; t < L * L; t += blockDim.x) {
      const int j = t / L, kk = t % L;
      float p = 0.0f, ds = 0.0f;
      if (is_block || kk <= j) {
        float s = 0.0f, dp = 0.0f;
        for (int e = 0; e < HD; ++e) {
          s = fmaf(sQ[j * HD + e], sK[kk * HD + e], s);
          dp = fmaf(sdO[j * HD + e], sV[kk * HD + e], dp);
        }
        const int64_t row = b0 + j;
        p = expf(s * mt.scale - lseb[(int64_t)h * mt.Rb + row]);
        ds = p * (dp - delta[(int64_t)h * R + mt.Nq + row]);
      }
      sP[j][kk] = p;
      sdS[j][kk] = ds;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < L * HD; t += blockDim.x) {
      const int j = t / HD, e = t % HD;
      float acc = 0.0f;
      for (int kk = 0; kk < L; ++kk) acc = fmaf(sdS[j][kk], sK[kk * HD + e], acc);
      dq_acc[((mt.Nq + b0 + j) * mt.hq + h) * HD + e] += mt.scale * acc;
      // rows of the tile double as keys: key kk = j here
      float dk = 0.0f, dv = 0.0f;
      for (int jj = 0; jj < L; ++jj) {
        dk = fmaf(sdS[jj][j], sQ[jj * HD + e], dk);
        dv = fmaf(sP[jj][j], sdO[jj * HD + e], dv);
      }
      sdK[t] += mt.scale * dk;
      sdV[t] += dv;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < L * HD; i += blockDim.x) {
    const int r = i / HD, e = i % HD;
    const int64_t dst = ((int64_t)(b0 + r) * mt.hkv + g) * HD + e;
    dkb[dst] = from_f32<T>(sdK[i]);
    dvb[dst] = from_f32<T>(sdV[i]);
  }
}

hipError_t launch_branch_local_bwd(const Meta &mt, ba_dtype_t dt, const void *qb, const void *kb, const void *vb,
                                   const void *dob, const float *lseb, const float *delta, float *dq_acc,
                                   void *dkb, void *dvb, hipStream_t st) {
  if (mt.A == 0 || mt.Rb == 0) return hipSuccess;
  const unsigned grid = (unsigned)(mt.A * mt.hkv);
#define BA_LAUNCH(T, HD)                                                                                  \
  branch_local_bwd_kernel<T, HD><<<grid, 256, 0, st>>>(mt, (const T *)qb, (const T *)kb, (const T *)vb, \
                                                       (const T *)dob, lseb, delta, dq_acc, (T *)dkb, (T *)dvb)
  if (dt == BA_F32) { if (mt.d == 128) BA_LAUNCH(float, 128); else BA_LAUNCH(float, 64); }
  else { if (mt.d == 128) BA_LAUNCH(bf16, 128); else BA_LAUNCH(bf16, 64); }
#undef BA_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) per (row, head), float32, layout [Hq, Nq + Rb].
// HD/VEC consecutive lanes share one (row, head) and reduce with shuffles.
template <class T, int HD>
__global__ void bwd_preprocess_kernel(int64_t Nq, int64_t Rb, int hq, const T *__restrict__ o,
                                      const T *__restrict__ d_o, const T *__restrict__ ob,
                                      const T *__restrict__ d_ob, float *__restrict__ delta) {
  typedef typename Vec16<T>::type V;
  constexpr int VEC = Vec16<T>::n, TPR = HD / VEC;
  const int64_t R = Nq + Rb;
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t pair = t / TPR;
  const int c = (int)(t % TPR);
  float acc = 0.0f;
  const bool ok = pair < R * hq;
  int64_t r = 0;
  int h = 0;
  if (ok) {
    r = pair / hq;
    h = (int)(pair % hq);
    const T *po = r < Nq ? o + (r * hq + h) * HD : ob + ((r - Nq) * hq + h) * HD;
    const T *pd = r < Nq ? d_o + (r * hq + h) * HD : d_ob + ((r - Nq) * hq + h) * HD;
    const V a = reinterpret_cast<const V *>(po)[c];
    const V b = reinterpret_cast<const V *>(pd)[c];
#pragma unroll
    for (int i = 0; i < VEC; ++i) acc = fmaf(to_f32(a[i]), to_f32(b[i]), acc);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (ok && c == 0) delta[(int64_t)h * R + r] = acc;
}

hipError_t launch_bwd_preprocess(const Meta &mt, ba_dtype_t dt, const void *o, const void *d_o, const void *ob,
                                 const void *d_ob, float *delta, hipStream_t st) {
  const int64_t R = mt.Nq + mt.Rb;
  if (R == 0) return hipSuccess;
#define BA_LAUNCH(T, HD)                                                                                    \
  bwd_preprocess_kernel<T, HD><<<grid_for(R * mt.hq * (HD / Vec16<T>::n), 256), 256, 0, st>>>(            \
      mt.Nq, mt.Rb, mt.hq, (const T *)o, (const T *)d_o, (const T *)ob, (const T *)d_ob, delta)
  if (dt == BA_F32) { if (mt.d == 128) BA_LAUNCH(float, 128); else BA_LAUNCH(float, 64); }
  else { if (mt.d == 128) BA_LAUNCH(bf16, 128); else BA_LAUNCH(bf16, 64); }
#undef BA_LAUNCH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
template <class OutT>
__global__ void convert_kernel(const float *__restrict__ acc, int64_t n4, OutT *__restrict__ out) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n4; i += stride) {
    const f32x4 x = reinterpret_cast<const f32x4 *>(acc)[i];
    if constexpr (sizeof(OutT) == 4) {
      reinterpret_cast<f32x4 *>(out)[i] = x;
    } else {
      bf16x4 y = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
      reinterpret_cast<bf16x4 *>(out)[i] = y;
    }
  }
}

hipError_t launch_convert_rows(const float *acc, int64_t n, void *out, ba_dtype_t dt, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t n4 = n / 4;
  const unsigned grid = (unsigned)std::min<int64_t>((n4 + 255) / 256, 65536);
  if (dt == BA_F32) convert_kernel<float><<<grid, 256, 0, st>>>(acc, n4, (float *)out);
  else convert_kernel<bf16><<<grid, 256, 0, st>>>(acc, n4, (bf16 *)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// float32 main-sequence forward: one wave per (row, q head), lanes over d.
// Every row attends its visible main keys [row_lo, row_hi] with an online
// softmax; main rows get their final output, branch rows the float32 partial.
template <int HD>
__global__ __launch_bounds__(256) void main_fwd_f32_kernel(Meta mt, const float *__restrict__ q,
                                                           const float *__restrict__ qb, const float *__restrict__ k,
                                                           const float *__restrict__ v, float *__restrict__ o,
                                                           float *__restrict__ lse, float *__restrict__ o_pre,
                                                           float *__restrict__ lse_pre) {
  constexpr int E = HD / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t w = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int64_t R = mt.Nq + mt.Rb;
  if (w >= R * mt.hq) return;
  const int64_t r = w / mt.hq;
  const int idx = (int)(w % mt.hq);  // = g * G + hj
  const int g = idx / mt.G;
  const int h = mt.group_heads[idx];
  const float *qp = r < mt.Nq ? q + (r * mt.hq + h) * HD : qb + ((r - mt.Nq) * mt.hq + h) * HD;
  float qv[E], acc[E];
  for (int e = 0; e < E; ++e) { qv[e] = qp[lane + 64 * e]; acc[e] = 0.0f; }
  float mx = -INFINITY, sum = 0.0f;
  const int lo = mt.row_lo[r], hi = mt.row_hi[r];
  for (int u = lo; u <= hi; ++u) {
    const float *kp = k + ((int64_t)u * mt.hkv + g) * HD;
    const float *vp = v + ((int64_t)u * mt.hkv + g) * HD;
    float s = 0.0f;
    for (int e = 0; e < E; ++e) s = fmaf(qv[e], kp[lane + 64 * e], s);
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    s *= mt.scale;
    const float mn = fmaxf(mx, s);
    const float alpha = expf(mx - mn), p = expf(s - mn);
    sum = sum * alpha + p;
    for (int e = 0; e < E; ++e) acc[e] = fmaf(acc[e], alpha, p * vp[lane + 64 * e]);
    mx = mn;
  }
  const float inv = 1.0f / sum;
  const float l = mx + logf(sum);
  float *op = r < mt.Nq ? o + (r * mt.hq + h) * HD : o_pre + ((r - mt.Nq) * mt.hq + h) * HD;
  for (int e = 0; e < E; ++e) op[lane + 64 * e] = acc[e] * inv;
  if (lane == 0) {
    if (r < mt.Nq) lse[(int64_t)h * mt.Nq + r] = l;
    else lse_pre[(int64_t)h * mt.Rb + (r - mt.Nq)] = l;
  }
}

hipError_t launch_main_fwd_f32(const Meta &mt, const float *q, const float *qb, const float *k, const float *v,
                               float *o, float *lse, float *o_pre, float *lse_pre, hipStream_t st) {
  const int64_t waves = (mt.Nq + mt.Rb) * mt.hq;
  if (waves == 0) return hipSuccess;
  const unsigned grid = grid_for(waves * 64, 256);
  if (mt.d == 128) main_fwd_f32_kernel<128><<<grid, 256, 0, st>>>(mt, q, qb, k, v, o, lse, o_pre, lse_pre);
  else main_fwd_f32_kernel<64><<<grid, 256, 0, st>>>(mt, q, qb, k, v, o, lse, o_pre, lse_pre);
  return hipGetLastError();
}

// float32 main-sequence backward, dQ part: one wave per (row, q head):
// dQ_r = scale * sum_u P_ru (dO_r.V_u - D_r) K_u over the row's main keys,
// with P_ru = exp(scale q_r.k_u - LSE_r) and the final LSE. Overwrites dq_acc.
template <int HD>
__global__ __launch_bounds__(256) void main_bwd_dq_f32_kernel(Meta mt, const float *__restrict__ q,
                                                              const float *__restrict__ qb,
                                                              const float *__restrict__ k, const float *__restrict__ v,
                                                              const float *__restrict__ d_o,
                                                              const float *__restrict__ d_ob,
                                                              const float *__restrict__ lse,
                                                              const float *__restrict__ lseb,
                                                              const float *__restrict__ delta,
                                                              float *__restrict__ dq_acc) {
  constexpr int E = HD / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  const int64_t R = mt.Nq + mt.Rb;
  if (w >= R * mt.hq) return;
  const int64_t r = w / mt.hq;
  const int idx = (int)(w % mt.hq);
  const int g = idx / mt.G;
  const int h = mt.group_heads[idx];
  const bool main = r < mt.Nq;
  const int64_t off = main ? (r * mt.hq + h) * HD : ((r - mt.Nq) * mt.hq + h) * HD;
  const float *qp = (main ? q : qb) + off;
  const float *dp = (main ? d_o : d_ob) + off;
  const float L = main ? lse[(int64_t)h * mt.Nq + r] : lseb[(int64_t)h * mt.Rb + (r - mt.Nq)];
  const float D = delta[(int64_t)h * R + r];
  float qv[E], dov[E], acc[E];
  for (int e = 0; e < E; ++e) { qv[e] = qp[lane + 64 * e]; dov[e] = dp[lane + 64 * e]; acc[e] = 0.0f; }
  for (int u = mt.row_lo[r]; u <= mt.row_hi[r]; ++u) {
    const float *kp = k + ((int64_t)u * mt.hkv + g) * HD;
    const float *vp = v + ((int64_t)u * mt.hkv + g) * HD;
    float s = 0.0f, dpv = 0.0f;
    for (int e = 0; e < E; ++e) {
      s = fmaf(qv[e], kp[lane + 64 * e], s);
      dpv = fmaf(dov[e], vp[lane + 64 * e], dpv);
    }
    for (int o2 = 32; o2 >= 1; o2 >>= 1) {
      s += __shfl_xor(s, o2, 64);
      dpv += __shfl_xor(dpv, o2, 64);
    }
    const float p = expf(s * mt.scale - L);
    const float ds = p * (dpv - D);
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kp[lane + 64 * e], acc[e]);
  }
  float *out = dq_acc + (r * mt.hq + h) * HD;
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = mt.scale * acc[e];
}

// float32 main-sequence backward, dK/dV part: one wave per (main key, kv head):
// dK_u = scale * sum dS_ru q_r and dV_u = sum P_ru dO_r over every (row, q head
// of the group) that sees key u; those rows lie in the key tile's query tiles.
template <int HD>
__global__ __launch_bounds__(256) void main_bwd_dkdv_f32_kernel(Meta mt, const float *__restrict__ q,
                                                                const float *__restrict__ qb,
                                                                const float *__restrict__ k,
                                                                const float *__restrict__ v,
                                                                const float *__restrict__ d_o,
                                                                const float *__restrict__ d_ob,
                                                                const float *__restrict__ lse,
                                                                const float *__restrict__ lseb,
                                                                const float *__restrict__ delta,
                                                                float *__restrict__ dk, float *__restrict__ dv) {
  constexpr int E = HD / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w = (blockIdx.x * (int64_t)blockDim.x + threadIdx.x) >> 6;
  if (w >= (int64_t)mt.n_ktiles * kBwdKeys * mt.hkv) return;
  const int g = (int)(w % mt.hkv);
  const int64_t kt_i = w / mt.hkv / kBwdKeys;
  const int ku = (int)(w / mt.hkv % kBwdKeys);
  const KTile kt = mt.ktiles[kt_i];
  const int u = kt.key_lo + ku;
  if (u >= kt.key_hi) return;
  const int64_t R = mt.Nq + mt.Rb;
  float kv[E], vv[E], adk[E], adv[E];
  for (int e = 0; e < E; ++e) {
    kv[e] = k[((int64_t)u * mt.hkv + g) * HD + lane + 64 * e];
    vv[e] = v[((int64_t)u * mt.hkv + g) * HD + lane + 64 * e];
    adk[e] = adv[e] = 0.0f;
  }
  for (int ti = kt.qt_begin; ti < kt.qt_end; ++ti) {
    const QTile qt = mt.qtiles[ti];
    for (int i = 0; i < qt.nrows; ++i) {
      const int r = mt.tile_row_id[qt.row_begin + i];
      if (mt.tile_row_end[qt.row_begin + i] < u) continue;
      const bool main = r < mt.Nq;
      for (int hj = 0; hj < mt.G; ++hj) {
        const int h = mt.group_heads[g * mt.G + hj];
        const int64_t off = main ? ((int64_t)r * mt.hq + h) * HD : ((int64_t)(r - mt.Nq) * mt.hq + h) * HD;
        const float *qp = (main ? q : qb) + off;
        const float *dp = (main ? d_o : d_ob) + off;
        const float L = main ? lse[(int64_t)h * mt.Nq + r] : lseb[(int64_t)h * mt.Rb + (r - mt.Nq)];
        const float D = delta[(int64_t)h * R + r];
        float qv[E], dov[E], s = 0.0f, dpv = 0.0f;
        for (int e = 0; e < E; ++e) {
          qv[e] = qp[lane + 64 * e];
          dov[e] = dp[lane + 64 * e];
          s = fmaf(qv[e], kv[e], s);
          dpv = fmaf(dov[e], vv[e], dpv);
        }
        for (int o2 = 32; o2 >= 1; o2 >>= 1) {
          s += __shfl_xor(s, o2, 64);
          dpv += __shfl_xor(dpv, o2, 64);
        }
        const float p = expf(s * mt.scale - L);
        const float ds = p * (dpv - D);
        for (int e = 0; e < E; ++e) {
          adk[e] = fmaf(ds, qv[e], adk[e]);
          adv[e] = fmaf(p, dov[e], adv[e]);
        }
      }
    }
  }
  for (int e = 0; e < E; ++e) {
    dk[((int64_t)u * mt.hkv + g) * HD + lane + 64 * e] = mt.scale * adk[e];
    dv[((int64_t)u * mt.hkv + g) * HD + lane + 64 * e] = adv[e];
  }
}

hipError_t launch_main_bwd_f32(const Meta &mt, const float *q, const float *qb, const float *k, const float *v,
                               const float *d_o, const float *d_ob, const float *lse, const float *lseb,
                               const float *delta, float *dq_acc, float *dk, float *dv, hipStream_t st) {
  const int64_t wq = (mt.Nq + mt.Rb) * mt.hq;
  if (wq > 0) {
    const unsigned grid = grid_for(wq * 64, 256);
    if (mt.d == 128)
      main_bwd_dq_f32_kernel<128><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dq_acc);
    else
      main_bwd_dq_f32_kernel<64><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dq_acc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t wk = (int64_t)mt.n_ktiles * kBwdKeys * mt.hkv;
  if (wk > 0) {
    const unsigned grid = grid_for(wk * 64, 256);
    if (mt.d == 128)
      main_bwd_dkdv_f32_kernel<128><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dk, dv);
    else
      main_bwd_dkdv_f32_kernel<64><<<grid, 256, 0, st>>>(mt, q, qb, k, v, d_o, d_ob, lse, lseb, delta, dk, dv);
  }
  return hipGetLastError();
}

}  // namespace ba
