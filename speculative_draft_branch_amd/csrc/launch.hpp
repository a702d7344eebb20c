// Host-side launchers of the device kernels (one per kernel family).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace ba {

hipError_t launch_fill_f32(float *p, int64_t n, float v, hipStream_t st);
hipError_t launch_lse_merge(int64_t rows, int heads, int d, const float *oa, const float *la, const float *ob,
                            const float *lb, void *oo, ba_dtype_t out_dtype, float *lo, hipStream_t st);
hipError_t launch_branch_local_fwd(const Meta &mt, ba_dtype_t dt, const void *qb, const void *kb, const void *vb,
                                   float *o_loc, float *lse_loc, hipStream_t st);
hipError_t launch_branch_local_bwd(const Meta &mt, ba_dtype_t dt, const void *qb, const void *kb, const void *vb,
                                   const void *dob, const float *lseb, const float *delta, float *dq_acc,
                                   void *dkb, void *dvb, hipStream_t st);
// bf16 branch-local kernels on 16x16 MFMA. Forward: the float32 partial
// o_loc/lse_loc of the split path. Backward: dkb, dvb (the branch rows' dQ
// comes from the main dq kernel, which takes the branch keys as its last tiles).
hipError_t launch_branch_fwd_bf16(const Meta &mt, const bf16 *qb, const bf16 *kb, const bf16 *vb, float *o_loc,
                                  float *lse_loc, hipStream_t st);
hipError_t launch_branch_bwd_bf16(const Meta &mt, const bf16 *qb, const bf16 *kb, const bf16 *vb, const bf16 *dob,
                                  const float *lseb, const float *delta, bf16 *dkb, bf16 *dvb, hipStream_t st);
hipError_t launch_bwd_preprocess(const Meta &mt, ba_dtype_t dt, const void *o, const void *d_o, const void *ob,
                                 const void *d_ob, float *delta, hipStream_t st);
hipError_t launch_convert_rows(const float *acc, int64_t n, void *out, ba_dtype_t dt, hipStream_t st);
// float32 main-sequence kernels (plain wave-per-row form)
hipError_t launch_main_fwd_f32(const Meta &mt, const float *q, const float *qb, const float *k, const float *v,
                               float *o, float *lse, float *o_pre, float *lse_pre, hipStream_t st);
hipError_t launch_main_bwd_f32(const Meta &mt, const float *q, const float *qb, const float *k, const float *v,
                               const float *d_o, const float *d_ob, const float *lse, const float *lseb,
                               const float *delta, float *dq_acc, float *dk, float *dv, hipStream_t st);
// bf16 MFMA main-sequence kernels
// V^T tiles of each sequence: [tile][Hkv][d][64 keys], keys of each 16-key group
// stored in MFMA operand-slot order; keys past the sequence end are zero.
// With win_lo < win_hi (a ring step) only the tiles meeting [win_lo, win_hi) are
// written, from v holding the window's rows (row 0 = position win_lo).
hipError_t launch_vt_transpose_bf16(const Meta &mt, const bf16 *v, bf16 *vt, hipStream_t st, int win_lo = 0,
                                    int win_hi = 0);
// Forward with the branch keys as the last key tiles of each unit: final o/ob, lse/lseb.
hipError_t launch_main_fwd_fused_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *vt,
                                      const bf16 *kb, const bf16 *vbt, bf16 *o, float *lse, bf16 *ob, float *lseb,
                                      hipStream_t st);
hipError_t launch_vbt_transpose_bf16(const Meta &mt, const bf16 *vb, bf16 *vbt, hipStream_t st);
hipError_t launch_main_fwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *vt,
                                bf16 *o, float *lse, float *o_pre, float *lse_pre, hipStream_t st);
// One ring step: every row against the main keys of its prefix inside
// [win_lo, win_hi) (k_win: those rows only; vt: their V^T tiles), merged into
// the running float32 o_run [Nq+Rb][Hq][d] / lse_run [Hq][Nq+Rb].
hipError_t launch_ring_fwd_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k_win, const bf16 *vt,
                                int win_lo, int win_hi, float *o_run, float *lse_run, hipStream_t st);
// What the dq kernel stages for the dK/dV kernel (query-tile order) and the
// branch-local backward, besides dq and dqb.
struct BwdStage {
  bf16 *qt, *dot;   // [n_qtiles][Hkv][128][d]: Q * scale * log2(e) (bf16), dO
  float *lt, *dtt;  // [n_qtiles][Hkv][128]: -LSE * log2(e), -D
  int *et;          // [n_qtiles][kTileMetaWords]: row ends, then end_min, end_max, rows
  float *delta;     // [Hq][Nq + Rb]: D = rowsum(dO * O)
};
hipError_t launch_main_bwd_dq_bf16(const Meta &mt, const bf16 *q, const bf16 *qb, const bf16 *k, const bf16 *v,
                                   const bf16 *d_o, const bf16 *d_ob, const float *lse, const float *lseb,
                                   const bf16 *o, const bf16 *ob, const bf16 *kb, const bf16 *vb, bf16 *dq,
                                   bf16 *dqb, const BwdStage &sg, hipStream_t st);
// dkv_acc: null, or float32 dK, dV accumulators [N][Hkv][d] (zeroed) into
// which every workgroup adds instead of writing dk, dv (plans with split key tiles).
hipError_t launch_main_bwd_dkdv_bf16(const Meta &mt, const bf16 *k, const bf16 *v, const bf16 *qt, const bf16 *dot,
                                     const float *lt, const float *dtt, const int *et, bf16 *dk, bf16 *dv,
                                     float *dkv_acc, hipStream_t st);

}  // namespace ba
