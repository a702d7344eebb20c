/*
 * branch_attn.h -- C ABI of the MI355X (gfx950) speculative-draft branch-attention library.
 *
 * The operator: every query row attends, with one softmax, to the keys it may
 * see. Main-sequence rows see the causal prefix of their own packed sequence.
 * Draft-branch rows (EAGLE-3 training-time-test branches of depth k, or
 * DFlash-style draft blocks) see the causal main prefix up to and including
 * their anchor token plus keys of their own branch: 1..j for TTT query j, the
 * whole block for a block query. The library computes this the way the paper
 * decomposes it: a main-sequence part over the packed causal prefix that emits
 * output plus log-sum-exp, a branch-local part against the branch's own K/V,
 * and the online-softmax (log-sum-exp) merge of the two partials.
 *   - decomposition and merge: evolve.pub review, "Scope & Claims" (section 3.2,
 *     Eq. 2) and "Frequently asked questions" (how branch attention runs under
 *     context parallelism); rcap.io explainer, paragraph on branch attention
 *     under context parallelism;
 *   - packed variable-length batches without padding: rcap.io explainer,
 *     results paragraph on the CP kernel;
 *   - branches hang off the main sequence and never extend it: cere-bro wiki,
 *     "Mechanism".
 *
 * Conventions for every entry point
 *   - Tensors are row-major with head_dim contiguous:
 *       q, o, do      [num_q, Hq, d]       k, v, dk, dv    [N, Hkv, d]
 *       qb, ob, dob   [Rb, Hq, d]          kb, vb, dkb, dvb [Rb, Hkv, d]
 *     N = cu_seqlens[num_seqs] main key rows; Rb = total branch rows. Branch
 *     row b is both a query (qb[b]) and a key/value (kb[b], vb[b]).
 *   - LSE buffers are float32 [Hq, rows] (head-major), natural log of
 *     sum(exp(scale * q.k)) over the keys the row sees.
 *   - Element type: BA_BF16 (bfloat16) or BA_F32 for q/k/v/o and gradients;
 *     accumulation is always float32.
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned. Problem
 *     description arrays (ba_problem_t) are HOST pointers.
 *   - Work is enqueued on the caller's stream, in order, and is asynchronous.
 *     The library never allocates or frees device memory and never
 *     synchronizes a stream; the caller owns every buffer, including the
 *     workspace, and must keep them alive until the stream has run the work.
 *   - Workspaces must be ordinary (coarse-grained) device memory, as from
 *     hipMalloc or a torch CUDA tensor: the backward of plans with split key
 *     tiles adds into the workspace with float32 atomics that assume it, and
 *     the bf16 forward and backward kernels take their work items from
 *     counters in the workspace (reset by the call itself). A workspace holds
 *     one call's state: calls that may overlap in time need separate ones.
 *   - Errors are status codes; no C++ exception crosses this boundary. A
 *     non-OK status leaves a message for ba_last_error() (thread-local).
 *     NaN/Inf in the data are propagated, never checked.
 */
#ifndef BRANCH_ATTN_H
#define BRANCH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BA_ABI_VERSION 1

typedef enum {
  BA_OK = 0,
  BA_EINVAL = 1,        /* malformed problem or bad pointer/size argument */
  BA_EUNSUPPORTED = 2,  /* well-formed but outside what the kernels handle (e.g. head_dim) */
  BA_EWORKSPACE = 3,    /* workspace missing or smaller than ba_workspace_bytes() */
  BA_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} ba_status_t;

typedef enum { BA_F32 = 0, BA_BF16 = 1 } ba_dtype_t;

/* Branch modes. TTT: query j (1-based) of the branch sees branch keys 1..j.
 * BLOCK: every query of the block sees all keys of the block. */
typedef enum { BA_TTT = 0, BA_BLOCK = 1 } ba_mode_t;

/* Host-side description of one packed batch. Every array is a HOST pointer and
 * is copied by ba_plan_create(); the caller may free it afterwards. */
typedef struct {
  ba_dtype_t dtype;          /* element type of every q/k/v/o/gradient tensor of calls using the plan */
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;          /* d: 64 or 128 */
  float softmax_scale;       /* 0 -> 1/sqrt(head_dim) */
  const int32_t *kv_head_of; /* [Hq] kv head of each q head, every kv head serving Hq/Hkv q heads;
                                NULL -> contiguous groups, kv_head_of[h] = h / (Hq/Hkv) */
  int32_t num_seqs;          /* S >= 1 */
  const int32_t *cu_seqlens; /* [S+1] packed sequence offsets: cu[0] = 0, non-decreasing */
  int32_t num_q;             /* number of main query rows; ignored when q_pos == NULL */
  const int32_t *q_pos;      /* [num_q] strictly increasing packed positions in [0, N) of the main
                                query rows; NULL -> every position (num_q = N) */
  int32_t num_anchors;       /* A >= 0 */
  const int32_t *anchors;    /* [A] strictly increasing packed positions in [0, N) */
  const int32_t *cu_branch;  /* [A+1] branch row offsets: cu_branch[0] = 0, non-decreasing, each
                                branch at most 32 rows; NULL -> uniform branch_len */
  int32_t branch_len;        /* TTT depth / block size of every branch when cu_branch == NULL */
  const uint8_t *mode;       /* [A] ba_mode_t per anchor; NULL -> uniform_mode */
  ba_mode_t uniform_mode;
} ba_problem_t;

typedef struct ba_plan ba_plan_t; /* opaque, host memory, immutable after creation */

/* Validate a problem and build its execution plan: per-row key ranges, query
 * tiles grouped by prefix end, key tiles for the backward pass, and the
 * longest-first launch orders. Pure host work, no GPU involved.
 * Returns BA_EINVAL for a malformed problem (non-monotone offsets, positions
 * out of range or unsorted, Hq % Hkv != 0, an unbalanced kv_head_of, a branch
 * longer than 32 rows, bad mode), BA_EUNSUPPORTED for head_dim not in {64,128}.
 * On success *out owns a plan to release with ba_plan_destroy(). */
ba_status_t ba_plan_create(const ba_problem_t *problem, ba_plan_t **out);
void ba_plan_destroy(ba_plan_t *plan);

/* Workspace bytes a call needs: pass 0 = branch_attn_fwd, 1 = branch_attn_bwd,
 * 2 = ba_main_fwd / ba_branch_local_fwd / the split-path entry points. */
size_t ba_workspace_bytes(const ba_plan_t *plan, int pass);

/* Sizes derived by the plan: [0] N main key rows, [1] num_q main query rows,
 * [2] Rb branch rows, [3] number of forward query tiles, [4] number of
 * backward key tiles. Returns BA_EINVAL on NULL arguments. */
ba_status_t ba_plan_sizes(const ba_plan_t *plan, int64_t out[5]);

/* Visible (row, key) pairs per q head: [0] main rows x main keys, [1] branch
 * rows x main keys, [2] branch rows x branch keys. The algorithmic flop count of
 * a forward pass is 4 * d * Hq * (sum of the three). */
ba_status_t ba_plan_pairs(const ba_plan_t *plan, int64_t out[3]);

/* Forward pass: o/lse for main rows, ob/lseb for branch rows (merged result).
 * BA_BF16: the metadata upload, the transposes of V and of the branch V, and
 * one kernel in which every row attends its causal main prefix and then, as
 * the last key tiles of the same online softmax, its own branch's keys, so the
 * log-sum-exp merge of the two parts happens inside that pass (cere-bro wiki,
 * "Mechanism": the branch part rides in the same ring pass) and no partial
 * reaches HBM. BA_F32: the main-sequence kernel (float32 partial for branch
 * rows), the branch-local kernel and lse_merge.
 * workspace: device buffer of ws_bytes >= ba_workspace_bytes(plan, 0). */
ba_status_t branch_attn_fwd(const ba_plan_t *plan,
                            const void *q, const void *k, const void *v,
                            const void *qb, const void *kb, const void *vb,
                            void *o, float *lse, void *ob, float *lseb,
                            void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): branch_attn_fwd without a
 * workspace argument. Its scratch (plan metadata, work counters, transposed V
 * tiles; for float32 plans the float32 partials) lives in a fixed array of
 * ba_fwd_noalloc_max_bytes() = 64 MiB of device memory per GPU, which the
 * library holds from its first use on that GPU until the process ends; the
 * call allocates and frees nothing. Problems whose ba_workspace_bytes(plan, 0)
 * exceeds that size return BA_EWORKSPACE without enqueuing work. Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race, so serialize them.
 * Results are identical to branch_attn_fwd's. Arguments as branch_attn_fwd. */
ba_status_t branch_attn_fwd_noalloc(const ba_plan_t *plan,
                                    const void *q, const void *k, const void *v,
                                    const void *qb, const void *kb, const void *vb,
                                    void *o, float *lse, void *ob, float *lseb, void *stream);
size_t ba_fwd_noalloc_max_bytes(void);

/* Backward pass: exact gradients of the merged forward, given the forward's
 * outputs (o, lse, ob, lseb) and the upstream gradients (d_o, d_ob). Every
 * gradient buffer is overwritten, not accumulated. The merge needs no backward
 * of its own: both parts are differentiated through the final LSE.
 * Definition: the merged forward is one softmax over the union of each row's
 * main-prefix and branch keys (rcap.io explainer, paragraph on branch attention
 * under context parallelism: the two partials are joined by the same
 * log-sum-exp step ring attention uses, leaving the numerics unchanged; evolve.pub
 * review, "Scope & Claims", section 3.2 and Eq. 2). The pages print no
 * backward; this is the exact gradient of that softmax:
 *   P = exp(S - LSE), D = rowsum(dO * O), dS = P * (dO V^T - D),
 *   dQ = scale dS K, dK = scale dS^T Q and dV = P^T dO summed over the q heads
 *   of each kv head, for main and branch keys alike.
 * workspace: ws_bytes >= ba_workspace_bytes(plan, 1). */
ba_status_t branch_attn_bwd(const ba_plan_t *plan,
                            const void *q, const void *k, const void *v,
                            const void *qb, const void *kb, const void *vb,
                            const void *o, const float *lse, const void *ob, const float *lseb,
                            const void *d_o, const void *d_ob,
                            void *dq, void *dk, void *dv, void *dqb, void *dkb, void *dvb,
                            void *workspace, size_t ws_bytes, void *stream);

/* Online-softmax merge of two partial results over disjoint key sets (Eq. 2 as
 * named in the evolve.pub review, "Scope & Claims"):
 *   L = M + log(exp(La - M) + exp(Lb - M)), M = max(La, Lb);
 *   O = exp(La - L) * Oa + exp(Lb - L) * Ob.
 * o_a, o_b: float32 [rows, heads, head_dim]; lse_a, lse_b, lse_out: float32
 * [heads, rows]. An empty partial (O = 0, LSE = -inf) is the identity; two empty
 * partials give O = 0, LSE = -inf (never NaN). o_out has out_dtype; it may
 * alias o_a when out_dtype is BA_F32, and lse_out may alias lse_a.
 * head_dim must be a multiple of 4. */
ba_status_t lse_merge(int64_t rows, int32_t heads, int32_t head_dim,
                      const float *o_a, const float *lse_a, const float *o_b, const float *lse_b,
                      void *o_out, ba_dtype_t out_dtype, float *lse_out, void *stream);

/* Split path, the pieces branch_attn_fwd chains (exposed for tests and for
 * callers that merge elsewhere). Both upload the plan metadata into the
 * workspace (ws_bytes >= ba_workspace_bytes(plan, 2)).
 * The split is the paper's decomposition: a main-sequence part over the packed
 * causal prefix that emits output plus log-sum-exp, and a branch-local part
 * against K/V that never leave the branch's anchor, joined by Eq. 2 (evolve.pub
 * review, "Scope & Claims", section 3.2 and Eq. 2, and "Frequently asked
 * questions" on branch attention under context parallelism; rcap.io explainer,
 * paragraph on branch attention under context parallelism).
 * ba_main_fwd: every row against its causal main prefix: final o/lse for main
 * rows, float32 partial o_pre [Rb,Hq,d] / lse_pre [Hq,Rb] for branch rows.
 * ba_branch_local_fwd: branch rows against their own branch keys only:
 * float32 partial o_loc [Rb,Hq,d] / lse_loc [Hq,Rb]. */
ba_status_t ba_main_fwd(const ba_plan_t *plan, const void *q, const void *qb,
                        const void *k, const void *v,
                        void *o, float *lse, float *o_pre, float *lse_pre,
                        void *workspace, size_t ws_bytes, void *stream);
ba_status_t ba_branch_local_fwd(const ba_plan_t *plan, const void *qb, const void *kb, const void *vb,
                                float *o_loc, float *lse_loc,
                                void *workspace, size_t ws_bytes, void *stream);

/* One step of a context-parallel ring, forward, main keys only (evolve.pub
 * review, section 3.2 and Eq. 2; rcap.io explainer, ring attention: each rank
 * receives a chunk of the main K/V per step and merges the partial result by
 * the log-sum-exp step). Every row -- main rows 0..Nq-1, then branch rows
 * Nq..Nq+Rb-1 -- attends the main keys of its causal prefix whose packed
 * positions lie in the window [win_lo, win_hi), and that partial is merged
 * into the running float32 result in place:
 *   o_run [Nq+Rb, Hq, d], lse_run [Hq, Nq+Rb] (natural-log LSE).
 * Start from o_run = 0, lse_run = -inf. After steps whose windows tile [0, N),
 * in any order, o_run/lse_run equal ba_main_fwd's o, lse (main rows) and
 * o_pre, lse_pre (branch rows) up to rounding; the branch-local part is not
 * included (it never leaves the rank) and joins with lse_merge.
 * k_win, v_win: bf16 [win_hi - win_lo, Hkv, d], the K/V rows of the window
 * only (row 0 = position win_lo), as a ring delivers them. The window need not
 * align with sequences or tiles. A row that sees no key of the window keeps
 * its running value; an empty window (win_lo == win_hi) enqueues nothing.
 * Rows are updated without atomics: calls that overlap on one o_run race.
 * BA_BF16 plans only (BA_EUNSUPPORTED otherwise); BA_EINVAL unless
 * 0 <= win_lo <= win_hi <= N. workspace: ws_bytes >= ba_workspace_bytes(plan, 2). */
ba_status_t ba_ring_step_fwd(const ba_plan_t *plan, const void *q, const void *qb,
                             const void *k_win, const void *v_win, int64_t win_lo, int64_t win_hi,
                             float *o_run, float *lse_run,
                             void *workspace, size_t ws_bytes, void *stream);

/* Opt-in per-kernel timing for profiling: while enabled, every kernel launch
 * and metadata upload of the library is bracketed by HIP events recorded on the
 * call's stream. ba_timing_read() waits for the recorded events (not for the
 * stream) and returns, for kernel id 0 <= id < ba_timing_kernels(), the summed
 * duration in milliseconds and the number of launches since the last reset.
 * Disabled by default; enabling adds two event records per launch. Process-wide
 * and thread-safe; ba_timing_reset() drops every record. */
ba_status_t ba_timing_enable(int on);
ba_status_t ba_timing_reset(void);
int ba_timing_kernels(void);
const char *ba_timing_kernel_name(int id);
ba_status_t ba_timing_read(int id, double *total_ms, int64_t *launches);

const char *ba_status_str(ba_status_t status);
const char *ba_last_error(void);
int ba_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BRANCH_ATTN_H */
