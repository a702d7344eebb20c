// C-ABI entry points: argument checks, metadata upload into the caller's
// workspace, and the stream-ordered kernel sequence of each pass.
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"

using namespace ba;

namespace ba {

unsigned persistent_grid(int64_t items, const int *counters) {
  if (!counters) return (unsigned)items;
  static std::atomic<int> cus[64];  // compute units per device, 0 until read
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cus[dev].load();
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev].store(n);
  }
  return (unsigned)std::min<int64_t>(items, n);
}

}  // namespace ba

namespace {

// ---------------------------------------------------------------------------
// Opt-in per-kernel timing: HIP events recorded on the launch stream.
enum KernelId {
  K_UPLOAD = 0, K_MAIN_FWD, K_BRANCH_LOCAL_FWD, K_LSE_MERGE, K_BWD_PREPROCESS, K_MAIN_BWD_DQ, K_MAIN_BWD_DKDV,
  K_BRANCH_LOCAL_BWD, K_DQ_CONVERT, K_VT_TRANSPOSE, K_RING_FWD, K_VBT_TRANSPOSE, K_COUNT
};
const char *kKernelNames[K_COUNT] = {"metadata_upload", "main_fwd", "branch_local_fwd", "lse_merge",
                                     "bwd_preprocess", "main_bwd_dq", "main_bwd_dkdv", "branch_local_bwd",
                                     "dq_convert",      "vt_transpose", "ring_step_fwd",    "vbt_transpose"};

struct TimingState {
  std::mutex mu;
  std::atomic<bool> on{false};
  struct Rec { int id; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[K_COUNT] = {};
  int64_t launches[K_COUNT] = {};
};
TimingState &timing() {
  static TimingState *t = new TimingState();  // never destroyed: events may outlive static teardown
  return *t;
}

hipEvent_t take_event(TimingState &t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is on.
class Timed {
 public:
  Timed(int id, hipStream_t st) : id_(id), st_(st) {
    TimingState &t = timing();
    if (!t.on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(t.mu);
    a_ = take_event(t);
    b_ = take_event(t);
    if (a_ && b_ && hipEventRecord(a_, st_) == hipSuccess) active_ = true;
  }
  ~Timed() {
    if (!active_) return;
    TimingState &t = timing();
    std::lock_guard<std::mutex> lk(t.mu);
    if (hipEventRecord(b_, st_) == hipSuccess) t.pending.push_back({id_, a_, b_});
  }

 private:
  int id_;
  hipStream_t st_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool active_ = false;
};

void drain(TimingState &t) {
  for (auto &r : t.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.b) == hipSuccess && hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      t.total_ms[r.id] += ms;
      t.launches[r.id] += 1;
    }
    t.pool.push_back(r.a);
    t.pool.push_back(r.b);
  }
  t.pending.clear();
}

Meta make_meta(const ba_plan *pl, const void *ws) {
  const uint8_t *b = static_cast<const uint8_t *>(ws);
  const BlobLayout &L = pl->layout;
  Meta m{};
  m.group_heads = reinterpret_cast<const int32_t *>(b + L.group_heads);
  m.qtiles = reinterpret_cast<const QTile *>(b + L.qtiles);
  m.fwd_order = reinterpret_cast<const int32_t *>(b + L.fwd_order);
  m.fwd_pairs = reinterpret_cast<const int32_t *>(b + L.fwd_pairs);
  m.fwd_triples = reinterpret_cast<const int32_t *>(b + L.fwd_triples);
  m.tile_row_id = reinterpret_cast<const int32_t *>(b + L.tile_row_id);
  m.tile_row_end = reinterpret_cast<const int32_t *>(b + L.tile_row_end);
  m.row_lo = reinterpret_cast<const int32_t *>(b + L.row_lo);
  m.row_hi = reinterpret_cast<const int32_t *>(b + L.row_hi);
  m.cu_branch = reinterpret_cast<const int32_t *>(b + L.cu_branch);
  m.mode = reinterpret_cast<const int32_t *>(b + L.mode);
  m.ktiles = reinterpret_cast<const KTile *>(b + L.ktiles);
  m.bwd_order = reinterpret_cast<const int32_t *>(b + L.bwd_order);
  m.vt_tiles = reinterpret_cast<const int32_t *>(b + L.vt_tiles);
  m.vt_base = reinterpret_cast<const int32_t *>(b + L.vt_base);
  m.brow_lo = reinterpret_cast<const int32_t *>(b + L.brow_lo);
  m.brow_hi = reinterpret_cast<const int32_t *>(b + L.brow_hi);
  m.fwd_pair_bk = reinterpret_cast<const int32_t *>(b + L.fwd_pair_bk);
  m.fwd_triple_bk = reinterpret_cast<const int32_t *>(b + L.fwd_triple_bk);
  m.fwd_unit_bt = reinterpret_cast<const int32_t *>(b + L.fwd_unit_bt);
  m.vbt_start = reinterpret_cast<const int32_t *>(b + L.vbt_start);
  m.N = pl->N;
  m.Nq = pl->Nq;
  m.Rb = pl->Rb;
  m.A = pl->A;
  m.hq = pl->hq;
  m.hkv = pl->hkv;
  m.G = pl->G;
  m.d = pl->d;
  m.rows_per_tile = pl->rows_per_tile;
  m.n_qtiles = pl->n_qtiles;
  m.n_ktiles = pl->n_ktiles;
  m.n_fwd_pairs = pl->n_fwd_pairs;
  m.n_fwd_triples = pl->n_fwd_triples;
  m.n_vt_tiles = pl->n_vt_tiles;
  m.n_vbt_tiles = pl->n_vbt_tiles;
  m.max_branch = pl->max_branch;
  m.scale = pl->scale;
  return m;
}

ba_status_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return BA_OK;
  return set_error(BA_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// A tensor pointer must be non-NULL when the tensor has elements, and 16-byte aligned.
ba_status_t check_ptr(const void *p, int64_t elems, const char *name) {
  if (elems == 0) return BA_OK;
  if (!p) return set_error(BA_EINVAL, std::string(name) + " is NULL");
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return set_error(BA_EINVAL, std::string(name) + " is not 16-byte aligned");
  return BA_OK;
}

ba_status_t check_ws(const ba_plan *pl, const void *ws, size_t ws_bytes, int pass) {
  const size_t need = ba_workspace_bytes(pl, pass);
  if (!ws || ws_bytes < need)
    return set_error(BA_EWORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                         std::to_string(ws ? ws_bytes : 0));
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return set_error(BA_EINVAL, "workspace must be 256-byte aligned");
  return BA_OK;
}

ba_status_t upload(const ba_plan *pl, void *ws, hipStream_t st) {
  Timed tm(K_UPLOAD, st);
  return hip_status(hipMemcpyAsync(ws, pl->blob.data(), pl->blob.size(), hipMemcpyHostToDevice, st),
                    "metadata upload");
}

#define BA_TRY(x)                       \
  do {                                  \
    ba_status_t _s = (x);               \
    if (_s != BA_OK) return _s;         \
  } while (0)
#define BA_HIP(x, what) BA_TRY(hip_status((x), what))

ba_status_t run_main_fwd(const ba_plan *pl, const Meta &mt, const void *q, const void *qb, const void *k,
                         const void *v, void *o, float *lse, float *o_pre, float *lse_pre, void *ws,
                         hipStream_t st) {
  if (pl->dtype == BA_BF16) {
    bf16 *vt = reinterpret_cast<bf16 *>(static_cast<uint8_t *>(ws) + pl->off_vt);
    {
      Timed tv(K_VT_TRANSPOSE, st);
      BA_HIP(launch_vt_transpose_bf16(mt, (const bf16 *)v, vt, st), "V transpose");
    }
    Timed tm(K_MAIN_FWD, st);
    BA_HIP(launch_main_fwd_bf16(mt, (const bf16 *)q, (const bf16 *)qb, (const bf16 *)k, vt, (bf16 *)o, lse, o_pre,
                                lse_pre, st),
           "main-sequence forward");
  } else {
    Timed tm(K_MAIN_FWD, st);
    BA_HIP(launch_main_fwd_f32(mt, (const float *)q, (const float *)qb, (const float *)k, (const float *)v,
                               (float *)o, lse, o_pre, lse_pre, st),
           "main-sequence forward");
  }
  return BA_OK;
}

template <class F>
ba_status_t timed(int id, hipStream_t st, const char *what, F &&f) {
  Timed tm(id, st);
  return hip_status(f(), what);
}

ba_status_t check_plan(const ba_plan *pl) {
  if (!pl) return set_error(BA_EINVAL, "plan is NULL");
  return BA_OK;
}

// Scratch of the allocation-free forward: one array per device, held for the
// life of the process. Host code never passes the array's name to a kernel
// (on the host that name is a stand-in, not a device address); it passes the
// address hipGetSymbolAddress returns, once per device, with that device
// current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

ba_status_t scratch_of_current_device(void **out) {
  int dev = -1;
  BA_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return set_error(BA_EUNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    BA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0)
      return set_error(BA_EHIP, "scratch address is NULL or not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BA_OK;
}

// 32-bit words of the work-counter region (the whole region, a multiple of 64,
// which the fill kernel's 4-word steps cover exactly).
int64_t queue_words(const ba_plan *pl) { return (int64_t)(pl->off_vt - pl->off_queue) / 4; }

// The forward pass after argument checks: workspace of at least
// ba_workspace_bytes(plan, 0) bytes.
ba_status_t fwd_body(const ba_plan *pl, const void *q, const void *k, const void *v, const void *qb, const void *kb,
                     const void *vb, void *o, float *lse, void *ob, float *lseb, void *workspace, hipStream_t st) {
  BA_TRY(upload(pl, workspace, st));
  Meta mt = make_meta(pl, workspace);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if (pl->dtype == BA_BF16) {
    // The branch keys are the last key tiles of the main kernel's online
    // softmax: one pass gives every row's final output (no partials, no merge).
    // Its workgroups take their units from per-kv-head counters.
    mt.queue_units = reinterpret_cast<int *>(ws + pl->off_queue);
    bf16 *vt = reinterpret_cast<bf16 *>(ws + pl->off_vt);
    bf16 *vbt = reinterpret_cast<bf16 *>(ws + pl->off_vbt);
    BA_TRY(timed(K_VT_TRANSPOSE, st, "V transpose",
                 [&] { return launch_vt_transpose_bf16(mt, (const bf16 *)v, vt, st); }));
    BA_TRY(timed(K_VBT_TRANSPOSE, st, "branch V transpose",
                 [&] { return launch_vbt_transpose_bf16(mt, (const bf16 *)vb, vbt, st); }));
    return timed(K_MAIN_FWD, st, "forward (main prefix and branch keys)", [&] {
      hipError_t e = launch_fill_f32(reinterpret_cast<float *>(mt.queue_units), queue_words(pl), 0.0f, st);
      if (e != hipSuccess) return e;
      return launch_main_fwd_fused_bf16(mt, (const bf16 *)q, (const bf16 *)qb, (const bf16 *)k, vt, (const bf16 *)kb,
                                        vbt, (bf16 *)o, lse, (bf16 *)ob, lseb, st);
    });
  }
  float *o_pre = reinterpret_cast<float *>(ws + pl->off_o_pre);
  float *lse_pre = reinterpret_cast<float *>(ws + pl->off_lse_pre);
  BA_TRY(run_main_fwd(pl, mt, q, qb, k, v, o, lse, o_pre, lse_pre, workspace, st));
  float *o_loc = reinterpret_cast<float *>(ws + pl->off_o_loc);
  float *lse_loc = reinterpret_cast<float *>(ws + pl->off_lse_loc);
  BA_TRY(timed(K_BRANCH_LOCAL_FWD, st, "branch-local forward",
               [&] { return launch_branch_local_fwd(mt, pl->dtype, qb, kb, vb, o_loc, lse_loc, st); }));
  BA_TRY(timed(K_LSE_MERGE, st, "lse_merge", [&] {
    return launch_lse_merge(pl->Rb, pl->hq, pl->d, o_pre, lse_pre, o_loc, lse_loc, ob, pl->dtype, lseb, st);
  }));
  return BA_OK;
}

ba_status_t check_fwd_args(const ba_plan *pl, const void *q, const void *k, const void *v, const void *qb,
                           const void *kb, const void *vb, const void *o, const float *lse, const void *ob,
                           const float *lseb) {
  BA_TRY(check_plan(pl));
  const int64_t hd = (int64_t)pl->hq * pl->d, kd = (int64_t)pl->hkv * pl->d;
  BA_TRY(check_ptr(q, pl->Nq * hd, "q"));
  BA_TRY(check_ptr(k, pl->N * kd, "k"));
  BA_TRY(check_ptr(v, pl->N * kd, "v"));
  BA_TRY(check_ptr(qb, pl->Rb * hd, "qb"));
  BA_TRY(check_ptr(kb, pl->Rb * kd, "kb"));
  BA_TRY(check_ptr(vb, pl->Rb * kd, "vb"));
  BA_TRY(check_ptr(o, pl->Nq * hd, "o"));
  BA_TRY(check_ptr(lse, pl->Nq * pl->hq, "lse"));
  BA_TRY(check_ptr(ob, pl->Rb * hd, "ob"));
  BA_TRY(check_ptr(lseb, pl->Rb * pl->hq, "lseb"));
  return BA_OK;
}

}  // namespace

extern "C" {

ba_status_t ba_main_fwd(const ba_plan_t *pl, const void *q, const void *qb, const void *k, const void *v, void *o,
                        float *lse, float *o_pre, float *lse_pre, void *workspace, size_t ws_bytes, void *stream) {
  BA_TRY(check_plan(pl));
  const int64_t hd = (int64_t)pl->hq * pl->d, kd = (int64_t)pl->hkv * pl->d;
  BA_TRY(check_ptr(q, pl->Nq * hd, "q"));
  BA_TRY(check_ptr(qb, pl->Rb * hd, "qb"));
  BA_TRY(check_ptr(k, pl->N * kd, "k"));
  BA_TRY(check_ptr(v, pl->N * kd, "v"));
  BA_TRY(check_ptr(o, pl->Nq * hd, "o"));
  BA_TRY(check_ptr(lse, pl->Nq * pl->hq, "lse"));
  BA_TRY(check_ptr(o_pre, pl->Rb * hd, "o_pre"));
  BA_TRY(check_ptr(lse_pre, pl->Rb * pl->hq, "lse_pre"));
  BA_TRY(check_ws(pl, workspace, ws_bytes, 2));
  hipStream_t st = static_cast<hipStream_t>(stream);
  BA_TRY(upload(pl, workspace, st));
  return run_main_fwd(pl, make_meta(pl, workspace), q, qb, k, v, o, lse, o_pre, lse_pre, workspace, st);
}

ba_status_t ba_branch_local_fwd(const ba_plan_t *pl, const void *qb, const void *kb, const void *vb, float *o_loc,
                                float *lse_loc, void *workspace, size_t ws_bytes, void *stream) {
  BA_TRY(check_plan(pl));
  const int64_t hd = (int64_t)pl->hq * pl->d, kd = (int64_t)pl->hkv * pl->d;
  BA_TRY(check_ptr(qb, pl->Rb * hd, "qb"));
  BA_TRY(check_ptr(kb, pl->Rb * kd, "kb"));
  BA_TRY(check_ptr(vb, pl->Rb * kd, "vb"));
  BA_TRY(check_ptr(o_loc, pl->Rb * hd, "o_loc"));
  BA_TRY(check_ptr(lse_loc, pl->Rb * pl->hq, "lse_loc"));
  BA_TRY(check_ws(pl, workspace, ws_bytes, 2));
  hipStream_t st = static_cast<hipStream_t>(stream);
  BA_TRY(upload(pl, workspace, st));
  const Meta mt = make_meta(pl, workspace);
  BA_TRY(timed(K_BRANCH_LOCAL_FWD, st, "branch-local forward", [&] {
    if (pl->dtype == BA_BF16)
      return launch_branch_fwd_bf16(mt, (const bf16 *)qb, (const bf16 *)kb, (const bf16 *)vb, o_loc, lse_loc, st);
    return launch_branch_local_fwd(mt, pl->dtype, qb, kb, vb, o_loc, lse_loc, st);
  }));
  return BA_OK;
}

ba_status_t ba_ring_step_fwd(const ba_plan_t *pl, const void *q, const void *qb, const void *k_win,
                             const void *v_win, int64_t win_lo, int64_t win_hi, float *o_run, float *lse_run,
                             void *workspace, size_t ws_bytes, void *stream) {
  BA_TRY(check_plan(pl));
  if (pl->dtype != BA_BF16) return set_error(BA_EUNSUPPORTED, "ba_ring_step_fwd: bf16 only");
  if (win_lo < 0 || win_lo > win_hi || win_hi > pl->N)
    return set_error(BA_EINVAL, "ba_ring_step_fwd: need 0 <= win_lo <= win_hi <= N");
  const int64_t hd = (int64_t)pl->hq * pl->d, kd = (int64_t)pl->hkv * pl->d, R = pl->Nq + pl->Rb;
  BA_TRY(check_ptr(q, pl->Nq * hd, "q"));
  BA_TRY(check_ptr(qb, pl->Rb * hd, "qb"));
  BA_TRY(check_ptr(k_win, (win_hi - win_lo) * kd, "k_win"));
  BA_TRY(check_ptr(v_win, (win_hi - win_lo) * kd, "v_win"));
  BA_TRY(check_ptr(o_run, R * hd, "o_run"));
  BA_TRY(check_ptr(lse_run, R * pl->hq, "lse_run"));
  BA_TRY(check_ws(pl, workspace, ws_bytes, 2));
  if (win_lo == win_hi) return BA_OK;  // an empty window is the identity
  hipStream_t st = static_cast<hipStream_t>(stream);
  BA_TRY(upload(pl, workspace, st));
  const Meta mt = make_meta(pl, workspace);
  bf16 *vt = reinterpret_cast<bf16 *>(static_cast<uint8_t *>(workspace) + pl->off_vt);
  BA_TRY(timed(K_VT_TRANSPOSE, st, "V transpose (window)", [&] {
    return launch_vt_transpose_bf16(mt, (const bf16 *)v_win, vt, st, (int)win_lo, (int)win_hi);
  }));
  return timed(K_RING_FWD, st, "ring step forward", [&] {
    return launch_ring_fwd_bf16(mt, (const bf16 *)q, (const bf16 *)qb, (const bf16 *)k_win, vt, (int)win_lo,
                                (int)win_hi, o_run, lse_run, st);
  });
}

ba_status_t lse_merge(int64_t rows, int32_t heads, int32_t head_dim, const float *o_a, const float *lse_a,
                      const float *o_b, const float *lse_b, void *o_out, ba_dtype_t out_dtype, float *lse_out,
                      void *stream) {
  if (rows < 0 || heads < 1 || head_dim < 4 || head_dim % 4 != 0 || 64 % (head_dim / 4) != 0)
    return set_error(BA_EINVAL, "lse_merge: need rows >= 0, heads >= 1, head_dim/4 dividing 64");
  if (out_dtype != BA_F32 && out_dtype != BA_BF16) return set_error(BA_EINVAL, "lse_merge: bad out_dtype");
  const int64_t n = rows * heads * head_dim, nl = rows * heads;
  BA_TRY(check_ptr(o_a, n, "o_a"));
  BA_TRY(check_ptr(o_b, n, "o_b"));
  BA_TRY(check_ptr(o_out, n, "o_out"));
  if (nl && (!lse_a || !lse_b || !lse_out)) return set_error(BA_EINVAL, "lse_merge: NULL lse pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  BA_TRY(timed(K_LSE_MERGE, st, "lse_merge", [&] {
    return launch_lse_merge(rows, heads, head_dim, o_a, lse_a, o_b, lse_b, o_out, out_dtype, lse_out, st);
  }));
  return BA_OK;
}

ba_status_t branch_attn_fwd(const ba_plan_t *pl, const void *q, const void *k, const void *v, const void *qb,
                            const void *kb, const void *vb, void *o, float *lse, void *ob, float *lseb,
                            void *workspace, size_t ws_bytes, void *stream) {
  BA_TRY(check_fwd_args(pl, q, k, v, qb, kb, vb, o, lse, ob, lseb));
  BA_TRY(check_ws(pl, workspace, ws_bytes, 0));
  return fwd_body(pl, q, k, v, qb, kb, vb, o, lse, ob, lseb, workspace, static_cast<hipStream_t>(stream));
}

size_t ba_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

ba_status_t branch_attn_fwd_noalloc(const ba_plan_t *pl, const void *q, const void *k, const void *v, const void *qb,
                                    const void *kb, const void *vb, void *o, float *lse, void *ob, float *lseb,
                                    void *stream) {
  BA_TRY(check_fwd_args(pl, q, k, v, qb, kb, vb, o, lse, ob, lseb));
  const size_t need = ba_workspace_bytes(pl, 0);
  if (need > kScratchBytes)
    return set_error(BA_EWORKSPACE, "branch_attn_fwd_noalloc: the problem needs " + std::to_string(need) +
                                        " bytes of scratch, more than its fixed " + std::to_string(kScratchBytes) +
                                        " bytes; use branch_attn_fwd with a workspace");
  void *ws = nullptr;
  BA_TRY(scratch_of_current_device(&ws));
  return fwd_body(pl, q, k, v, qb, kb, vb, o, lse, ob, lseb, ws, static_cast<hipStream_t>(stream));
}

ba_status_t branch_attn_bwd(const ba_plan_t *pl, const void *q, const void *k, const void *v, const void *qb,
                            const void *kb, const void *vb, const void *o, const float *lse, const void *ob,
                            const float *lseb, const void *d_o, const void *d_ob, void *dq, void *dk, void *dv,
                            void *dqb, void *dkb, void *dvb, void *workspace, size_t ws_bytes, void *stream) {
  BA_TRY(check_plan(pl));
  const int64_t hd = (int64_t)pl->hq * pl->d, kd = (int64_t)pl->hkv * pl->d;
  BA_TRY(check_ptr(q, pl->Nq * hd, "q"));
  BA_TRY(check_ptr(k, pl->N * kd, "k"));
  BA_TRY(check_ptr(v, pl->N * kd, "v"));
  BA_TRY(check_ptr(qb, pl->Rb * hd, "qb"));
  BA_TRY(check_ptr(kb, pl->Rb * kd, "kb"));
  BA_TRY(check_ptr(vb, pl->Rb * kd, "vb"));
  BA_TRY(check_ptr(o, pl->Nq * hd, "o"));
  BA_TRY(check_ptr(lse, pl->Nq * pl->hq, "lse"));
  BA_TRY(check_ptr(ob, pl->Rb * hd, "ob"));
  BA_TRY(check_ptr(lseb, pl->Rb * pl->hq, "lseb"));
  BA_TRY(check_ptr(d_o, pl->Nq * hd, "d_o"));
  BA_TRY(check_ptr(d_ob, pl->Rb * hd, "d_ob"));
  BA_TRY(check_ptr(dq, pl->Nq * hd, "dq"));
  BA_TRY(check_ptr(dk, pl->N * kd, "dk"));
  BA_TRY(check_ptr(dv, pl->N * kd, "dv"));
  BA_TRY(check_ptr(dqb, pl->Rb * hd, "dqb"));
  BA_TRY(check_ptr(dkb, pl->Rb * kd, "dkb"));
  BA_TRY(check_ptr(dvb, pl->Rb * kd, "dvb"));
  BA_TRY(check_ws(pl, workspace, ws_bytes, 1));
  hipStream_t st = static_cast<hipStream_t>(stream);
  BA_TRY(upload(pl, workspace, st));
  Meta mt = make_meta(pl, workspace);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  float *delta = reinterpret_cast<float *>(ws + pl->off_delta);
  float *dq_acc = reinterpret_cast<float *>(ws + pl->off_dq_acc);
  if (pl->dtype == BA_BF16) {
    bf16 *qt = reinterpret_cast<bf16 *>(ws + pl->off_qt);
    bf16 *dot = reinterpret_cast<bf16 *>(ws + pl->off_dot);
    float *lt = reinterpret_cast<float *>(ws + pl->off_lt);
    float *dtt = reinterpret_cast<float *>(ws + pl->off_dt);
    int *et = reinterpret_cast<int *>(ws + pl->off_et);
    // dQ of every row, over its main prefix and then its branch keys, in bf16;
    // the same kernel takes D = rowsum(dO * O) and stages the query tiles the
    // dK/dV kernel streams (the backward preprocess).
    const BwdStage sg{qt, dot, lt, dtt, et, delta};
    // Both kernels take their work items from per-kv-head counters.
    mt.queue_units = reinterpret_cast<int *>(ws + pl->off_queue);
    mt.queue_ktiles = mt.queue_units + pl->hkv;
    BA_TRY(timed(K_MAIN_BWD_DQ, st, "backward (dq)", [&] {
      hipError_t e = launch_fill_f32(reinterpret_cast<float *>(mt.queue_units), queue_words(pl), 0.0f, st);
      if (e != hipSuccess) return e;
      return launch_main_bwd_dq_bf16(mt, (const bf16 *)q, (const bf16 *)qb, (const bf16 *)k, (const bf16 *)v,
                                     (const bf16 *)d_o, (const bf16 *)d_ob, lse, lseb, (const bf16 *)o,
                                     (const bf16 *)ob, (const bf16 *)kb, (const bf16 *)vb, (bf16 *)dq, (bf16 *)dqb,
                                     sg, st);
    }));
    // Split key tiles: every dK/dV workgroup adds into zeroed float32
    // accumulators, converted to bf16 afterwards (a fill kernel, not a memset).
    float *dkv_acc = pl->dkv_split ? reinterpret_cast<float *>(ws + pl->off_dkv_acc) : nullptr;
    const int64_t nkv = pl->N * kd;
    BA_TRY(timed(K_MAIN_BWD_DKDV, st, "main-sequence backward (dk, dv)", [&] {
      if (dkv_acc) {
        hipError_t e = launch_fill_f32(dkv_acc, 2 * nkv, 0.0f, st);
        if (e != hipSuccess) return e;
      }
      hipError_t e = launch_main_bwd_dkdv_bf16(mt, (const bf16 *)k, (const bf16 *)v, qt, dot, lt, dtt, et,
                                               (bf16 *)dk, (bf16 *)dv, dkv_acc, st);
      if (e != hipSuccess || !dkv_acc) return e;
      e = launch_convert_rows(dkv_acc, nkv, dk, pl->dtype, st);
      if (e != hipSuccess) return e;
      return launch_convert_rows(dkv_acc + nkv, nkv, dv, pl->dtype, st);
    }));
  } else {
    BA_TRY(timed(K_BWD_PREPROCESS, st, "backward preprocess",
                 [&] { return launch_bwd_preprocess(mt, pl->dtype, o, d_o, ob, d_ob, delta, st); }));
    BA_TRY(timed(K_MAIN_BWD_DKDV, st, "main-sequence backward", [&] {
      return launch_main_bwd_f32(mt, (const float *)q, (const float *)qb, (const float *)k, (const float *)v,
                                 (const float *)d_o, (const float *)d_ob, lse, lseb, delta, dq_acc, (float *)dk,
                                 (float *)dv, st);
    }));
  }
  if (pl->dtype == BA_BF16)  // dK, dV of the branch keys
    return timed(K_BRANCH_LOCAL_BWD, st, "branch-local backward (dkb, dvb)", [&] {
      return launch_branch_bwd_bf16(mt, (const bf16 *)qb, (const bf16 *)kb, (const bf16 *)vb, (const bf16 *)d_ob, lseb,
                                    delta, (bf16 *)dkb, (bf16 *)dvb, st);
    });
  BA_TRY(timed(K_BRANCH_LOCAL_BWD, st, "branch-local backward", [&] {
    return launch_branch_local_bwd(mt, pl->dtype, qb, kb, vb, d_ob, lseb, delta, dq_acc, dkb, dvb, st);
  }));
  BA_TRY(timed(K_DQ_CONVERT, st, "dq convert", [&] {
    hipError_t e = launch_convert_rows(dq_acc, pl->Nq * hd, dq, pl->dtype, st);
    if (e != hipSuccess) return e;
    return launch_convert_rows(dq_acc + pl->Nq * hd, pl->Rb * hd, dqb, pl->dtype, st);
  }));
  return BA_OK;
}

ba_status_t ba_timing_enable(int on) {
  timing().on.store(on != 0);
  return BA_OK;
}

ba_status_t ba_timing_reset(void) {
  TimingState &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  drain(t);
  for (int i = 0; i < K_COUNT; ++i) {
    t.total_ms[i] = 0.0;
    t.launches[i] = 0;
  }
  return BA_OK;
}

int ba_timing_kernels(void) { return K_COUNT; }

const char *ba_timing_kernel_name(int id) { return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : nullptr; }

ba_status_t ba_timing_read(int id, double *total_ms, int64_t *launches) {
  if (id < 0 || id >= K_COUNT || !total_ms || !launches) return set_error(BA_EINVAL, "ba_timing_read: bad argument");
  TimingState &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  drain(t);
  *total_ms = t.total_ms[id];
  *launches = t.launches[id];
  return BA_OK;
}

}  // extern "C"
