// Host-only driver for the planner (plan.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_plan_sanitizers.py. It builds plans
// for seeded random problems (sequence, query, anchor and branch layouts, head
// maps, both dtypes and head sizes) and for malformed ones, and checks the
// status of each call; any memory or UB error aborts under the sanitizers.
// Usage: plan_sanitize <seed> <count>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "branch_attn.h"

namespace {

struct Rng {  // xorshift64*
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 0x2545F4914F6CDD1Dull;
  }
  int range(int lo, int hi) { return lo + (int)(next() % (uint64_t)(hi - lo + 1)); }  // inclusive
  bool coin(int pct) { return range(0, 99) < pct; }
};

// Owns the arrays a ba_problem_t points at.
struct Case {
  std::vector<int32_t> cu, qpos, anchors, cub, heads;
  std::vector<uint8_t> mode;
  ba_problem_t p{};
  void wire() {
    p.cu_seqlens = cu.data();
    p.q_pos = qpos.empty() ? nullptr : qpos.data();
    p.anchors = anchors.empty() ? nullptr : anchors.data();
    p.cu_branch = cub.empty() ? nullptr : cub.data();
    p.kv_head_of = heads.empty() ? nullptr : heads.data();
    p.mode = mode.empty() ? nullptr : mode.data();
  }
};

Case random_case(Rng &r) {
  Case c;
  const int hkv_opts[] = {1, 2, 4, 8};
  const int hkv = hkv_opts[r.range(0, 3)];
  const int G = r.range(1, 8);
  c.p.dtype = r.coin(50) ? BA_BF16 : BA_F32;
  c.p.num_kv_heads = hkv;
  c.p.num_q_heads = hkv * G;
  c.p.head_dim = r.coin(50) ? 64 : 128;
  c.p.softmax_scale = r.coin(70) ? 0.0f : 0.3f;
  if (r.coin(30)) {  // strided map: every kv head serves G q heads
    c.heads.resize(c.p.num_q_heads);
    for (int h = 0; h < c.p.num_q_heads; ++h) c.heads[h] = h % hkv;
  }
  const int S = r.range(1, 6);
  const int maxlen = r.coin(20) ? 6000 : 700;
  c.cu.push_back(0);
  for (int s = 0; s < S; ++s) c.cu.push_back(c.cu.back() + (r.coin(10) ? 0 : r.range(1, maxlen)));
  const int N = c.cu.back();
  c.p.num_seqs = S;
  if (N > 0 && r.coin(30)) {  // a strictly increasing subset of positions as main rows
    for (int i = 0; i < N; ++i)
      if (r.coin(40)) c.qpos.push_back(i);
    if (c.qpos.empty()) c.qpos.push_back(N - 1);
    c.p.num_q = (int32_t)c.qpos.size();
  }
  if (N > 0 && r.coin(85)) {
    const int every = r.range(1, 40);
    for (int i = r.range(0, every - 1); i < N; i += every) c.anchors.push_back(i);
  }
  const int A = (int)c.anchors.size();
  c.p.num_anchors = A;
  if (r.coin(40)) {
    c.cub.push_back(0);
    for (int a = 0; a < A; ++a) c.cub.push_back(c.cub.back() + r.range(0, 32));
  } else {
    c.p.branch_len = r.range(1, 32);
  }
  if (r.coin(40)) {
    c.mode.resize(A);
    for (int a = 0; a < A; ++a) c.mode[a] = (uint8_t)(r.coin(50) ? BA_TTT : BA_BLOCK);
  } else {
    c.p.uniform_mode = r.coin(50) ? BA_TTT : BA_BLOCK;
  }
  c.wire();
  return c;
}

int failures = 0;

void expect(bool ok, const char *what, int idx) {
  if (!ok) {
    std::fprintf(stderr, "case %d: %s (%s)\n", idx, what, ba_last_error());
    ++failures;
  }
}

// Build a plan, query everything it exposes, release it. Returns the status.
ba_status_t exercise(const ba_problem_t *p) {
  ba_plan_t *plan = nullptr;
  const ba_status_t st = ba_plan_create(p, &plan);
  if (st != BA_OK) return st;
  volatile size_t sink = 0;
  for (int pass = -1; pass <= 3; ++pass) sink = sink + ba_workspace_bytes(plan, pass);
  int64_t sizes[5], pairs[3];
  if (ba_plan_sizes(plan, sizes) != BA_OK || ba_plan_pairs(plan, pairs) != BA_OK) {
    ba_plan_destroy(plan);
    return BA_EINVAL;
  }
  for (int i = 0; i < 3; ++i)
    if (pairs[i] < 0) {
      ba_plan_destroy(plan);
      return BA_EINVAL;
    }
  ba_plan_destroy(plan);
  return BA_OK;
}

}  // namespace

int main(int argc, char **argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int count = argc > 2 ? std::atoi(argv[2]) : 200;
  Rng r(seed);
  int n_ok = 0, n_bad = 0;
  for (int i = 0; i < count; ++i) {
    Case c = random_case(r);
    const bool valid = c.cu.back() > 0;  // an empty batch may be refused, never mishandled
    const ba_status_t st = exercise(&c.p);
    if (valid) expect(st == BA_OK, "valid problem refused", i);
    n_ok += st == BA_OK;

    // One malformation at a time; each must be refused with the right status.
    const int N = c.cu.back();
    const int A = c.p.num_anchors;
    {
      Case b = c;
      b.cu[0] = 1;
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "cu_seqlens[0] != 0 accepted", i);
    }
    if (c.p.num_seqs >= 2 && c.cu[1] > 0) {
      Case b = c;
      b.cu[1] = b.cu[2] + 1;  // non-monotone offsets
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "decreasing cu_seqlens accepted", i);
    }
    if (A >= 1) {
      Case b = c;
      b.anchors[A - 1] = N;  // out of range
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "anchor past the end accepted", i);
    }
    if (A >= 2) {
      Case b = c;
      b.anchors[1] = b.anchors[0];  // not strictly increasing
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "repeated anchor accepted", i);
    }
    if (A >= 1) {
      Case b = c;
      if (b.cub.empty()) {
        b.p.branch_len = 33;
      } else {
        for (int a = 0; a <= A; ++a) b.cub[a] = a == 0 ? 0 : b.cub[a - 1] + (a == 1 ? 33 : 1);
      }
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "branch of 33 rows accepted", i);
    }
    if (A >= 1 && !c.mode.empty()) {
      Case b = c;
      b.mode[0] = 7;
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "bad mode accepted", i);
    }
    if (c.qpos.size() >= 2) {
      Case b = c;
      b.qpos[1] = b.qpos[0];
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "repeated query position accepted", i);
    }
    {
      Case b = c;
      b.p.num_q_heads = b.p.num_kv_heads * 3 + (b.p.num_kv_heads > 1 ? 1 : 0);
      b.heads.clear();
      b.wire();
      if (b.p.num_q_heads % b.p.num_kv_heads != 0)
        expect(exercise(&b.p) == BA_EINVAL, "Hq % Hkv != 0 accepted", i);
    }
    if (c.p.num_kv_heads >= 2) {
      Case b = c;
      b.heads.assign(b.p.num_q_heads, 0);  // every q head on kv head 0
      b.wire();
      expect(exercise(&b.p) == BA_EINVAL, "unbalanced kv_head_of accepted", i);
    }
    {
      Case b = c;
      b.p.head_dim = 96;
      b.wire();
      expect(exercise(&b.p) == BA_EUNSUPPORTED, "head_dim 96 not reported unsupported", i);
    }
    ++n_bad;
  }
  {  // a full-size plan: a 13-chunk sequence of 16384-token chunks whose chunks 3
     // and 12 hold the main rows, each an anchor of a depth-7 branch (GQA 32/8, d 128)
    Case c;
    c.p.dtype = BA_BF16;
    c.p.num_q_heads = 32;
    c.p.num_kv_heads = 8;
    c.p.head_dim = 128;
    c.p.num_seqs = 1;
    c.cu = {0, 13 * 16384};
    for (int chunk : {3, 12})
      for (int i = 0; i < 16384; ++i) c.qpos.push_back(chunk * 16384 + i);
    c.p.num_q = (int32_t)c.qpos.size();
    c.anchors = c.qpos;
    c.p.num_anchors = (int32_t)c.anchors.size();
    c.p.branch_len = 7;
    c.p.uniform_mode = BA_TTT;
    c.wire();
    expect(exercise(&c.p) == BA_OK, "full-size plan refused", -2);
  }
  ba_plan_t *plan = nullptr;
  expect(ba_plan_create(nullptr, &plan) == BA_EINVAL, "NULL problem accepted", -1);
  ba_plan_destroy(nullptr);
  std::printf("plans: %d built, %d malformed sets refused, %d failures\n", n_ok, n_bad, failures);
  return failures == 0 ? 0 : 1;
}
