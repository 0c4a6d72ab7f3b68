// Host-side paths of the C ABI, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU: shape validation
// and workspace layout, tree-spec validation (valid and malformed rank
// tables), the calibrated sparse-tree builder, and the argument checks of
// the step, the decoding loop and the static-workspace step. Every device
// pointer is a fake aligned address and every call is made to fail its
// validation before a launch, so nothing reaches the GPU. Exits non-zero
// on the first unexpected return code.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <set>
#include <vector>

#include "medusa.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int rc) {
  if (!ok) {
    fprintf(stderr, "unexpected: %s (rc %d, %s)\n", what, rc, medusa_last_error());
    ++failures;
  }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t{1} << 20) + off); }

medusa_shape shape7b() {
  medusa_shape s{};
  s.B = 1; s.d = 4096; s.V = 32000; s.K = 5; s.H = 32; s.Dh = 128; s.Lmax = 2112;
  s.N = 45; s.P = 12; s.s_max = 3; s.dtype = MEDUSA_BF16;
  return s;
}

// A random prefix-closed tree in canonical order (depth, then lexicographic)
// as a [N][K] rank table, -1 padded.
std::vector<int32_t> random_tree(std::mt19937& rng, int K, int S, int budget, int* N, int* P) {
  std::set<std::vector<int>> nodes;
  std::vector<std::vector<int>> frontier = {{}};
  while ((int)nodes.size() < budget && !frontier.empty()) {
    const size_t i = rng() % frontier.size();
    std::vector<int> p = frontier[i];
    const int r = (int)(rng() % S);
    std::vector<int> c = p;
    c.push_back(r);
    if ((int)c.size() <= K && !nodes.count(c)) {
      nodes.insert(c);
      frontier.push_back(c);
    }
    if (rng() % 4 == 0) frontier.erase(frontier.begin() + i);
  }
  std::vector<std::vector<int>> v(nodes.begin(), nodes.end());
  std::stable_sort(v.begin(), v.end(), [](const std::vector<int>& a, const std::vector<int>& b) {
    return a.size() < b.size();
  });
  std::set<std::vector<int>> parents;
  for (auto& t : v) parents.insert(std::vector<int>(t.begin(), t.end() - 1));
  *P = 0;
  for (auto& t : v) *P += !parents.count(t);
  if (v.empty()) *P = 1;
  *N = (int)v.size();
  std::vector<int32_t> ranks((size_t)*N * K, -1);
  for (int n = 0; n < *N; ++n)
    for (size_t j = 0; j < v[n].size(); ++j) ranks[(size_t)n * K + j] = v[n][j];
  return ranks;
}

int call_tree(const medusa_shape& s, const int32_t* ranks) {
  return medusa_build_tree(&s, ranks, MEDUSA_DRAFT_TOPK, (int32_t*)fake(), (int32_t*)fake(),
                           nullptr, nullptr, nullptr, (int32_t*)fake(), (int32_t*)fake(),
                           (uint8_t*)fake(), (int32_t*)fake(), (int32_t*)fake(),
                           (int32_t*)fake(), (int32_t*)fake(), nullptr);
}

medusa_step_args step_args(const int32_t* ranks, bool exact) {
  medusa_step_args a;
  memset(&a, 0, sizeof(a));
  void** p = reinterpret_cast<void**>(&a);
  // every pointer member a fake aligned address, then the non-pointers
  for (size_t i = 0; i < sizeof(a) / sizeof(void*); ++i) p[i] = fake();
  a.b1_or_null = nullptr;
  a.kv_len_out_or_null = nullptr;
  a.tree_ranks_host = ranks;
  a.draft_mode = exact ? MEDUSA_DRAFT_SAMPLE : MEDUSA_DRAFT_TOPK;
  a.mode = exact ? MEDUSA_EXACT : MEDUSA_TYPICAL;
  a.rope_theta = 10000.f;
  a.temperature = 1.f;
  a.eps = 0.09f;
  a.delta = 0.3f;
  return a;
}

}  // namespace

int main() {
  std::mt19937 rng(20261202);
  // ---- shapes and workspace layout ----
  for (int it = 0; it < 4000; ++it) {
    medusa_shape s{};
    s.B = (int)(rng() % 70) - 2;
    s.Dh = (rng() % 3 == 0) ? 64 : ((rng() % 2) ? 128 : (int)(rng() % 200));
    s.H = (int)(rng() % 48) + (rng() % 10 == 0 ? -1 : 1);
    s.d = (rng() % 8 == 0) ? (int)(rng() % 9000) : s.H * s.Dh;
    s.V = (int)(rng() % 70000) - 5;
    s.K = (int)(rng() % 11) - 1;
    s.Lmax = (int)(rng() % 9000) - 5;
    s.N = (int)(rng() % 300) - 5;
    s.P = (int)(rng() % 300) - 5;
    s.s_max = (int)(rng() % 20) - 2;
    s.dtype = (rng() % 10 == 0) ? 7 : (int)(rng() % 2);
    const size_t n = medusa_workspace_bytes(&s);
    expect(n == 0 || n % 256 == 0, "workspace size alignment", 0);
  }
  // ---- tree specs: random valid trees reach the path-count check ----
  for (int it = 0; it < 600; ++it) {
    const int K = 1 + (int)(rng() % MEDUSA_MAX_K), S = 1 + (int)(rng() % MEDUSA_MAX_S);
    int N = 0, P = 0;
    std::vector<int32_t> ranks = random_tree(rng, K, S, 1 + (int)(rng() % 255), &N, &P);
    medusa_shape s = shape7b();
    s.K = K; s.s_max = S; s.N = N; s.P = P + 1;   // a path count that cannot match
    const int rc = call_tree(s, N ? ranks.data() : nullptr);
    expect(rc == MEDUSA_ERR_ARG && strstr(medusa_last_error(), "paths"), "valid tree, P mismatch", rc);
    // the same table, corrupted: a rank beyond the pool, a gap, a swap
    if (N >= 2) {
      std::vector<int32_t> bad = ranks;
      const int n = (int)(rng() % N);
      switch (rng() % 3) {
        case 0: bad[(size_t)n * K] = S; break;
        case 1: if (K > 1) { bad[(size_t)n * K] = -1; bad[(size_t)n * K + 1] = 0; } break;
        default: std::swap(bad[0], bad[(size_t)(N - 1) * K]); break;
      }
      // (a change that keeps the table valid still fails the path count)
      const int rc2 = call_tree(s, bad.data());
      expect(rc2 == MEDUSA_ERR_ARG, "corrupted tree", rc2);
    }
  }
  // ---- calibrated sparse tree ----
  for (int it = 0; it < 300; ++it) {
    const int K = 1 + (int)(rng() % MEDUSA_MAX_K), S = 1 + (int)(rng() % MEDUSA_MAX_S);
    const int budget = (int)(rng() % MEDUSA_MAX_T);
    std::vector<double> a((size_t)K * S);
    std::uniform_real_distribution<double> u(0.0, 1.0);
    for (auto& x : a) x = (rng() % 7 == 0) ? 0.0 : u(rng);
    std::vector<int32_t> ranks((size_t)std::max(budget, 1) * K);
    std::vector<double> w(std::max(budget, 1));
    std::vector<int32_t> order(std::max(budget, 1));
    int n = -1;
    const int rc = medusa_sparse_tree(K, S, a.data(), budget, ranks.data(), w.data(), order.data(), &n);
    expect(rc == MEDUSA_OK && n >= 0 && n <= budget, "sparse tree", rc);
    for (int i = 1; i < n; ++i) expect(w[i] >= 0.0, "sparse tree weight", rc);
  }
  {
    double a[2] = {0.5, -1.0};
    int32_t r[4];
    int n = 0;
    const int rc = medusa_sparse_tree(1, 2, a, 2, r, nullptr, nullptr, &n);
    expect(rc == MEDUSA_ERR_ARG, "negative table entry", rc);
  }
  // ---- step, loop and static-workspace argument checks ----
  {
    int N = 0, P = 0;
    std::mt19937 r2(7);
    std::vector<int32_t> ranks = random_tree(r2, 5, 3, 45, &N, &P);
    medusa_shape s = shape7b();
    s.N = N; s.P = P;
    const size_t ws = medusa_workspace_bytes(&s);
    expect(ws > 0, "workspace of a valid shape", 0);
    for (int exact = 0; exact < 2; ++exact) {
      medusa_step_args a = step_args(ranks.data(), exact);
      a.E = nullptr;
      int rc = medusa_step(&s, &a, fake(), ws, nullptr);
      expect(rc == MEDUSA_ERR_ARG, "step with a null embedding", rc);
      a = step_args(ranks.data(), exact);
      a.u_resample_or_null = exact ? static_cast<float*>(fake(4)) : nullptr;
      a.h_next = exact ? a.h_next : static_cast<float*>(fake(8));
      rc = medusa_generate(&s, &a, 7, (int32_t*)fake(), (int32_t*)fake(), fake(), ws, nullptr);
      expect(rc == MEDUSA_ERR_ARG, "loop with a misaligned buffer", rc);
      a = step_args(ranks.data(), exact);
      rc = medusa_step(&s, &a, fake(), ws - 256, nullptr);
      expect(rc == MEDUSA_ERR_WORKSPACE, "step with a short workspace", rc);
    }
    medusa_shape big = s;   // 8 sequences over an 8192-row cache: more than the array
    big.B = 8;
    big.Lmax = 8192;
    medusa_step_args a = step_args(ranks.data(), false);
    const int rc = medusa_step_static(&big, &a, nullptr);
    expect(rc == MEDUSA_ERR_WORKSPACE, "static step beyond its workspace", rc);
  }
  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("host paths ok\n");
  return 0;
}
