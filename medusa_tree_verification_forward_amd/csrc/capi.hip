// C ABI of the Medusa verify-step library: host-side validation, workspace
// layout and dispatch to the gfx950 kernels. See include/medusa.h for the
// contract of every entry point.
#include "medusa.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include <math.h>

#include "kernels.h"

using namespace medusa;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return MEDUSA_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MEDUSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                         \
  do {                                                                         \
    if (!(p)) return fail(MEDUSA_ERR_ARG, "%s: null pointer", #p);             \
    if (!aligned16(p)) return fail(MEDUSA_ERR_ARG, "%s: not 16-byte aligned", #p); \
  } while (0)
#define OPTIONAL_PTR(p)                                                        \
  do {                                                                         \
    if ((p) && !aligned16(p)) return fail(MEDUSA_ERR_ARG, "%s: not 16-byte aligned", #p); \
  } while (0)

// Rows per wave of the head streams (a workgroup has 4 waves). W1: the
// fewest that let all K d rows run as one wave of resident workgroups (0:
// the launcher computes it). W2: 56 rows a wave and the workgroups per head
// that cover the V rows with them -- measured fastest for the 7B heads (715
// workgroups; 40, 48, 54, 58, 60 and 64 rows, and grids filling exactly 3 or
// 4 workgroups per compute unit, were 0.6-15 us slower).
constexpr int kW1Rows = 0;
constexpr int kW2Rows = 56;
void w2_grid(int V, int& G, int& rpw) {
  rpw = kW2Rows;
  G = (V + 4 * rpw - 1) / (4 * rpw);
}


constexpr size_t kCounterBytes = 64 * 1024;   // workspace bytes reserved at offset 0 for counters
// the block's last MEDUSA_MAX_B counters belong to the composite step's commit
constexpr size_t kCommitCounter = kCounterBytes / sizeof(int) - MEDUSA_MAX_B;

int check_shape(const medusa_shape* s) {
  if (!s) return fail(MEDUSA_ERR_ARG, "shape: null pointer");
  if (s->dtype != MEDUSA_BF16 && s->dtype != MEDUSA_F32)
    return fail(MEDUSA_ERR_ARG, "dtype %d is neither MEDUSA_BF16 nor MEDUSA_F32", s->dtype);
  if (s->B < 1 || s->d < 1 || s->V < 1 || s->K < 1 || s->H < 1 || s->Dh < 1 || s->Lmax < 1 ||
      s->N < 0 || s->P < 1 || s->s_max < 1)
    return fail(MEDUSA_ERR_ARG, "shape has a non-positive size");
  if (s->H * s->Dh != s->d) return fail(MEDUSA_ERR_ARG, "H*Dh (%d) != d (%d)", s->H * s->Dh, s->d);
  if (s->V < s->s_max) return fail(MEDUSA_ERR_ARG, "V (%d) < s_max (%d)", s->V, s->s_max);
  if (s->B > MEDUSA_MAX_B) return fail(MEDUSA_ERR_UNSUPPORTED, "B=%d > %d", s->B, MEDUSA_MAX_B);
  if (s->K > MEDUSA_MAX_K) return fail(MEDUSA_ERR_UNSUPPORTED, "K=%d > %d", s->K, MEDUSA_MAX_K);
  if (s->s_max > MEDUSA_MAX_S)
    return fail(MEDUSA_ERR_UNSUPPORTED, "s_max=%d > %d", s->s_max, MEDUSA_MAX_S);
  if (s->N + 1 > MEDUSA_MAX_T)
    return fail(MEDUSA_ERR_UNSUPPORTED, "T=%d > %d", s->N + 1, MEDUSA_MAX_T);
  if (s->P > s->N + 1) return fail(MEDUSA_ERR_ARG, "P=%d > T=%d", s->P, s->N + 1);
  if (s->d % 64 != 0) return fail(MEDUSA_ERR_UNSUPPORTED, "d=%d is not a multiple of 64", s->d);
  if (s->Dh != 64 && s->Dh != 128)
    return fail(MEDUSA_ERR_UNSUPPORTED, "Dh=%d is not 64 or 128", s->Dh);
  if ((size_t)gemm_groups_max(3 * s->d) * gemm_passes_max(s->B * (s->N + 1)) > kCommitCounter)
    return fail(MEDUSA_ERR_UNSUPPORTED, "d=%d with %d tree rows needs too many GEMM counters",
                s->d, s->B * (s->N + 1));
  return MEDUSA_OK;
}

// ---- workspace layout ----------------------------------------------------------

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  size_t counters = 0;
  // heads
  size_t z = 0, part_val = 0, part_id = 0, part_m = 0, part_s = 0, afrag = 0;
  int G = 0;
  // attention
  size_t att_o = 0, att_ml = 0;
  int NS = 0;
  // verify
  size_t q = 0, o_elem = 0, y_elem = 0, lm_part = 0, gemm_part = 0;
  // posterior (exact)
  size_t pw = 0, exact_dec = 0;
  size_t total = 0;
};

Layout layout_for(const medusa_shape* s) {
  Layout L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.counters = take(kCounterBytes);
  const size_t B = s->B, K = s->K, d = s->d, S = s->s_max;
  const int Gmax = heads_row_blocks_max(s->V, kW2Rows);
  {
    int rpw;
    w2_grid(s->V, L.G, rpw);
  }
  L.z = take(B * K * d * 4);
  L.part_val = take(B * K * Gmax * S * 4);
  L.part_id = take(B * K * Gmax * S * 4);
  L.part_m = take(B * K * Gmax * 4);
  L.part_s = take(B * K * Gmax * 4);
  L.afrag = take((K + 1) * 32 * d);
  const size_t T = s->N + 1, H = s->H, Dh = s->Dh, V = s->V;
  const size_t es = s->dtype == MEDUSA_F32 ? 4 : 2;
  L.NS = attn_splits(s->Lmax);
  L.att_o = take(B * H * L.NS * T * Dh * 4);
  L.att_ml = take(B * H * L.NS * T * 2 * 4);
  L.q = take(B * T * d * es);
  L.o_elem = take(B * T * d * es);
  L.y_elem = take((B * T + 15) / 16 * 16 * d * es);   // A-fragment order, whole m-tiles
  // LM records [M][stripes][4]
  L.lm_part = take(B * T * (size_t)lm_record_slots(s->V) * 4 * 4);
  {
    const bool f32 = s->dtype == MEDUSA_F32;
    // QKV / O-proj partials [groups][KS][M][cols] (groups * cols < N + 128)
    const int M = (int)(B * T);
    const size_t q_need = (size_t)gemm_splits(EPI_QKV, 3 * s->d, s->d, f32, M) * B * T * (3 * d + 128);
    const size_t o_need = (size_t)gemm_splits(EPI_OPROJ, s->d, s->d, f32, M) * B * T * (d + 128);
    L.gemm_part = take(std::max(q_need, o_need) * 4);
  }
  L.pw = take(B * V * 4);
  L.exact_dec = take(B * T * 2 * 4);
  L.total = off;
  return L;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_workspace(const medusa_shape* s, void* ws, size_t bytes, Layout* L) {
  *L = layout_for(s);
  if (!ws) return fail(MEDUSA_ERR_WORKSPACE, "workspace: null pointer");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace: not 256-byte aligned");
  if (bytes < L->total)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, L->total);
  return MEDUSA_OK;
}

// ---- tree spec ------------------------------------------------------------------
// Validates the host rank table and reduces it to (parent, own rank) per node.
int make_plan(const medusa_shape* s, const int32_t* ranks, TreePlan* plan, int* P_out) {
  const int N = s->N, K = s->K, T = N + 1;
  if (N > 0 && !ranks) return fail(MEDUSA_ERR_ARG, "tree_ranks: null pointer");
  std::vector<std::vector<int>> tup(N);
  for (int n = 0; n < N; ++n) {
    bool ended = false;
    for (int j = 0; j < K; ++j) {
      const int r = ranks[(size_t)n * K + j];
      if (r < 0) {
        ended = true;
        continue;
      }
      if (ended) return fail(MEDUSA_ERR_ARG, "tree_ranks row %d: rank after -1 padding", n);
      if (r >= s->s_max)
        return fail(MEDUSA_ERR_ARG, "tree_ranks row %d: rank %d >= s_max %d", n, r, s->s_max);
      tup[n].push_back(r);
    }
    if (tup[n].empty()) return fail(MEDUSA_ERR_ARG, "tree_ranks row %d: empty rank path", n);
  }
  auto canon_less = [](const std::vector<int>& a, const std::vector<int>& b) {
    if (a.size() != b.size()) return a.size() < b.size();
    return a < b;
  };
  for (int n = 1; n < N; ++n)
    if (!canon_less(tup[n - 1], tup[n]))
      return fail(MEDUSA_ERR_ARG,
                  "tree_ranks rows %d,%d: not in canonical order (depth, then lexicographic) "
                  "or duplicated",
                  n - 1, n);
  memset(plan, 0, sizeof(*plan));
  plan->T = T;
  plan->K = K;
  std::vector<char> has_child(T, 0);
  for (int n = 0; n < N; ++n) {
    int par = 0;
    if (tup[n].size() > 1) {
      std::vector<int> pre(tup[n].begin(), tup[n].end() - 1);
      // canonical order sorts parents before children: binary search
      auto it = std::lower_bound(tup.begin(), tup.begin() + n, pre, canon_less);
      if (it == tup.begin() + n || *it != pre)
        return fail(MEDUSA_ERR_ARG, "tree_ranks row %d: not prefix-closed", n);
      par = (int)(it - tup.begin()) + 1;
    }
    plan->parent[n + 1] = (uint8_t)par;
    plan->last_rank[n + 1] = (uint8_t)tup[n].back();
    plan->depth[n + 1] = (uint8_t)tup[n].size();
    has_child[par] = 1;
  }
  int P = 0;
  for (int n = 1; n < T; ++n) P += !has_child[n];
  if (T == 1) P = 1;
  *P_out = P;
  return MEDUSA_OK;
}

}  // namespace

extern "C" {

const char* medusa_last_error(void) { return g_err.c_str(); }

const char* medusa_version(void) { return "medusa-mi355x 0.1 (gfx950)"; }

size_t medusa_workspace_bytes(const medusa_shape* shape) {
  if (check_shape(shape) != MEDUSA_OK) return 0;
  return layout_for(shape).total;
}

}  // extern "C"

namespace {

// Heads, optionally writing the tree tokens and positions in the merge
// (fuse_plan != null: top-s drafting inside the composite step).
int heads_impl(const medusa_shape* shape, const float* h, const void* W1,
               const void* W1_packed_or_null, const float* b1_or_null, const void* W2,
               const void* W2_packed_or_null,
               int32_t* topk_ids, float* topk_logits,
               float* head_lse_or_null, float* head_logits_or_null, float* z_or_null,
               void* workspace, size_t workspace_bytes, void* stream, const TreePlan* fuse_plan,
               const int32_t* root_tok, const int32_t* kv_len, int32_t* tree_tokens,
               int32_t* position_ids, const float* u_draft_or_null, bool dry,
               hipEvent_t ev_w2_start = nullptr, hipEvent_t ev_w2_end = nullptr) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE_PTR(h);
  REQUIRE_PTR(W1);
  REQUIRE_PTR(W2);
  REQUIRE_PTR(topk_ids);
  REQUIRE_PTR(topk_logits);
  OPTIONAL_PTR(b1_or_null);
  OPTIONAL_PTR(W1_packed_or_null);
  OPTIONAL_PTR(W2_packed_or_null);
  OPTIONAL_PTR(head_lse_or_null);
  OPTIONAL_PTR(head_logits_or_null);
  OPTIONAL_PTR(z_or_null);
  if (fuse_plan && u_draft_or_null && !head_logits_or_null)
    return fail(MEDUSA_ERR_ARG, "sampled drafting needs head_logits");
  Layout L;
  rc = check_workspace(shape, workspace, workspace_bytes, &L);
  if (rc) return rc;
  if (dry) return MEDUSA_OK;
  HeadsArgs a{};
  a.f32 = shape->dtype == MEDUSA_F32;
  a.B = shape->B;
  a.d = shape->d;
  a.V = shape->V;
  a.K = shape->K;
  a.S = shape->s_max;
  a.h = h;
  a.W1 = W1;
  a.W1_packed = W1_packed_or_null;
  a.b1 = b1_or_null;
  a.W2 = W2;
  a.W2_packed = W2_packed_or_null;
  a.z = z_or_null ? z_or_null : at<float>(workspace, L.z);
  a.head_logits = head_logits_or_null;
  a.topk_ids = topk_ids;
  a.topk_logits = topk_logits;
  a.lse = head_lse_or_null;
  a.part_val = at<float>(workspace, L.part_val);
  a.part_id = at<int>(workspace, L.part_id);
  a.part_m = at<float>(workspace, L.part_m);
  a.part_s = at<float>(workspace, L.part_s);
  a.afrag = at<char>(workspace, L.afrag);
  a.G = L.G;
  a.w1_rows_per_wave = kW1Rows;
  {
    int G;
    w2_grid(shape->V, G, a.w2_rows_per_wave);
  }
  a.ev_before = ev_w2_start;
  a.ev_after = ev_w2_end;
  if (fuse_plan) {
    a.fuse_tree = true;
    a.plan = *fuse_plan;
    a.root_tok = root_tok;
    a.kv_len = kv_len;
    a.tree_tokens = tree_tokens;
    a.position_ids = position_ids;
    a.u_draft = u_draft_or_null;
  }
  hipError_t e = launch_heads(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "heads launch");
  return ok();
}

}  // namespace

extern "C" {

int medusa_heads_forward(const medusa_shape* shape, const float* h, const void* W1,
                         const void* W1_packed_or_null, const float* b1_or_null,
                         const void* W2, const void* W2_packed_or_null, int32_t* topk_ids,
                         float* topk_logits, float* head_lse_or_null,
                         float* head_logits_or_null, float* z_or_null, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return heads_impl(shape, h, W1, W1_packed_or_null, b1_or_null, W2, W2_packed_or_null,
                    topk_ids, topk_logits,
                    head_lse_or_null,
                    head_logits_or_null, z_or_null, workspace, workspace_bytes, stream, nullptr,
                    nullptr, nullptr, nullptr, nullptr, nullptr, false);
}

}  // extern "C"

namespace {

int tree_impl(const medusa_shape* shape, const int32_t* tree_ranks_host, int draft_mode,
              const int32_t* root_tok, const int32_t* topk_ids, const float* head_logits_or_null,
              const float* head_lse_or_null, const float* u_draft_or_null, const int32_t* kv_len,
              int32_t* tree_tokens, uint8_t* tree_mask, int32_t* position_ids, int32_t* retrieve,
              int32_t* parent, int32_t* depth, void* stream, bool dry) {
  // tree_mask, retrieve, parent and depth are optional (see medusa.h)
  int rc = check_shape(shape);
  if (rc) return rc;
  if (draft_mode != MEDUSA_DRAFT_TOPK && draft_mode != MEDUSA_DRAFT_SAMPLE)
    return fail(MEDUSA_ERR_ARG, "draft_mode %d unknown", draft_mode);
  REQUIRE_PTR(root_tok);
  REQUIRE_PTR(kv_len);
  REQUIRE_PTR(tree_tokens);
  REQUIRE_PTR(position_ids);
  OPTIONAL_PTR(tree_mask);
  OPTIONAL_PTR(retrieve);
  OPTIONAL_PTR(parent);
  OPTIONAL_PTR(depth);
  if (draft_mode == MEDUSA_DRAFT_TOPK) {
    REQUIRE_PTR(topk_ids);
  } else {
    REQUIRE_PTR(head_logits_or_null);
    REQUIRE_PTR(head_lse_or_null);
    REQUIRE_PTR(u_draft_or_null);
  }
  TreeArgs a{};
  int P = 0;
  rc = make_plan(shape, tree_ranks_host, &a.plan, &P);
  if (rc) return rc;
  if (P != shape->P)
    return fail(MEDUSA_ERR_ARG, "tree has %d root-to-leaf paths, shape.P is %d", P, shape->P);
  if (dry) return MEDUSA_OK;
  a.B = shape->B;
  a.V = shape->V;
  a.S = shape->s_max;
  a.P = P;
  a.sample = draft_mode == MEDUSA_DRAFT_SAMPLE;
  a.root_tok = root_tok;
  a.topk_ids = topk_ids;
  a.head_logits = head_logits_or_null;
  a.head_lse = head_lse_or_null;
  a.u_draft = u_draft_or_null;
  a.kv_len = kv_len;
  a.tokens = tree_tokens;
  a.mask = tree_mask;
  a.position_ids = position_ids;
  a.retrieve = retrieve;
  a.parent = parent;
  a.depth = depth;
  hipError_t e = launch_tree(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tree launch");
  return ok();
}

}  // namespace

extern "C" {

int medusa_build_tree(const medusa_shape* shape, const int32_t* tree_ranks_host,
                      int draft_mode, const int32_t* root_tok, const int32_t* topk_ids,
                      const float* head_logits_or_null, const float* head_lse_or_null,
                      const float* u_draft_or_null, const int32_t* kv_len,
                      int32_t* tree_tokens, uint8_t* tree_mask, int32_t* position_ids,
                      int32_t* retrieve, int32_t* parent, int32_t* depth, void* stream) {
  return tree_impl(shape, tree_ranks_host, draft_mode, root_tok, topk_ids, head_logits_or_null,
                   head_lse_or_null, u_draft_or_null, kv_len, tree_tokens, tree_mask,
                   position_ids, retrieve, parent, depth, stream, false);
}

int medusa_tree_attention(const medusa_shape* shape, const void* q, const void* k_tree,
                          const void* v_tree, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, const uint8_t* tree_mask, float scale,
                          float* out, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k_tree);
  REQUIRE_PTR(v_tree);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(kv_len);
  REQUIRE_PTR(tree_mask);
  REQUIRE_PTR(out);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(MEDUSA_ERR_ARG, "scale must be positive");
  Layout L;
  rc = check_workspace(shape, workspace, workspace_bytes, &L);
  if (rc) return rc;
  AttnArgs a{};
  a.f32 = shape->dtype == MEDUSA_F32;
  a.B = shape->B;
  a.T = shape->N + 1;
  a.H = shape->H;
  a.Dh = shape->Dh;
  a.Lmax = shape->Lmax;
  a.q = q;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_len = kv_len;
  a.mask = tree_mask;
  a.scale = scale;
  a.NS = L.NS;
  a.part_o = at<float>(workspace, L.att_o);
  a.part_ml = at<float>(workspace, L.att_ml);
  a.out = out;
  a.out_elem = nullptr;
  hipError_t e = launch_tree_attention(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tree attention launch");
  return ok();
}

size_t medusa_packed_weight_bytes(const medusa_shape* shape, int rows) {
  if (check_shape(shape) != MEDUSA_OK) return 0;
  if (rows < 1) {
    fail(MEDUSA_ERR_ARG, "rows must be positive");
    return 0;
  }
  ok();
  return packed_weight_bytes(rows, shape->d, shape->dtype == MEDUSA_F32);
}

int medusa_pack_weight(const medusa_shape* shape, int kind, const void* W, int rows,
                       void* W_packed, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (rows < 1) return fail(MEDUSA_ERR_ARG, "rows must be positive");
  if (kind != MEDUSA_PACK_PLAIN && kind != MEDUSA_PACK_QKV)
    return fail(MEDUSA_ERR_ARG, "pack kind %d unknown", kind);
  if (kind == MEDUSA_PACK_QKV && rows != 3 * shape->d)
    return fail(MEDUSA_ERR_ARG, "MEDUSA_PACK_QKV needs rows = 3d = %d, got %d", 3 * shape->d,
                rows);
  REQUIRE_PTR(W);
  REQUIRE_PTR(W_packed);
  if (W == W_packed) return fail(MEDUSA_ERR_ARG, "W and W_packed must not overlap");
  hipError_t e = launch_pack_weight(shape->dtype == MEDUSA_F32, W, rows, shape->d,
                                    kind == MEDUSA_PACK_QKV ? shape->Dh : 0, W_packed,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

}  // extern "C"

namespace {

// Verify forward (shared by medusa_verify_forward and medusa_step).
int verify_impl(const medusa_shape* shape, const void* E, const void* W_qkv, const void* W_o,
                const void* W_lm, float rope_theta, const int32_t* tree_tokens,
                const int32_t* position_ids, const uint8_t* tree_mask, const int32_t* parent,
                const void* k_cache, const void* v_cache, const int32_t* kv_len,
                float temperature, void* k_tree_out, void* v_tree_out, float* y_out,
                float* row_stats, int32_t* row_argmax, float* child_logit,
                float* verify_logits_or_null, void* workspace, size_t workspace_bytes,
                void* stream, bool dry, bool merge_rows = true) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE_PTR(E);
  REQUIRE_PTR(W_qkv);
  REQUIRE_PTR(W_o);
  REQUIRE_PTR(W_lm);
  REQUIRE_PTR(tree_tokens);
  REQUIRE_PTR(position_ids);
  REQUIRE_PTR(tree_mask);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(kv_len);
  REQUIRE_PTR(k_tree_out);
  REQUIRE_PTR(v_tree_out);
  REQUIRE_PTR(y_out);
  REQUIRE_PTR(row_stats);
  REQUIRE_PTR(row_argmax);
  REQUIRE_PTR(child_logit);
  OPTIONAL_PTR(verify_logits_or_null);
  if (!(rope_theta > 1.f) || !isfinite(rope_theta))
    return fail(MEDUSA_ERR_ARG, "rope_theta must be > 1");
  if (!(temperature > 0.f) || !isfinite(temperature))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive");
  Layout L;
  rc = check_workspace(shape, workspace, workspace_bytes, &L);
  if (rc) return rc;
  if (dry) return MEDUSA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool f32 = shape->dtype == MEDUSA_F32;
  const int T = shape->N + 1, M = shape->B * T, d = shape->d;

  GemmParams g{};
  g.f32 = f32;
  g.T = T;
  g.H = shape->H;
  g.Dh = shape->Dh;
  g.a_mtiles = (M + 15) / 16;   // y in the LM head's A-fragment order
  // 1. q, k, v = RoPE(E[tok] Wq^T), RoPE(E[tok] Wk^T), E[tok] Wv^T
  g.M = M;
  g.N = 3 * d;
  g.K = d;
  g.A = E;
  g.lda = d;
  g.a_rows = tree_tokens;
  g.a_nrows = shape->V;
  g.W = W_qkv;
  g.pos = position_ids;
  g.log_theta = log((double)rope_theta);
  g.q_out = at<char>(workspace, L.q);
  g.k_out = k_tree_out;
  g.v_out = v_tree_out;
  g.part = at<float>(workspace, L.gemm_part);
  g.counters = at<int>(workspace, L.counters);
  hipError_t e = launch_qkv(g, st);
  if (e != hipSuccess) return hip_fail(e, "qkv launch");
  // 2. tree attention, output rounded to the storage type
  AttnArgs a{};
  a.f32 = f32;
  a.B = shape->B;
  a.T = T;
  a.H = shape->H;
  a.Dh = shape->Dh;
  a.Lmax = shape->Lmax;
  a.q = g.q_out;
  a.k_tree = k_tree_out;
  a.v_tree = v_tree_out;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_len = kv_len;
  a.mask = tree_mask;
  a.scale = 1.0f / sqrtf((float)shape->Dh);
  a.NS = L.NS;
  a.part_o = at<float>(workspace, L.att_o);
  a.part_ml = at<float>(workspace, L.att_ml);
  a.out = nullptr;
  a.out_elem = at<char>(workspace, L.o_elem);
  e = launch_tree_attention(a, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  // 3. y = x + o Wo^T
  GemmParams go = g;
  go.N = d;
  go.A = a.out_elem;
  go.a_rows = nullptr;
  go.a_nrows = shape->V;   // rows of E for the residual
  go.W = W_o;
  go.E = E;
  go.tokens = tree_tokens;
  go.y_out = y_out;
  go.y_elem = at<char>(workspace, L.y_elem);
  e = launch_oproj(go, st);
  if (e != hipSuccess) return hip_fail(e, "output projection launch");
  // 4. logits = y W_lm^T with row statistics and child logits
  GemmParams gl = g;
  gl.N = shape->V;
  gl.A = go.y_elem;
  gl.a_rows = nullptr;
  gl.W = W_lm;
  gl.tokens = tree_tokens;
  gl.parent = parent;
  gl.inv_tau = 1.0f / temperature;
  gl.part = at<float>(workspace, L.lm_part);
  gl.child_logit = child_logit;
  gl.logits_out = verify_logits_or_null;
  e = launch_lm_head(gl, row_stats, row_argmax, st, merge_rows);
  if (e != hipSuccess) return hip_fail(e, "lm head launch");
  return ok();
}

}  // namespace

extern "C" {

int medusa_verify_forward(const medusa_shape* shape, const void* E, const void* W_qkv,
                          const void* W_o, const void* W_lm, float rope_theta,
                          const int32_t* tree_tokens, const int32_t* position_ids,
                          const uint8_t* tree_mask, const int32_t* parent,
                          const void* k_cache, const void* v_cache, const int32_t* kv_len,
                          float temperature, void* k_tree_out, void* v_tree_out,
                          float* y_out, float* row_stats, int32_t* row_argmax,
                          float* child_logit, float* verify_logits_or_null,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(shape, E, W_qkv, W_o, W_lm, rope_theta, tree_tokens, position_ids,
                     tree_mask, parent, k_cache, v_cache, kv_len, temperature, k_tree_out,
                     v_tree_out, y_out, row_stats, row_argmax, child_logit,
                     verify_logits_or_null, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

namespace {

int posterior_impl(const medusa_shape* shape, int mode, float temperature, float eps,
                   float delta, const float* row_stats, const int32_t* row_argmax,
                   const float* child_logit, const float* verify_logits_or_null,
                   const int32_t* tree_tokens, const int32_t* parent, const int32_t* retrieve,
                   const float* head_logits_or_null, const float* head_lse_or_null,
                   const float* u_accept_or_null, const float* u_resample_or_null,
                   int32_t* accept_len, int32_t* best_path, int32_t* last_node,
                   int32_t* out_tokens, int32_t* next_root, void* workspace,
                   size_t workspace_bytes, void* stream, bool dry) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_EXACT)
    return fail(MEDUSA_ERR_ARG, "mode %d unknown", mode);
  if (!(temperature > 0.f) || !isfinite(temperature))
    return fail(MEDUSA_ERR_ARG, "temperature must be positive");
  REQUIRE_PTR(tree_tokens);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(retrieve);
  REQUIRE_PTR(accept_len);
  REQUIRE_PTR(best_path);
  REQUIRE_PTR(last_node);
  REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(next_root);
  if (mode == MEDUSA_GREEDY) {
    REQUIRE_PTR(row_argmax);
  } else if (mode == MEDUSA_TYPICAL) {
    REQUIRE_PTR(row_argmax);
    REQUIRE_PTR(row_stats);
    REQUIRE_PTR(child_logit);
    if (!(eps >= 0.f) || !(delta >= 0.f)) return fail(MEDUSA_ERR_ARG, "eps, delta must be >= 0");
  } else {
    REQUIRE_PTR(verify_logits_or_null);
    REQUIRE_PTR(head_logits_or_null);
    REQUIRE_PTR(head_lse_or_null);
    REQUIRE_PTR(u_accept_or_null);
    REQUIRE_PTR(u_resample_or_null);
  }
  Layout L;
  rc = check_workspace(shape, workspace, workspace_bytes, &L);
  if (rc) return rc;
  if (dry) return MEDUSA_OK;
  PostArgs a{};
  a.mode = mode;
  a.B = shape->B;
  a.T = shape->N + 1;
  a.K = shape->K;
  a.P = shape->P;
  a.V = shape->V;
  a.inv_tau = 1.0f / temperature;
  a.eps = eps;
  a.delta = delta;
  a.row_stats = row_stats;
  a.row_argmax = row_argmax;
  a.child_logit = child_logit;
  a.verify_logits = verify_logits_or_null;
  a.tokens = tree_tokens;
  a.parent = parent;
  a.retrieve = retrieve;
  a.head_logits = head_logits_or_null;
  a.head_lse = head_lse_or_null;
  a.u_accept = u_accept_or_null;
  a.u_resample = u_resample_or_null;
  a.pw = at<float>(workspace, L.pw);
  a.exact_dec = at<int32_t>(workspace, L.exact_dec);
  a.accept_len = accept_len;
  a.best_path = best_path;
  a.last_node = last_node;
  a.out_tokens = out_tokens;
  a.next_root = next_root;
  hipError_t e = launch_posterior(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "posterior launch");
  return ok();
}

}  // namespace

extern "C" {

int medusa_evaluate_posterior(const medusa_shape* shape, int mode, float temperature,
                              float eps, float delta, const float* row_stats,
                              const int32_t* row_argmax, const float* child_logit,
                              const float* verify_logits_or_null,
                              const int32_t* tree_tokens, const int32_t* parent,
                              const int32_t* retrieve, const float* head_logits_or_null,
                              const float* head_lse_or_null, const float* u_accept_or_null,
                              const float* u_resample_or_null, int32_t* accept_len,
                              int32_t* best_path, int32_t* last_node, int32_t* out_tokens,
                              int32_t* next_root, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return posterior_impl(shape, mode, temperature, eps, delta, row_stats, row_argmax, child_logit,
                        verify_logits_or_null, tree_tokens, parent, retrieve,
                        head_logits_or_null, head_lse_or_null, u_accept_or_null,
                        u_resample_or_null, accept_len, best_path, last_node, out_tokens,
                        next_root, workspace, workspace_bytes, stream, false);
}

}  // extern "C"

namespace {
int commit_impl(const medusa_shape* shape, const int32_t* last_node, const int32_t* parent,
                const void* k_tree, const void* v_tree, const float* y, void* k_cache,
                void* v_cache, int32_t* kv_len, int32_t* kv_len_out, float* h_next,
                void* stream, bool dry) {
  int rc = check_shape(shape);
  if (rc) return rc;
  REQUIRE_PTR(last_node);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(k_tree);
  REQUIRE_PTR(v_tree);
  REQUIRE_PTR(y);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  REQUIRE_PTR(kv_len);
  REQUIRE_PTR(h_next);
  OPTIONAL_PTR(kv_len_out);
  if (dry) return MEDUSA_OK;
  CommitArgs a{};
  a.f32 = shape->dtype == MEDUSA_F32;
  a.B = shape->B;
  a.T = shape->N + 1;
  a.K = shape->K;
  a.H = shape->H;
  a.Dh = shape->Dh;
  a.d = shape->d;
  a.Lmax = shape->Lmax;
  a.last_node = last_node;
  a.parent = parent;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.y = y;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.kv_len = kv_len;
  a.kv_len_out = kv_len_out;
  a.h_next = h_next;
  hipError_t e = launch_commit(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "commit launch");
  return ok();
}
}  // namespace

extern "C" {

int medusa_commit(const medusa_shape* shape, const int32_t* last_node, const int32_t* parent,
                  const void* k_tree, const void* v_tree, const float* y, void* k_cache,
                  void* v_cache, int32_t* kv_len, float* h_next, void* stream) {
  return commit_impl(shape, last_node, parent, k_tree, v_tree, y, k_cache, v_cache, kv_len,
                     nullptr, h_next, stream, false);
}

}  // extern "C"

namespace {

// The composite step. With dry set it runs every check of every stage and
// launches nothing, so that a caller can validate a whole step (or a whole
// loop of steps) before its first launch.
int step_impl(const medusa_shape* shape, const medusa_step_args* x, void* workspace,
              size_t workspace_bytes, void* stream, bool dry, hipEvent_t ev_w2_start = nullptr,
              hipEvent_t ev_w2_end = nullptr) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!x) return fail(MEDUSA_ERR_ARG, "args: null pointer");
  const int mode = x->mode;
  if (mode != MEDUSA_GREEDY && mode != MEDUSA_TYPICAL && mode != MEDUSA_EXACT)
    return fail(MEDUSA_ERR_ARG, "mode %d unknown", mode);
  if (x->draft_mode != MEDUSA_DRAFT_TOPK && x->draft_mode != MEDUSA_DRAFT_SAMPLE)
    return fail(MEDUSA_ERR_ARG, "draft_mode %d unknown", x->draft_mode);
  // spec-only topology written once by medusa_build_tree, read here
  REQUIRE_PTR(x->tree_mask);
  REQUIRE_PTR(x->parent);
  REQUIRE_PTR(x->retrieve);
  REQUIRE_PTR(x->root_tok);
  REQUIRE_PTR(x->kv_len);
  REQUIRE_PTR(x->tree_tokens);
  REQUIRE_PTR(x->position_ids);
  TreePlan plan;
  int P = 0;
  rc = make_plan(shape, x->tree_ranks_host, &plan, &P);
  if (rc) return rc;
  if (P != shape->P)
    return fail(MEDUSA_ERR_ARG, "tree has %d root-to-leaf paths, shape.P is %d", P, shape->P);
  Layout L;
  rc = check_workspace(shape, workspace, workspace_bytes, &L);
  if (rc) return rc;
  const bool fuse_tree = x->draft_mode == MEDUSA_DRAFT_TOPK;
  // greedy / typical: posterior and commit in one kernel, checked here
  const bool fuse_post = mode != MEDUSA_EXACT;
  if (fuse_post) {
    REQUIRE_PTR(x->accept_len);
    REQUIRE_PTR(x->best_path);
    REQUIRE_PTR(x->last_node);
    REQUIRE_PTR(x->out_tokens);
    REQUIRE_PTR(x->next_root);
    REQUIRE_PTR(x->h_next);
    OPTIONAL_PTR(x->kv_len_out_or_null);
    if (mode == MEDUSA_TYPICAL && (!(x->eps >= 0.f) || !(x->delta >= 0.f)))
      return fail(MEDUSA_ERR_ARG, "eps, delta must be >= 0");
  }
  // 1. heads, with the tree's tokens and positions: top-s drafting in the
  // head merge, sampled drafting in workgroups launched beside it
  rc = heads_impl(shape, x->h, x->W1, x->W1_packed_or_null, x->b1_or_null, x->W2,
                  x->W2_packed_or_null, x->topk_ids,
                  x->topk_logits,
                  x->head_lse_or_null, x->head_logits_or_null, x->z_or_null, workspace,
                  workspace_bytes, stream, &plan, x->root_tok, x->kv_len, x->tree_tokens,
                  x->position_ids, fuse_tree ? nullptr : x->u_draft_or_null, dry, ev_w2_start,
                  ev_w2_end);
  if (rc) return rc;
  // 2. sampled drafting: the tree sampler's checks (its draws ran with the heads)
  if (!fuse_tree && dry) {
    rc = tree_impl(shape, x->tree_ranks_host, x->draft_mode, x->root_tok, x->topk_ids,
                   x->head_logits_or_null, x->head_lse_or_null, x->u_draft_or_null, x->kv_len,
                   x->tree_tokens, nullptr, x->position_ids, nullptr, nullptr, nullptr, stream,
                   true);
    if (rc) return rc;
  }
  // 3. verify forward
  rc = verify_impl(shape, x->E, x->W_qkv, x->W_o, x->W_lm, x->rope_theta, x->tree_tokens,
                   x->position_ids, x->tree_mask, x->parent, x->k_cache, x->v_cache, x->kv_len,
                   x->temperature, x->k_tree, x->v_tree, x->y, x->row_stats, x->row_argmax,
                   x->child_logit, x->verify_logits_or_null, workspace, workspace_bytes, stream,
                   dry, fuse_post);
  if (rc) return rc;
  // 4. posterior and commit (exact mode: the two calls' checks, then the
  // node-parallel posterior with the walk and the commit in one kernel)
  if (!fuse_post) {
    rc = posterior_impl(shape, mode, x->temperature, x->eps, x->delta, x->row_stats,
                        x->row_argmax, x->child_logit, x->verify_logits_or_null, x->tree_tokens,
                        x->parent, x->retrieve, x->head_logits_or_null, x->head_lse_or_null,
                        x->u_accept_or_null, x->u_resample_or_null, x->accept_len, x->best_path,
                        x->last_node, x->out_tokens, x->next_root, workspace, workspace_bytes,
                        stream, true);
    if (rc) return rc;
    rc = commit_impl(shape, x->last_node, x->parent, x->k_tree, x->v_tree, x->y,
                     x->k_cache, x->v_cache, x->kv_len, x->kv_len_out_or_null, x->h_next,
                     stream, true);
    if (rc) return rc;
  }
  if (dry) return MEDUSA_OK;
  PostArgs a{};
  a.mode = mode;
  a.B = shape->B;
  a.T = shape->N + 1;
  a.K = shape->K;
  a.P = shape->P;
  a.V = shape->V;
  a.inv_tau = 1.0f / x->temperature;
  a.eps = x->eps;
  a.delta = x->delta;
  a.child_logit = x->child_logit;
  a.tokens = x->tree_tokens;
  a.parent = x->parent;
  a.retrieve = x->retrieve;
  a.accept_len = x->accept_len;
  a.best_path = x->best_path;
  a.last_node = x->last_node;
  a.out_tokens = x->out_tokens;
  a.next_root = x->next_root;
  a.verify_logits = x->verify_logits_or_null;
  a.head_logits = x->head_logits_or_null;
  a.head_lse = x->head_lse_or_null;
  a.u_accept = x->u_accept_or_null;
  a.u_resample = x->u_resample_or_null;
  a.pw = at<float>(workspace, L.pw);
  a.exact_dec = at<int32_t>(workspace, L.exact_dec);
  if (!fuse_post) {
    // exact mode: the LM head's row-statistics merge runs with the posterior
    a.lm_part = at<float>(workspace, L.lm_part);
    a.lm_G = lm_head_blocks(shape->V, a.B * a.T, shape->dtype == MEDUSA_F32);
    a.row_stats_out = x->row_stats;
    a.row_argmax_out = x->row_argmax;
  }
  CommitArgs c{};
  c.f32 = shape->dtype == MEDUSA_F32;
  c.B = shape->B;
  c.T = shape->N + 1;
  c.K = shape->K;
  c.H = shape->H;
  c.Dh = shape->Dh;
  c.d = shape->d;
  c.Lmax = shape->Lmax;
  c.parent = x->parent;
  c.k_tree = x->k_tree;
  c.v_tree = x->v_tree;
  c.y = x->y;
  c.k_cache = x->k_cache;
  c.v_cache = x->v_cache;
  c.kv_len = x->kv_len;
  c.kv_len_out = x->kv_len_out_or_null;
  c.h_next = x->h_next;
  c.counters = at<int>(workspace, L.counters) + kCommitCounter;
  a.row_stats = x->row_stats;
  a.row_argmax = x->row_argmax;
  hipError_t e = launch_posterior_commit(a, c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "posterior launch");
  return ok();
}

}  // namespace

extern "C" {

int medusa_step(const medusa_shape* shape, const medusa_step_args* x, void* workspace,
                size_t workspace_bytes, void* stream) {
  const int rc = step_impl(shape, x, workspace, workspace_bytes, stream, true);
  if (rc) return rc;
  return step_impl(shape, x, workspace, workspace_bytes, stream, false);
}

int medusa_step_timed(const medusa_shape* shape, const medusa_step_args* x, void* workspace,
                      size_t workspace_bytes, void* stream, void* ev_w2_start, void* ev_w2_end) {
  if (!ev_w2_start || !ev_w2_end) return fail(MEDUSA_ERR_ARG, "step_timed: null event");
  const int rc = step_impl(shape, x, workspace, workspace_bytes, stream, true);
  if (rc) return rc;
  return step_impl(shape, x, workspace, workspace_bytes, stream, false,
                   static_cast<hipEvent_t>(ev_w2_start), static_cast<hipEvent_t>(ev_w2_end));
}

}  // extern "C"

// ---- calibrated sparse tree (host) -------------------------------------------------
namespace {

// A rank path and its weight prod_j a[j][r_j]; the weight of a child is its
// parent's times one more factor, the product taken in path order.
struct TreePath {
  double w;
  int len;
  int8_t r[MEDUSA_MAX_K];
};

// Lexicographic order of rank paths (a proper prefix comes first).
bool path_less(const TreePath& x, const TreePath& y) {
  const int n = std::min(x.len, y.len);
  for (int i = 0; i < n; ++i)
    if (x.r[i] != y.r[i]) return x.r[i] < y.r[i];
  return x.len < y.len;
}

// x is picked before y: larger weight, then the lexicographically smaller path.
bool picked_before(const TreePath& x, const TreePath& y) {
  if (x.w != y.w) return x.w > y.w;
  return path_less(x, y);
}

}  // namespace

extern "C" {

int medusa_sparse_tree(int K, int S, const double* a_host, int budget, int32_t* tree_ranks_host,
                       double* weights_host_or_null, int32_t* pick_order_host_or_null,
                       int32_t* n_nodes_host) {
  if (!a_host || !tree_ranks_host || !n_nodes_host)
    return fail(MEDUSA_ERR_ARG, "sparse tree: null pointer");
  if (K < 1 || S < 1 || budget < 0)
    return fail(MEDUSA_ERR_ARG, "sparse tree: K=%d, S=%d, budget=%d", K, S, budget);
  if (K > MEDUSA_MAX_K || S > MEDUSA_MAX_S || budget > MEDUSA_MAX_T - 1)
    return fail(MEDUSA_ERR_UNSUPPORTED, "sparse tree: K=%d > %d, S=%d > %d or budget=%d > %d", K,
                MEDUSA_MAX_K, S, MEDUSA_MAX_S, budget, MEDUSA_MAX_T - 1);
  for (int i = 0; i < K * S; ++i)
    if (!(a_host[i] >= 0.0) || !std::isfinite(a_host[i]))
      return fail(MEDUSA_ERR_ARG, "sparse tree: a[%d][%d] = %g is not a finite probability",
                  i / S, i % S, a_host[i]);
  // frontier: a heap whose top is the path picked next
  auto heap_less = [](const TreePath& x, const TreePath& y) { return picked_before(y, x); };
  std::vector<TreePath> frontier;
  frontier.reserve((size_t)S * (budget + 1));
  for (int r = 0; r < S; ++r) {
    TreePath t{};
    t.w = 1.0 * a_host[r];
    t.len = 1;
    t.r[0] = (int8_t)r;
    frontier.push_back(t);
  }
  std::make_heap(frontier.begin(), frontier.end(), heap_less);
  std::vector<TreePath> picks;
  picks.reserve(budget);
  while ((int)picks.size() < budget && !frontier.empty()) {
    std::pop_heap(frontier.begin(), frontier.end(), heap_less);
    const TreePath best = frontier.back();
    frontier.pop_back();
    picks.push_back(best);
    if (best.len < K) {
      for (int r = 0; r < S; ++r) {
        TreePath c = best;
        c.w = best.w * a_host[best.len * S + r];
        c.r[c.len++] = (int8_t)r;
        frontier.push_back(c);
        std::push_heap(frontier.begin(), frontier.end(), heap_less);
      }
    }
  }
  // canonical order: depth, then lexicographic
  const int N = (int)picks.size();
  std::vector<int> idx(N);
  for (int i = 0; i < N; ++i) idx[i] = i;
  std::sort(idx.begin(), idx.end(), [&](int x, int y) {
    if (picks[x].len != picks[y].len) return picks[x].len < picks[y].len;
    return path_less(picks[x], picks[y]);
  });
  std::vector<int> canon_of(N);
  for (int c = 0; c < N; ++c) {
    const TreePath& t = picks[idx[c]];
    canon_of[idx[c]] = c;
    for (int j = 0; j < K; ++j) tree_ranks_host[(size_t)c * K + j] = j < t.len ? t.r[j] : -1;
    if (weights_host_or_null) weights_host_or_null[c] = t.w;
  }
  if (pick_order_host_or_null)
    for (int i = 0; i < N; ++i) pick_order_host_or_null[i] = canon_of[i];
  *n_nodes_host = N;
  return ok();
}

}  // extern "C"

// ---- decode loop -------------------------------------------------------------------
extern "C" {

int medusa_generate(const medusa_shape* shape, const medusa_step_args* args, int n_steps,
                    int32_t* out_tokens_steps, int32_t* accept_len_steps, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!args) return fail(MEDUSA_ERR_ARG, "generate: args: null pointer");
  REQUIRE_PTR(out_tokens_steps);
  REQUIRE_PTR(accept_len_steps);
  if (n_steps < 0) return fail(MEDUSA_ERR_ARG, "generate: n_steps=%d", n_steps);
  if (args->kv_len_out_or_null)
    return fail(MEDUSA_ERR_ARG, "generate: the loop advances kv_len in place (kv_len_out_or_null must be NULL)");
  REQUIRE_PTR(args->h);
  REQUIRE_PTR(args->h_next);
  REQUIRE_PTR(args->root_tok);
  REQUIRE_PTR(args->next_root);
  const size_t B = shape->B, T = shape->N + 1, K1 = shape->K + 1;
  // the state alternates between (h, root_tok) and (h_next, next_root)
  float* hs[2] = {const_cast<float*>(args->h), args->h_next};
  int32_t* roots[2] = {const_cast<int32_t*>(args->root_tok), args->next_root};
  const auto step_args = [&](int i) {
    medusa_step_args x = *args;
    const int cur = i & 1;
    x.h = hs[cur];
    x.root_tok = roots[cur];
    x.h_next = hs[cur ^ 1];
    x.next_root = roots[cur ^ 1];
    x.out_tokens = out_tokens_steps + (size_t)i * MEDUSA_ALIGN4(B * K1);
    x.accept_len = accept_len_steps + (size_t)i * MEDUSA_ALIGN4(B);
    // per-step uniform blocks keep the 16-byte alignment of the first
    const size_t ustep = (size_t)i * MEDUSA_ALIGN4(B * T);
    if (args->u_draft_or_null) x.u_draft_or_null = args->u_draft_or_null + ustep;
    if (args->u_accept_or_null) x.u_accept_or_null = args->u_accept_or_null + ustep;
    if (args->u_resample_or_null) x.u_resample_or_null = args->u_resample_or_null + ustep;
    return x;
  };
  // every step is validated before the first launch
  for (int i = 0; i < n_steps; ++i) {
    const medusa_step_args x = step_args(i);
    rc = step_impl(shape, &x, workspace, workspace_bytes, stream, true);
    if (rc) return rc;
  }
  for (int i = 0; i < n_steps; ++i) {
    const medusa_step_args x = step_args(i);
    rc = step_impl(shape, &x, workspace, workspace_bytes, stream, false);
    if (rc) return rc;
  }
  if (n_steps & 1) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(hs[0], hs[1], B * shape->d * sizeof(float),
                                  hipMemcpyDeviceToDevice, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(roots[0], roots[1], B * sizeof(int32_t), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "generate: state copy");
  }
  return ok();
}

}  // extern "C"


// ---- step without a caller workspace -------------------------------------------
// The workspace lives in a file-scope device array, one copy per GPU, whose
// address each device reports once through hipGetSymbolAddress; host code
// uses that address only (the array's own name is a host-side stand-in).
namespace {

__device__ __align__(256) unsigned char scratch[MEDUSA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Zeroes n 16-byte words (the counter block every call needs at zero).
__global__ __launch_bounds__(256) void zero_words_kernel(uint4* p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "step_static: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MEDUSA_ERR_UNSUPPORTED, "step_static: device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "step_static: hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
      return fail(MEDUSA_ERR_HIP, "step_static: scratch address %p is not 256-byte aligned", p);
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MEDUSA_OK;
}

}  // namespace

extern "C" {

int medusa_step_static(const medusa_shape* shape, const medusa_step_args* x, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  const size_t need = layout_for(shape).total;
  if (need > (size_t)MEDUSA_STATIC_WORKSPACE_BYTES)
    return fail(MEDUSA_ERR_WORKSPACE,
                "step_static: this shape needs %zu workspace bytes, more than the %zu of the "
                "library's static workspace (use medusa_step with a caller workspace)",
                need, (size_t)MEDUSA_STATIC_WORKSPACE_BYTES);
  void* ws = nullptr;
  rc = scratch_for_current_device(&ws);
  if (rc) return rc;
  rc = step_impl(shape, x, ws, need, stream, true);
  if (rc) return rc;
  // the counters start at zero (the previous call left them so unless it
  // was cut short); a fill kernel rather than a memset, so that the call
  // can be captured in a graph
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int words = (int)(kCounterBytes / 16);
  hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                     static_cast<uint4*>(ws), words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "step_static: counter clear launch");
  return step_impl(shape, x, ws, need, stream, false);
}

}  // extern "C"
