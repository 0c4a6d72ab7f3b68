// Internal launch interface between the C ABI (capi.hip) and the kernels.
// Every argument here has been validated by the C ABI before a launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace medusa {

constexpr int MAXS_LDS = 16;   // top-s list slots (>= MEDUSA_MAX_S)
constexpr int MAXT = 256;      // tree rows
constexpr int MAXK = 8;        // tree depth

// ---- heads -------------------------------------------------------------------
struct HeadsArgs {
  bool f32;
  int B, d, V, K, S;
  const float* h;
  const void* W1;
  const float* b1;        // may be null
  const void* W2;
  float* z;               // [B][K][d]
  float* head_logits;     // [B][K][V] or null
  int* topk_ids;          // [B][K][S]
  float* topk_logits;     // [B][K][S]
  float* lse;             // [B][K] or null
  float* part_val;        // [B][K][G][S]
  int* part_id;           // [B][K][G][S]
  float* part_m;          // [B][K][G]
  float* part_s;          // [B][K][G]
  int G;                  // row blocks per head
  int w1_rows_per_wg;
  int w2_rows_per_wg;
};
hipError_t launch_heads(const HeadsArgs& a, hipStream_t st);

// ---- tree --------------------------------------------------------------------
// The host-validated tree spec, passed to the kernel by value: for node n
// (canonical order, node 0 = root) its parent index and the rank of its own
// token inside its depth's pool.
struct TreePlan {
  int T;
  int K;
  uint8_t parent[MAXT];      // parent[0] unused
  uint8_t last_rank[MAXT];   // last_rank[0] unused
};
struct TreeArgs {
  TreePlan plan;
  int B, V, S, P;
  int sample;                    // 0: top-s tokens, 1: draws from the head softmaxes
  const int32_t* root_tok;       // [B]
  const int32_t* topk_ids;       // [B][K][S]
  const float* head_logits;      // [B][K][V] (sample mode)
  const float* head_lse;         // [B][K] (sample mode)
  const float* u_draft;          // [B][T] (sample mode)
  const int32_t* kv_len;         // [B]
  int32_t* tokens;               // [B][T]
  uint8_t* mask;                 // [T][T]
  int32_t* position_ids;         // [B][T]
  int32_t* retrieve;             // [P][K+1]
  int32_t* parent;               // [T]
  int32_t* depth;                // [T]
};
hipError_t launch_tree(const TreeArgs& a, hipStream_t st);

}  // namespace medusa
