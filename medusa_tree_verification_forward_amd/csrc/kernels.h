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

// ---- tree --------------------------------------------------------------------
// The host-validated tree spec, passed to the kernel by value: for node n
// (canonical order, node 0 = root) its parent index and the rank of its own
// token inside its depth's pool.
struct TreePlan {
  int T;
  int K;
  uint8_t parent[MAXT];      // parent[0] unused
  uint8_t last_rank[MAXT];   // last_rank[0] unused
  uint8_t depth[MAXT];       // depth[0] = 0
};
// ---- heads -------------------------------------------------------------------
struct HeadsArgs {
  bool f32;
  int B, d, V, K, S;
  const float* h;
  const void* W1;
  const void* W1_packed;  // or null: W1 packed as one [K d][d] matrix (plain)
  const float* b1;        // may be null
  const void* W2;
  const void* W2_packed;  // or null: each head's W2_k packed (plain, rows = V), heads in order
  float* z;               // [B][K][d]
  float* head_logits;     // [B][K][V] or null
  int* topk_ids;          // [B][K][S]
  float* topk_logits;     // [B][K][S]
  float* lse;             // [B][K] or null
  float* part_val;        // [B][K][G][S]
  int* part_id;           // [B][K][G][S]
  float* part_m;          // [B][K][G]
  float* part_s;          // [B][K][G]
  void* afrag;            // (K + 1) * 32 * d bytes: MFMA A fragments of the batched passes
  int G;                  // row blocks per head (4 waves of w2_rows_per_wave rows)
  int w1_rows_per_wave;   // 1..64, or 0: the fewest that fit one wave of resident workgroups
  int w2_rows_per_wave;   // 4..64
  hipEvent_t ev_before;   // optional: recorded around the W2 kernel
  hipEvent_t ev_after;
  // optional (composite step): the tree's tokens and positions with the
  // merge -- top-s drafting (u_draft null): the merge of head k writes the
  // tokens of the depth-(k+1) nodes, head 0 the root token and every
  // position id; sampled drafting: workgroups beside the merge draw them
  // from head_logits with u_draft
  bool fuse_tree;
  TreePlan plan;
  const int32_t* root_tok;     // [B]
  const int32_t* kv_len;       // [B]
  int32_t* tree_tokens;        // [B][T]
  int32_t* position_ids;       // [B][T]
  const float* u_draft;        // [B][T] or null
};
hipError_t launch_heads(const HeadsArgs& a, hipStream_t st);
// Row blocks a head's partial records can need: the per-row streams'
// workgroups of 4 waves x rows_per_wave rows, or the batched passes' (3 or
// more sequences) smaller ones, whichever gives more.
int heads_row_blocks_max(int V, int rows_per_wave);

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
  uint8_t* mask;                 // [T][T] or null
  int32_t* position_ids;         // [B][T]
  int32_t* retrieve;             // [P][K+1] or null
  int32_t* parent;               // [T] or null
  int32_t* depth;                // [T] or null
};
hipError_t launch_tree(const TreeArgs& a, hipStream_t st);

// ---- node GEMMs (verify pass) ---------------------------------------------------
enum { EPI_QKV = 0, EPI_OPROJ = 1, EPI_LM = 2 };
struct GemmParams {
  bool f32;
  int M, N, K;                 // C[M][N] = A[M][K] * W[N][K]^T
  const void* A;               // [M][lda] (QKV, OPROJ) or A-fragment order (LM head)
  int lda;
  int a_mtiles;                // m-tiles of the fragment-ordered LM-head A and OPROJ y_elem
  const int32_t* a_rows;       // optional: A row of output row m is a_rows[m]
  int a_nrows;                 // rows of A (gathered indices are clamped into range)
  const void* W;
  // QKV epilogue
  int T, H, Dh;
  const int32_t* pos;          // [M] position ids
  double log_theta;
  void* q_out;
  void* k_out;
  void* v_out;                 // [M][H][Dh] storage type
  // OPROJ epilogue (and LM child logits)
  const void* E;
  const int32_t* tokens;       // [M]
  float* y_out;                // [M][N] fp32
  void* y_elem;                // storage type in A-fragment order over a_mtiles m-tiles
                               // (frag_index), rows M .. 16 a_mtiles - 1 zero
  // LM epilogue
  float inv_tau;
  float* part;                 // LM: [M][groups][4]; QKV/OPROJ: [groups][M][cols][KS]
  const int32_t* parent;       // [T]
  float* child_logit;          // [M]
  float* logits_out;           // [M][N] or null
  int* counters;               // split-K hand-off: one zeroed counter per (group, pass)
  int group_cols;              // set by the launcher
};
// Weights W[rows][K] of the node GEMMs are packed into MFMA tiles (see
// node_gemm.hip) before use; pair_dh = Dh reorders the rows of each head
// into rotation pairs (W_qkv), 0 keeps them in order.
size_t packed_weight_bytes(int rows, int K, bool f32);
hipError_t launch_pack_weight(bool f32, const void* W, int rows, int K, int pair_dh, void* out,
                              hipStream_t st);
int gemm_groups_max(int N);                // column groups of a node GEMM (upper bound)
int gemm_passes_max(int M);                // row passes (upper bound)
int lm_head_blocks(int N, int M, bool f32);   // row records of the LM head (per stripe or workgroup)
int lm_record_slots(int N);                // upper bound of lm_head_blocks over the configs
int gemm_splits(int epi, int N, int K, bool f32, int M);   // K slices of the QKV / output projection of M rows
hipError_t launch_qkv(const GemmParams& p, hipStream_t st);
hipError_t launch_oproj(const GemmParams& p, hipStream_t st);
// merge_rows = false leaves the row-statistics merge of the records in
// p.part to the caller (the exact-mode composite step runs it beside the
// node posterior).
hipError_t launch_lm_head(GemmParams p, float* row_stats, int* row_argmax, hipStream_t st,
                          bool merge_rows = true);
hipError_t launch_row_stats_merge(const float* part, int G, int M, float inv_tau,
                                  float* row_stats, int* row_argmax, hipStream_t st);

// ---- tree attention ---------------------------------------------------------------
constexpr int kAttnChunk = 256;   // prefix keys per split
struct AttnArgs {
  bool f32;
  int B, T, H, Dh, Lmax;
  const void* q;
  const void* k_tree;
  const void* v_tree;          // [B][T][H][Dh]
  const void* k_cache;
  const void* v_cache;         // [B][H][Lmax][Dh]
  const int32_t* kv_len;       // [B]
  const uint8_t* mask;         // [T][T]
  float scale;
  int NS;                      // prefix splits per (b, h) (kAttnChunk keys each)
  int NP;                      // partials per (b, h) the merge reads (set by the launcher)
  int qgroups;                 // per-wave kernel: groups of 3 query tiles
  int chunk_sets;              // per-wave kernel: units per query group (see `balanced`)
  int balanced;                // per-wave kernel: units are chunk_sets balanced ranges of all
                               // (b, h, chunk) in order, else (b, h, chunk set) triples
  float* part_o;               // [B][H][NS][Dh/16][T][16]
  float* part_ml;              // [B][H][NS][T][2]
  float* out;                  // [B][T][H][Dh] fp32 (or null)
  void* out_elem;              // [B][T][H][Dh] storage type (or null)
};
int attn_splits(int Lmax);
// prefix chunks of a sequence whose KV length is `len` (clamped to [0, Lmax])
__host__ __device__ inline int attn_chunks(int len, int Lmax) {
  const int L = len < 0 ? 0 : (len > Lmax ? Lmax : len);
  return (L + kAttnChunk - 1) / kAttnChunk;
}
int device_cus();   // compute units of the current device (cached per device)
hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st);

// ---- posterior and commit -------------------------------------------------------------
struct PostArgs {
  int mode;                    // 0 greedy, 1 typical, 2 exact
  int B, T, K, P, V;
  float inv_tau, eps, delta;
  const float* row_stats;      // [B][T][3]
  const int32_t* row_argmax;   // [B][T]
  const float* child_logit;    // [B][T]
  const float* verify_logits;  // [B][T][V] (exact)
  const int32_t* tokens;       // [B][T]
  const int32_t* parent;       // [T]
  const int32_t* retrieve;     // [P][K+1]
  const float* head_logits;    // [B][K][V] (exact)
  const float* head_lse;       // [B][K] (exact)
  const float* u_accept;       // [B][T] (exact)
  const float* u_resample;     // [B][T] (exact)
  float* pw;                   // [B][V] workspace (exact, large vocabularies)
  int32_t* exact_dec;          // [B][T][2] workspace (exact): first accepted child, draw
  int32_t* accept_len;
  int32_t* best_path;
  int32_t* last_node;
  int32_t* out_tokens;         // [B][K+1]
  int32_t* next_root;
  // exact-mode composite step: the row-statistics merge of the LM head's
  // records, run by extra workgroups of the node posterior (null: not)
  const float* lm_part;        // [B T][lm_G][4]
  int lm_G;
  float* row_stats_out;        // [B][T][3]
  int32_t* row_argmax_out;     // [B][T]
};
hipError_t launch_posterior(const PostArgs& a, hipStream_t st);

struct CommitArgs {
  bool f32;
  int B, T, K, H, Dh, d, Lmax;
  const int32_t* last_node;
  const int32_t* parent;
  const void* k_tree;
  const void* v_tree;
  const float* y;
  void* k_cache;
  void* v_cache;
  int32_t* kv_len;
  int32_t* kv_len_out;         // advanced lengths go here; null: kv_len in place
  float* h_next;
  int* counters;               // [B] zeroed, left at zero (composite step)
};
constexpr int kCommitParts = 16;   // composite step: workgroups per sequence, at most
hipError_t launch_commit(const CommitArgs& a, hipStream_t st);
// Composite step: greedy / typical posterior + commit in one kernel (several
// workgroups a sequence); exact mode: the node-parallel posterior, then the
// walk + commit in one kernel (large vocabularies: the separate kernels).
hipError_t launch_posterior_commit(const PostArgs& a, const CommitArgs& c, hipStream_t st);

}  // namespace medusa
