/*
 * medusa.h -- C ABI of the MI355X (gfx950) Medusa verify-step library.
 *
 * One Medusa draft-and-verify step, as the pages describe it:
 *   1. K Medusa heads read the shared last hidden state h and propose
 *      per-depth top-s token pools ("Medusa 深读", §3.1, head equation);
 *   2. the pools form a candidate tree stored with shared prefixes, with an
 *      ancestor-only attention mask and one position index per depth
 *      ("Medusa 深读", §6.1);
 *   3. the target model scores every tree node in one masked forward pass
 *      ("Medusa: Faster LLM text generation", Tree attention);
 *   4. an acceptance rule (greedy match, typical acceptance, exact p/q
 *      rejection) keeps the longest accepted prefix, whose first token is
 *      always committed ("Medusa 深读", §5; "Medusa: Faster LLM text
 *      generation", Acceptance rules).
 *
 * Conventions for every call:
 *   - Every pointer is DEVICE memory unless its comment says "host".
 *   - The caller owns every buffer, including the workspace. The library
 *     allocates no memory and keeps no state between calls; calls on one
 *     stream run in order, calls that share a workspace must not overlap.
 *   - All calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream). The library never synchronises.
 *   - Arguments are validated on the host before any launch. On failure the
 *     call returns a negative code, launches nothing and writes nothing;
 *     medusa_last_error() then describes the failure (thread-local).
 *   - Element type `elem` of weights, embeddings, KV cache and q/k/v is bf16
 *     (MEDUSA_BF16, uint16 bit patterns) or fp32 (MEDUSA_F32), per
 *     medusa_shape.dtype. Activations h, z, y and logits are fp32.
 *   - Matrices are row-major [out][in]: a projection computes X * W^T with
 *     both operands contiguous along the hidden dimension.
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codes ------------------------------------------------------------- */
#define MEDUSA_OK 0
#define MEDUSA_ERR_ARG (-1)          /* null/misaligned pointer, bad shape, bad tree spec */
#define MEDUSA_ERR_UNSUPPORTED (-2)  /* outside the kernels' limits (below)              */
#define MEDUSA_ERR_WORKSPACE (-3)    /* workspace smaller than medusa_workspace_bytes()  */
#define MEDUSA_ERR_CAPACITY (-4)     /* no KV room to commit a full path                 */
#define MEDUSA_ERR_HIP (-5)          /* a kernel launch failed                           */

#define MEDUSA_BF16 0
#define MEDUSA_F32 1

/* Acceptance rules ("Medusa 深读", §5 rule table). */
#define MEDUSA_GREEDY 0   /* accept while the draft equals the parent's argmax             */
#define MEDUSA_TYPICAL 1  /* accept iff p(x) > min(eps, delta*exp(-H(p))), p at temperature */
#define MEDUSA_EXACT 2    /* accept iff u*q(x) < p(x); on rejection p <- norm((p-q)+)        */

/* Drafting: top-s pools, or i.i.d. draws from the head softmaxes (exact mode). */
#define MEDUSA_DRAFT_TOPK 0
#define MEDUSA_DRAFT_SAMPLE 1

/* Kernel limits. */
#define MEDUSA_MAX_T 256      /* tree rows (root + nodes)          */
#define MEDUSA_MAX_K 8        /* heads = tree depth                */
#define MEDUSA_MAX_S 16       /* top-s pool width                  */
#define MEDUSA_MAX_B 64       /* sequences per call                */

/*
 * Problem shape. T = N + 1 tree rows (the root token is a real row of the
 * verify pass). P = number of root-to-leaf paths of the tree spec.
 * H * Dh must equal d.
 */
typedef struct medusa_shape {
  int32_t B;      /* sequences                                         */
  int32_t d;      /* hidden width, multiple of 64                      */
  int32_t V;      /* vocabulary                                        */
  int32_t K;      /* Medusa heads = tree depth, 1..MEDUSA_MAX_K        */
  int32_t H;      /* attention heads of the verifier layer             */
  int32_t Dh;     /* head dimension, 64 or 128                         */
  int32_t Lmax;   /* KV cache rows per (sequence, head)                */
  int32_t N;      /* non-root tree nodes, T = N + 1 <= MEDUSA_MAX_T    */
  int32_t P;      /* root-to-leaf paths of the tree                    */
  int32_t s_max;  /* pool width every head keeps, 1..MEDUSA_MAX_S      */
  int32_t dtype;  /* MEDUSA_BF16 or MEDUSA_F32                         */
} medusa_shape;

/* Message of the last failed call on this thread ("" if none). */
const char* medusa_last_error(void);

/* Library version string. */
const char* medusa_version(void);

/*
 * Workspace bytes that one call sequence of this shape needs (the largest
 * need of any call below, plus a counter block). Zero-fill a new workspace
 * once before its first use; every call leaves its counters at zero again,
 * so the same workspace may then serve any call of any shape that fits.
 */
size_t medusa_workspace_bytes(const medusa_shape* shape);

/*
 * Medusa heads ("Medusa 深读", §3.1, head equation; "Medusa Part I", Part 3,
 * ResidualBlock/MedusaHead):
 *   z_k    = h + SiLU(W1_k h + b1_k)          (fp32, not rounded)
 *   l_k    = W2_k z_k                          (fp32 accumulate)
 *   topk   = the s_max best tokens of l_k: higher logit first, lower id on ties
 *   lse_k  = log sum_v exp(l_k[v])
 * Head k (0-based) proposes depth k+1 of the tree.
 *
 *   h            [B][d] fp32
 *   W1           [K][d][d] elem;   b1_or_null [K][d] fp32 (NULL = no bias)
 *   W1_packed_or_null  W1 viewed as one [K d][d] matrix, packed by
 *                medusa_pack_weight (MEDUSA_PACK_PLAIN, rows = K d); NULL =
 *                none. Read instead of W1 by batches of 3 to 8 sequences in
 *                bf16; ignored otherwise.
 *   W2           [K][V][d] elem
 *   W2_packed_or_null  the K heads' W2_k each packed by medusa_pack_weight
 *                (MEDUSA_PACK_PLAIN, rows = V), head k at byte
 *                k * medusa_packed_weight_bytes(shape, V); NULL = none. Read
 *                instead of W2 by batches of 3 to 8 sequences in bf16 (their
 *                passes take 16 rows x 64 bytes per wave load from a row-major
 *                W2, 1 KB contiguous from the packed one); ignored otherwise.
 *   topk_ids     [B][K][s_max] int32   (out)
 *   topk_logits  [B][K][s_max] fp32    (out)
 *   head_lse     [B][K] fp32           (out, may be NULL)
 *   head_logits  [B][K][V] fp32        (out, may be NULL; needed to draft by sampling)
 *   z            [B][K][d] fp32        (out, may be NULL)
 */
int medusa_heads_forward(const medusa_shape* shape, const float* h, const void* W1,
                         const void* W1_packed_or_null, const float* b1_or_null,
                         const void* W2, const void* W2_packed_or_null, int32_t* topk_ids,
                         float* topk_logits, float* head_lse_or_null,
                         float* head_logits_or_null, float* z_or_null, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Calibrated sparse tree ("Medusa 深读", §6.2): from per-head rank
 * probabilities, choose the `budget` tree nodes (rank paths) that maximise
 * the expected accepted depth under the approximation that heads are
 * independent. A rank path (r_1 .. r_k) weighs w = prod_j a[j][r_j]; the
 * frontier starts with the depth-1 paths; `budget` times the frontier path
 * of largest weight (ties: the lexicographically smaller path, a prefix
 * first) joins the tree and its S children join the frontier. The expected
 * accepted depth is the sum of the chosen weights (tail-sum identity). Host
 * code only: no device memory, no stream, no GPU needed.
 *
 *   K, S                heads (1..MEDUSA_MAX_K) and ranks per head (1..MEDUSA_MAX_S)
 *   a_host              HOST [K][S] float64, a[k][i] = P(head k+1's true token
 *                       has 0-based rank i); finite and >= 0
 *   budget              nodes to choose, 0..MEDUSA_MAX_T-1 (fewer when the full
 *                       tree of sum_k S^k paths is smaller)
 *   tree_ranks_host     HOST [budget][K] int32 (out): the chosen paths in
 *                       canonical order (depth, then lexicographic), -1
 *                       padded, ready for medusa_build_tree / medusa_step
 *   weights_host_or_null     HOST [budget] float64 (out): w of each row
 *   pick_order_host_or_null  HOST [budget] int32 (out): row of the i-th pick
 *   n_nodes_host        HOST int32 (out): number of rows written
 * Returns MEDUSA_ERR_ARG for null pointers, negative sizes or a table entry
 * that is negative, infinite or NaN; MEDUSA_ERR_UNSUPPORTED beyond the limits.
 */
int medusa_sparse_tree(int K, int S, const double* a_host, int budget, int32_t* tree_ranks_host,
                       double* weights_host_or_null, int32_t* pick_order_host_or_null,
                       int32_t* n_nodes_host);

/*
 * Candidate tree ("Medusa 深读", §6.1; node-count equation): node 0 is the
 * root (the base LM head's token); node n >= 1 has rank path tree_ranks[n-1].
 *
 *   tree_ranks   HOST [N][K] int32, 0-based ranks, -1 padded. Must be
 *                prefix-closed and in canonical order (depth, then
 *                lexicographic); every rank < s_max. Validated on the host.
 *   draft_mode   MEDUSA_DRAFT_TOPK: tok(n) = topk_ids[depth-1][last rank];
 *                MEDUSA_DRAFT_SAMPLE: tok(n) = inverse-CDF draw from
 *                softmax(head_logits[depth-1]) with u_draft[b][n] (needs
 *                head_logits and head_lse).
 *   root_tok     [B] int32; kv_len [B] int32 (prefix lengths L_b)
 *   tree_tokens  [B][T] int32 (out)
 *   tree_mask    [T][T] uint8 (out): 1 iff column node is the row node or
 *                one of its ancestors
 *   position_ids [B][T] int32 (out): L_b + depth(n)
 *   retrieve     [P][K+1] int32 (out): node lists of root-to-leaf paths in
 *                lexicographic leaf order, -1 padded
 *   parent       [T] int32 (out, parent[0] = -1); depth [T] int32 (out)
 * tree_mask, retrieve, parent and depth depend only on tree_ranks: each may
 * be NULL to skip writing it (a decode loop writes them once per spec and
 * passes NULL afterwards); tree_tokens and position_ids are always written.
 */
int medusa_build_tree(const medusa_shape* shape, const int32_t* tree_ranks_host,
                      int draft_mode, const int32_t* root_tok, const int32_t* topk_ids,
                      const float* head_logits_or_null, const float* head_lse_or_null,
                      const float* u_draft_or_null, const int32_t* kv_len,
                      int32_t* tree_tokens, uint8_t* tree_mask, int32_t* position_ids,
                      int32_t* retrieve, int32_t* parent, int32_t* depth, void* stream);

/*
 * Tree attention ("Medusa: Faster LLM text generation", Tree attention;
 * "Medusa 深读", §6.1): for sequence b, head h and node i,
 *   o_i = softmax_j(scale * q_i . k_j) v_j
 * over the prefix rows j < kv_len[b] of the cache and the tree nodes j with
 * tree_mask[i][j] = 1.
 *
 *   q, k_tree, v_tree   [B][T][H][Dh] elem
 *   k_cache, v_cache    [B][H][Lmax][Dh] elem
 *   out                 [B][T][H][Dh] fp32 (out)
 */
int medusa_tree_attention(const medusa_shape* shape, const void* q, const void* k_tree,
                          const void* v_tree, const void* k_cache, const void* v_cache,
                          const int32_t* kv_len, const uint8_t* tree_mask, float scale,
                          float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Weight packing for the verification GEMMs (an MI355X layout, not a step of
 * the method). The verifier's projections read their weights as MFMA
 * operand tiles: tile (nt, kt) holds packed rows 16*nt .. 16*nt+15 and
 * columns c*kt .. c*kt+c-1 (c = 32 for bf16, 16 for fp32) of a row-major
 * [rows][d] matrix, stored as 64 consecutive 16-byte pieces, piece l =
 * packed row 16*nt + l%16, columns c*kt + (c/4)*(l/16) .. +c/4-1. Tile
 * (nt, kt) is stored at tile index kt*ntiles + nt (ntiles = ceil(rows/16)):
 * k-major, so the 16-row stripes that a launch streams side by side sit
 * next to each other. Packed rows past `rows` (up to the next multiple of 16)
 * are zero. The packed buffer is only meaningful to this library: produce
 * it with medusa_pack_weight in the process that uses it.
 * kind MEDUSA_PACK_PLAIN: packed row n is row n (W_o, W_lm).
 * kind MEDUSA_PACK_QKV (W_qkv, rows = 3d): within every block of Dh rows
 *   (one head of q, k or v) packed row 16*t + j is row 8*t + j for j < 8 and
 *   row Dh/2 + 8*t + j - 8 for j >= 8, so each tile holds 8 whole RoPE
 *   rotation pairs (i, i + Dh/2).
 *   W        [rows][d] elem, row-major (input, not modified)
 *   W_packed medusa_packed_weight_bytes(shape, rows) bytes, 16-byte aligned,
 *            not overlapping W (out)
 * Pack W_qkv, W_o and W_lm once, before the first medusa_verify_forward.
 * medusa_packed_weight_bytes returns 0 on an invalid shape or rows < 1.
 */
#define MEDUSA_PACK_PLAIN 0
#define MEDUSA_PACK_QKV 1
size_t medusa_packed_weight_bytes(const medusa_shape* shape, int rows);
int medusa_pack_weight(const medusa_shape* shape, int kind, const void* W, int rows,
                       void* W_packed, void* stream);

/*
 * Verification forward: one target layer over the T tree rows of every
 * sequence, then the verification LM head (the target scores the whole tree
 * in one pass, "Medusa: Faster LLM text generation", Tree attention). The
 * pages leave the target's internals open; this layer is
 *   x = E[tok];  q,k,v = RoPE(x Wq^T), RoPE(x Wk^T), x Wv^T  (theta = rope_theta,
 *   pairs (i, i+Dh/2), angle pos * theta^(-2i/Dh));  o = tree attention;
 *   y = x + o Wo^T;  l = y W_lm^T
 * with q, k, v, o and y rounded to elem before their next product.
 * Row statistics at temperature tau (for the posterior):
 *   row_stats[b][t] = { m = max_v l, S = sum_v e^{(l-m)/tau},
 *                       W = sum_v e^{(l-m)/tau} (l-m)/tau }
 *   (so p(x) = e^{(l_x-m)/tau}/S and H(p) = log S - W/S),
 *   row_argmax[b][t] = argmax_v l (lowest id on ties),
 *   child_logit[b][t] = l at row parent(t), column tree_tokens[b][t]
 *   (t >= 1; child_logit[b][0] = 0).
 *
 *   E [V][d] elem, row-major; W_qkv (3d rows: q, k, v blocks, packed with
 *   MEDUSA_PACK_QKV), W_o (d rows) and W_lm (V rows, both MEDUSA_PACK_PLAIN):
 *   elem, packed by medusa_pack_weight
 *   k_tree_out, v_tree_out [B][T][H][Dh] elem (out; rows to commit)
 *   y_out [B][T][d] fp32 (out); row_stats [B][T][3] fp32 (out);
 *   row_argmax [B][T] int32 (out); child_logit [B][T] fp32 (out);
 *   verify_logits_or_null [B][T][V] fp32 (out, optional; needed for exact mode)
 */
int medusa_verify_forward(const medusa_shape* shape, const void* E, const void* W_qkv,
                          const void* W_o, const void* W_lm, float rope_theta,
                          const int32_t* tree_tokens, const int32_t* position_ids,
                          const uint8_t* tree_mask, const int32_t* parent,
                          const void* k_cache, const void* v_cache, const int32_t* kv_len,
                          float temperature, void* k_tree_out, void* v_tree_out,
                          float* y_out, float* row_stats, int32_t* row_argmax,
                          float* child_logit, float* verify_logits_or_null,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Posterior and longest accepted prefix ("Medusa 深读", §5; "Medusa Part I",
 * Part 2; "Medusa: Faster LLM text generation", Acceptance rules).
 * The root is always accepted. A node is accepted iff its rule accepts it
 * and its parent is accepted. The committed node is the deepest accepted
 * node (lowest index among equals); a = its depth.
 *   GREEDY : tok(c) == row_argmax[parent(c)]
 *   TYPICAL: p > min(eps, delta*exp(-H)), p = e^{(child_logit-m)/tau}/S and
 *            H = log S - W/S from the parent's row_stats (strict >)
 *   EXACT  : children of an accepted node v are tried in index order with
 *            p = softmax(verify_logits[v]/tau), q = softmax(head_logits[depth(v)]);
 *            c is accepted iff u_accept[c]*q(tok) < p(tok), else p <- norm((p-q)+);
 *            with no child accepted (or v a leaf) next_root is an inverse-CDF
 *            draw from p with u_resample[v]. Needs verify_logits, head_logits,
 *            head_lse, u_accept, u_resample.
 * Outputs: accept_len [B] (= a), best_path [B] (first path through the
 * committed node), last_node [B], out_tokens [B][K+1] (root..committed
 * node, -1 padded), next_root [B] (argmax at the committed node for GREEDY
 * and TYPICAL; the residual or final draw for EXACT).
 */
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
                              void* stream);

/*
 * Commit ("Medusa: Faster LLM text generation", Introduction: the accepted
 * prefix becomes the next context): the K/V rows of the root..last_node path
 * go to cache rows kv_len[b] .. kv_len[b]+a, kv_len[b] += a+1, and
 * h_next[b] = y[b][last_node[b]] (the hidden state the next step's heads
 * read). A sequence whose kv_len + depth + 1 would pass Lmax is left
 * unchanged and its kv_len set to -1 (checked on the device).
 *   k_tree, v_tree [B][T][H][Dh] elem; y [B][T][d] fp32;
 *   k_cache, v_cache [B][H][Lmax][Dh] elem (in-out); kv_len [B] (in-out);
 *   h_next [B][d] fp32 (out)
 */
int medusa_commit(const medusa_shape* shape, const int32_t* last_node, const int32_t* parent,
                  const void* k_tree, const void* v_tree, const float* y, void* k_cache,
                  void* v_cache, int32_t* kv_len, float* h_next, void* stream);

/*
 * One whole verify step ("Medusa Part I", introduction: heads propose, the
 * tree is verified in one pass, the longest accepted prefix is committed;
 * the parts as above), all launches on one stream with no host
 * synchronisation, so a caller can capture it in a graph. It computes what
 * medusa_heads_forward, medusa_build_tree (tokens and positions only),
 * medusa_verify_forward, medusa_evaluate_posterior and medusa_commit compute
 * in that order, with the same arguments and results, except that:
 *  - tree_mask, parent and retrieve are inputs, written beforehand by one
 *    medusa_build_tree call for the same tree_ranks;
 *  - with MEDUSA_DRAFT_TOPK the head merge also writes tree_tokens and
 *    position_ids, and in greedy / typical mode one workgroup per sequence
 *    evaluates the posterior and commits.
 * Pointers are device memory unless marked; _or_null members may be NULL
 * where the corresponding call allows it. W_qkv, W_o and W_lm are packed
 * (medusa_pack_weight). Every part is validated before the first launch;
 * errors as for the individual calls (on an error nothing is launched).
 */
typedef struct {
  /* heads */
  const float* h;                  /* [B][d] */
  const void* W1;                  /* [K][d][d] elem */
  const float* b1_or_null;         /* [K][d] */
  const void* W2;                  /* [K][V][d] elem */
  /* tree */
  const int32_t* tree_ranks_host; /* HOST [N][K], see medusa_build_tree */
  int draft_mode;
  const int32_t* root_tok;         /* [B] */
  const float* u_draft_or_null;    /* [B][T] (MEDUSA_DRAFT_SAMPLE) */
  const uint8_t* tree_mask;        /* [T][T] (input) */
  const int32_t* parent;           /* [T] (input) */
  const int32_t* retrieve;         /* [P][K+1] (input) */
  /* verifier */
  const void* E;                   /* [V][d] elem */
  const void* W_qkv;               /* packed, MEDUSA_PACK_QKV */
  const void* W_o;                 /* packed */
  const void* W_lm;                /* packed */
  float rope_theta;
  void* k_cache;                   /* [B][H][Lmax][Dh] elem (in-out) */
  void* v_cache;
  int32_t* kv_len;                 /* [B] (in-out; only read when kv_len_out_or_null is set) */
  /* posterior */
  int mode;
  float temperature, eps, delta;
  const float* u_accept_or_null;   /* [B][T] (exact) */
  const float* u_resample_or_null; /* [B][T] (exact) */
  /* outputs */
  int32_t* topk_ids;               /* [B][K][s_max] */
  float* topk_logits;              /* [B][K][s_max] */
  float* head_lse_or_null;         /* [B][K] */
  float* head_logits_or_null;      /* [B][K][V] */
  float* z_or_null;                /* [B][K][d] */
  int32_t* tree_tokens;            /* [B][T] */
  int32_t* position_ids;           /* [B][T] */
  void* k_tree;                    /* [B][T][H][Dh] elem */
  void* v_tree;
  float* y;                        /* [B][T][d] */
  float* row_stats;                /* [B][T][3] */
  int32_t* row_argmax;             /* [B][T] */
  float* child_logit;              /* [B][T] */
  float* verify_logits_or_null;    /* [B][T][V] */
  int32_t* accept_len;             /* [B] */
  int32_t* best_path;              /* [B] */
  int32_t* last_node;              /* [B] */
  int32_t* out_tokens;             /* [B][K+1] */
  int32_t* next_root;              /* [B] */
  float* h_next;                   /* [B][d] */
  /* [B] or NULL: where the commit writes the advanced prefix lengths (kv_len
   * + a + 1, or -1). NULL advances kv_len in place, as medusa_commit does;
   * a separate buffer leaves kv_len unchanged, so that the same step can be
   * repeated over the same prefix (the appended cache rows are rewritten at
   * the same positions) without restoring kv_len in between. */
  int32_t* kv_len_out_or_null;
  /* heads: packed copies, as medusa_heads_forward's W2_packed_or_null and
   * W1_packed_or_null */
  const void* W2_packed_or_null;
  const void* W1_packed_or_null;
} medusa_step_args;

int medusa_step(const medusa_shape* shape, const medusa_step_args* args, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * medusa_step for timing tools: the same step, which also records the two
 * hipEvent_t handles ev_w2_start and ev_w2_end (both non-NULL, created by the
 * caller) on `stream` immediately before and after the vocabulary-projection
 * kernel (l_k = W2_k z_k with the fused top-s, "Medusa 深读", §3.1: the
 * step's dominant HBM stream), so that kernel can be timed alone inside a
 * running step loop. Keeps no state; results and errors as for medusa_step.
 */
int medusa_step_timed(const medusa_shape* shape, const medusa_step_args* args, void* workspace,
                      size_t workspace_bytes, void* stream, void* ev_w2_start, void* ev_w2_end);

/*
 * medusa_step for callers that cannot allocate device memory (code under
 * graph capture, serving loops or harnesses that forbid hipMalloc): the same
 * step with the same results, its workspace taken from a device array the
 * library owns, MEDUSA_STATIC_WORKSPACE_BYTES bytes on every GPU it runs on,
 * held until the process ends. The array of the calling thread's current
 * device is used; its address is looked up once per device. The call
 * allocates nothing; it clears the array's counter block with one small
 * kernel on `stream` before the step. Every call on one GPU shares that
 * GPU's array, so calls that overlap on one GPU (other streams, other
 * threads) race: serialise them. A shape whose medusa_workspace_bytes()
 * exceeds the array returns MEDUSA_ERR_WORKSPACE before anything runs;
 * other errors as for medusa_step.
 */
#define MEDUSA_STATIC_WORKSPACE_BYTES (64u << 20)
int medusa_step_static(const medusa_shape* shape, const medusa_step_args* args, void* stream);

/*
 * Decoding loop ("Medusa 深读", generate loop; "Medusa: Faster LLM text
 * generation", decoding with heads and tree attention): n_steps composite
 * steps back to back on one stream, each step's accepted prefix becoming the
 * next step's context with no host round trip, so the loop (or any number of
 * its steps) can be captured in one graph.
 *
 *   args             as for medusa_step, with the loop state in-out:
 *                    h [B][d] and root_tok [B] (the hidden state of the last
 *                    accepted token and the base model's next token) are read
 *                    by the first step and hold the state after the last one
 *                    on return; h_next and next_root are the loop's second
 *                    state buffer (overwritten); kv_len and the KV cache
 *                    advance in place (kv_len_out_or_null must be NULL);
 *                    out_tokens and accept_len are not used; the exact-mode
 *                    uniforms, when given, hold one [B][T] block per step,
 *                    step i's at element i * MEDUSA_ALIGN4(B * T) (so every
 *                    block keeps the 16-byte alignment of the first)
 *   n_steps          steps to run, >= 0
 *   out_tokens_steps int32 (out): step i's committed tokens (root, then the
 *                    accepted nodes), -1 padded, as a [B][K+1] block at
 *                    element i * MEDUSA_ALIGN4(B * (K+1))
 *   accept_len_steps int32 (out): step i's accepted depths a (the step
 *                    commits a + 1 tokens) as [B] at element i * MEDUSA_ALIGN4(B)
 *                    (the per-step blocks keep the 16-byte alignment)
 * The caller sizes the cache for kv_len + n_steps * (K + 1) rows. Every
 * step's arguments are validated before the first launch; errors as for
 * medusa_step (on an error nothing is launched).
 */
#define MEDUSA_ALIGN4(n) (((n) + 3) & ~3)
int medusa_generate(const medusa_shape* shape, const medusa_step_args* args, int n_steps,
                    int32_t* out_tokens_steps, int32_t* accept_len_steps, void* workspace,
                    size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MEDUSA_H */
