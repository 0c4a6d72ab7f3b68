// Candidate tree on gfx950 ("Medusa 深读", §6.1): topology, mask, position
// ids, root-to-leaf paths and node tokens.
//
// The host has validated the rank-path spec and reduced it to (parent, own
// rank, depth) per node. Per step, one thread per node writes
//   tokens     = the root token, or head (depth-1)'s token of the node's rank,
//   positions  = kv_len[b] + depth
// (in sampling mode the sampler's depth-1 workgroups write the positions
// and the root token, and the draws the other tokens).
// The topology, which only depends on the spec, is written when asked (once
// per spec is enough), by one workgroup with one thread per node (T <= 256):
//   mask[i][j] = 1 iff j is i or an ancestor of i,
//   paths      = the leaves in lexicographic rank-path order,
//   parent, depth.
// In sampling mode a second kernel draws each node's token from its depth's
// head softmax by inverse CDF.
#include "cdf.h"
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

__device__ __forceinline__ bool lex_less(const uint8_t* a, int da, const uint8_t* b, int db) {
  const int n = da < db ? da : db;
  for (int j = 0; j < n; ++j)
    if (a[j] != b[j]) return a[j] < b[j];
  return da < db;
}

__global__ __launch_bounds__(256) void tree_nodes_kernel(TreeArgs a) {
  const int b = blockIdx.x;
  const int n = threadIdx.x;
  const int T = a.plan.T, K = a.plan.K;
  if (n >= T) return;
  const int d = a.plan.depth[n];
  a.position_ids[(size_t)b * T + n] = a.kv_len[b] + d;
  int tok;
  if (n == 0)
    tok = a.root_tok[b];
  else
    tok = a.topk_ids[((size_t)b * K + (d - 1)) * a.S + a.plan.last_rank[n]];
  a.tokens[(size_t)b * T + n] = tok;
}

__global__ __launch_bounds__(256) void tree_topology_kernel(TreeArgs a) {
  const int n = threadIdx.x;
  const int T = a.plan.T, K = a.plan.K;
  __shared__ uint8_t par[MAXT], lrank[MAXT], dep[MAXT], has_child[MAXT];
  __shared__ uint8_t anc[MAXT][MAXK + 1];   // anc[n][k]: n's ancestor at depth k (k <= depth)
  __shared__ uint8_t tup[MAXT][MAXK];       // n's rank path
  if (n < T) {
    par[n] = a.plan.parent[n];
    lrank[n] = a.plan.last_rank[n];
    dep[n] = a.plan.depth[n];
    has_child[n] = 0;
  }
  __syncthreads();
  if (n < T) {
    const int d = dep[n];
    int x = n;
    anc[n][d] = (uint8_t)n;
    for (int j = d - 1; j >= 0; --j) {
      tup[n][j] = lrank[x];
      x = par[x];
      anc[n][j] = (uint8_t)x;
    }
    if (n >= 1) has_child[par[n]] = 1;
  }
  __syncthreads();
  const int d = n < T ? dep[n] : 0;
  // mask[i][j] = j is i or an ancestor of i, written cooperatively
  if (a.mask)
    for (int e = n; e < T * T; e += blockDim.x) {
      const int i = e / T, j = e - i * T;
      a.mask[e] = (dep[j] <= dep[i] && anc[i][dep[j]] == j) ? 1 : 0;
    }
  if (n >= T) return;
  if (a.parent) a.parent[n] = n == 0 ? -1 : (int)par[n];
  if (a.depth) a.depth[n] = d;
  const bool leaf = T == 1 ? true : (n >= 1 && !has_child[n]);
  if (!leaf || !a.retrieve) return;
  int p = 0;
  for (int m = 1; m < T; ++m)
    if (m != n && !has_child[m] && lex_less(tup[m], dep[m], tup[n], d)) ++p;
  int32_t* r = a.retrieve + (size_t)p * (K + 1);
  for (int j = 0; j <= d; ++j) r[j] = anc[n][j];
  for (int j = d + 1; j <= K; ++j) r[j] = -1;
}

// Inverse-CDF draws for sampling mode. One 1024-thread workgroup per
// (depth k, sequence b) builds the CDF of head k's softmax weights
// w_v = exp(l_v - lse) (cdf.h); thread n then draws node n's token with the
// node's uniform if node n has depth k + 1 (T <= 256 threads). The
// workgroups of depth 1 also write what the node kernel writes in top-s mode
// for every node: the position ids, and the root token.
__global__ __launch_bounds__(kCdfThreads) void tree_sample_kernel(TreeArgs a) {
  const int kd = blockIdx.x;     // 0-based head = depth - 1
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int T = a.plan.T, K = a.plan.K, V = a.V;
  const float* l = a.head_logits + ((size_t)b * K + kd) * V;
  const float lse = a.head_lse[(size_t)b * K + kd];
  __shared__ CdfLds sh;
  const ExpRow w{l, lse, V};
  const int dep = a.plan.depth[min(t, MAXT - 1)];
  const bool mine = t >= 1 && t < T && dep == kd + 1;
  const float u = mine ? a.u_draft[(size_t)b * T + t] : 0.f;
  if (kd == 0 && t < T) {
    a.position_ids[(size_t)b * T + t] = a.kv_len[b] + dep;
    if (t == 0) a.tokens[(size_t)b * T] = a.root_tok[b];
  }
  cdf_build<true>(w, V, sh);
  if (mine) a.tokens[(size_t)b * T + t] = cdf_draw(w, V, u, sh);
}

}  // namespace

hipError_t launch_tree(const TreeArgs& a, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (!a.sample) {
    hipLaunchKernelGGL(tree_nodes_kernel, dim3(a.B), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.mask || a.retrieve || a.parent || a.depth) {
    hipLaunchKernelGGL(tree_topology_kernel, dim3(1), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!a.sample) return e;
  hipLaunchKernelGGL(tree_sample_kernel, dim3(a.plan.K, a.B), dim3(kCdfThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace medusa
