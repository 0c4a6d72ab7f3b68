// Posterior evaluation, longest accepted prefix and commit on gfx950.
//
// Rules ("Medusa 深读", §5, acceptance equation and rule table; "Medusa Part
// I", Part 2; "Medusa: Faster LLM text generation", Acceptance rules):
//   greedy : child c accepted iff tok(c) == argmax of its parent's logits;
//   typical: p(tok(c)) > min(eps, delta * exp(-H)) with p, H of the parent's
//            tempered distribution, from its row statistics
//            (p = e^{(l-m)/tau}/S, H = log S - W/S);
//   exact  : children of an accepted node are tried in order, accepted iff
//            u*q(x) < p(x), else p <- norm((p - q)+); with no child accepted
//            (or at a leaf) the next root is an inverse-CDF draw from p.
// The root is always accepted; a node needs its parent accepted; the
// committed node is the deepest accepted node with the lowest index.
//
// Greedy/typical: one workgroup per sequence, one thread per node; the
// accepted-prefix flags are ANDed along each node's ancestor chain and the
// (depth, -index) maximum is found with DPP wave reductions.
// Exact: every node's p/q steps in a workgroup of its own (vocabularies up
// to 32768, held in LDS), then a walk over the nodes' decisions; larger
// vocabularies: one 1024-thread workgroup per sequence walks the tree, each
// p/q step a block-wide pass over the vocabulary in global memory.
#include <algorithm>
#include <type_traits>

#include "cdf.h"
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Parent of node x, clamped into [0, T); walks below stop after K steps, so
// a malformed parent array can neither fault nor loop.
__device__ __forceinline__ int parent_of(const int32_t* parent, int x, int T) {
  return min(max(parent[x], 0), T - 1);
}

__device__ __forceinline__ int wave_max_i(int v) {
  v = max(v, dppi<kDppQuadXor1>(v));
  v = max(v, dppi<kDppQuadXor2>(v));
  v = max(v, dppi<kDppRowRor4>(v));
  v = max(v, dppi<kDppRowRor8>(v));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Statistics of one verify row: max, S, W at temperature tau, argmax.
struct RowStat {
  float m, S, W;
  int am;
};

// A sequence's tree in LDS: clamped parents, node tokens, row statistics,
// acceptance flags and the decisions taken from them. Every walk along the
// ancestor chain reads these, never global memory.
struct TreeLds {
  int parent[MAXT];
  int tok[MAXT];
  RowStat stat[MAXT];
  uint8_t acc[MAXT];
  int wmax[16];
  int best, depth, bp, L;
  int path[MAXK + 1];
};

// Greedy / typical posterior of sequence b over the workgroup (blockDim.x >=
// T, a multiple of 64, at most 1024) from sh.parent, sh.tok, sh.stat and
// thread c's child logit cl: thread 0 writes accept_len, last_node,
// out_tokens and next_root (when `publish`); on return every thread sees
// sh.best, sh.depth.
__device__ void posterior_det_lds(const PostArgs& a, int b, float cl, TreeLds& sh,
                                  bool publish = true) {
  const int c = threadIdx.x;
  const int T = a.T;
  if (c < T) {
    bool ok = true;
    if (c > 0) {
      const RowStat ps = sh.stat[sh.parent[c]];
      if (a.mode == 0) {
        ok = sh.tok[c] == ps.am;
      } else {
        const float p = exp_e((cl - ps.m) * a.inv_tau) / ps.S;
        const float H = __logf(ps.S) - ps.W / ps.S;
        const float thr = fminf(a.eps, a.delta * exp_e(-H));
        ok = p > thr;
      }
    }
    sh.acc[c] = ok;
  }
  __syncthreads();
  int key = -1;
  int dep = 0;
  if (c < T) {
    bool ok = true;
    for (int x = c; x != 0 && dep < a.K; x = sh.parent[x]) {
      ok = ok && sh.acc[x];
      ++dep;
    }
    if (ok) key = (dep << 16) | (0xffff - c);
  }
  key = wave_max_i(key);
  const int nw = blockDim.x >> 6;
  if ((c & 63) == 0) sh.wmax[c >> 6] = key;
  __syncthreads();
  if (c == 0) {
    key = sh.wmax[0];
    for (int w = 1; w < nw; ++w) key = max(key, sh.wmax[w]);
    const int best = 0xffff - (key & 0xffff);
    const int depth = key >> 16;
    if (publish) {
      a.accept_len[b] = depth;
      a.last_node[b] = best;
      int* out = a.out_tokens + (size_t)b * (a.K + 1);
      for (int j = depth + 1; j <= a.K; ++j) out[j] = -1;
      int x = best;
      for (int j = depth; j >= 0; --j) {
        out[j] = sh.tok[x];
        x = sh.parent[x];
      }
      a.next_root[b] = sh.stat[best].am;
    }
    sh.best = best;
    sh.depth = depth;
    sh.bp = 0x7fffffff;
  }
  __syncthreads();
}

// Path rows of retrieve for thread c < P (entries 0..K), loaded up front.
__device__ __forceinline__ void load_path_row(const PostArgs& a, int (&ret)[MAXK + 1]) {
  const int c = threadIdx.x;
#pragma unroll
  for (int j = 0; j <= MAXK; ++j)
    ret[j] = (c < a.P && j <= a.K) ? a.retrieve[(size_t)c * (a.K + 1) + j] : -1;
}

// best_path: the lowest path index whose node at the committed depth is the
// committed node (0 if none; an LDS minimum over threads c < P).
__device__ void best_path_lds(const PostArgs& a, int b, const int (&ret)[MAXK + 1],
                              TreeLds& sh, bool publish = true) {
  const int c = threadIdx.x;
  int r = -1;
#pragma unroll
  for (int j = 0; j <= MAXK; ++j)
    if (j == sh.depth) r = ret[j];
  if (c < a.P && r == sh.best) atomicMin(&sh.bp, c);
  __syncthreads();
  if (c == 0 && publish) a.best_path[b] = sh.bp < a.P ? sh.bp : 0;
}

// Tree data of sequence b into LDS (threads c < T), from values the caller
// loaded into registers before (so that their loads fly with others).
__device__ __forceinline__ void stage_tree(int T, int par, int tk, TreeLds& sh) {
  const int c = threadIdx.x;
  if (c < T) {
    sh.parent[c] = min(max(par, 0), T - 1);
    sh.tok[c] = tk;
  }
}

__global__ __launch_bounds__(256) void posterior_kernel(PostArgs a) {
  const int b = blockIdx.x, c = threadIdx.x, T = a.T;
  __shared__ TreeLds sh;
  int par = 0, tk = 0;
  float cl = 0.f;
  RowStat st{0.f, 1.f, 0.f, 0};
  if (c < T) {
    const size_t r = (size_t)b * T + c;
    par = a.parent[c];
    tk = a.tokens[r];
    cl = a.child_logit[r];
    st = RowStat{a.row_stats[r * 3 + 0], a.row_stats[r * 3 + 1], a.row_stats[r * 3 + 2],
                 a.row_argmax[r]};
  }
  int ret[MAXK + 1];
  load_path_row(a, ret);
  stage_tree(T, par, tk, sh);
  if (c < T) sh.stat[c] = st;
  __syncthreads();
  posterior_det_lds(a, b, cl, sh);
  best_path_lds(a, b, ret, sh);
}

// ---- exact mode ----------------------------------------------------------------
// Block-wide helpers over a 1024-thread workgroup.
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += red[i];
  return s;
}
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = kNegInf;
  for (int i = 0; i < 16; ++i) s = fmaxf(s, red[i]);
  return s;
}

// Exact mode for any vocabulary: the target distribution lives in the
// workspace row pw and every pass is a block-wide loop over it.
__global__ __launch_bounds__(1024) void posterior_exact_kernel(PostArgs a) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int T = a.T, V = a.V, K = a.K;
  __shared__ float red[16];
  __shared__ CdfLds cdf;
  __shared__ int sh_taken, sh_next;
  float* pw = a.pw + (size_t)b * V;   // current target distribution p
  const int* tok = a.tokens + (size_t)b * T;
  const float* ur = a.u_resample + (size_t)b * T;
  const float* ua = a.u_accept + (size_t)b * T;

  // p = softmax(l_v / tau) into pw
  auto load_p = [&](int v) {
    const float* l = a.verify_logits + ((size_t)b * T + v) * V;
    float mx = kNegInf;
    for (int x = t; x < V; x += 1024) mx = fmaxf(mx, l[x] * a.inv_tau);
    mx = block_max(mx, red);
    float s = 0.f;
    for (int x = t; x < V; x += 1024) {
      const float e = exp_e(l[x] * a.inv_tau - mx);
      pw[x] = e;
      s += e;
    }
    s = block_sum(s, red);
    const float inv = 1.f / s;
    for (int x = t; x < V; x += 1024) pw[x] *= inv;
    __syncthreads();
  };

  int v = 0;
  int next = -1;
  load_p(0);
  while (true) {
    const int dv = [&] {
      int d = 0;
      for (int x = v; x != 0 && d < K; x = parent_of(a.parent, x, T)) ++d;
      return d;
    }();
    int taken = -1;
    bool has_kids = false;
    if (dv < K) {
      const float* hl = a.head_logits + ((size_t)b * K + dv) * V;
      const float lse = a.head_lse[(size_t)b * K + dv];
      for (int c = v + 1; c < T; ++c) {
        if (a.parent[c] != v) continue;
        has_kids = true;
        const int x = min(max(tok[c], 0), V - 1);
        const float qx = exp_e(hl[x] - lse);
        if (t == 0) sh_taken = (ua[c] * qx < pw[x]) ? 1 : 0;
        __syncthreads();
        const int acc = sh_taken;
        __syncthreads();
        if (acc) {
          taken = c;
          break;
        }
        // residual p <- norm(max(0, p - q)); kept when all zero
        float s = 0.f;
        for (int y = t; y < V; y += 1024) s += fmaxf(pw[y] - exp_e(hl[y] - lse), 0.f);
        s = block_sum(s, red);
        if (s > 0.f) {
          const float inv = 1.f / s;
          for (int y = t; y < V; y += 1024) pw[y] = fmaxf(pw[y] - exp_e(hl[y] - lse), 0.f) * inv;
        }
        __syncthreads();
      }
    }
    if (taken < 0) {
      const ScaledRow w{pw, 1.f, V};   // x 1 is exact
      cdf_build<true>(w, V, cdf);
      if (t == 0) sh_next = cdf_draw(w, V, ur[v], cdf);
      __syncthreads();
      next = sh_next;
      break;
    }
    v = taken;
    load_p(v);
  }
  if (t != 0) return;
  int depth = 0;
  for (int x = v; x != 0 && depth < K; x = parent_of(a.parent, x, T)) ++depth;
  a.accept_len[b] = depth;
  a.last_node[b] = v;
  int* out = a.out_tokens + (size_t)b * (K + 1);
  for (int j = depth + 1; j <= K; ++j) out[j] = -1;
  int x = v;
  for (int j = depth; j >= 0; --j) {
    out[j] = tok[x];
    x = parent_of(a.parent, x, T);
  }
  a.next_root[b] = next;
  int bp = 0;
  for (int p = 0; p < a.P; ++p)
    if (a.retrieve[(size_t)p * (K + 1) + depth] == v) {
      bp = p;
      break;
    }
  a.best_path[b] = bp;
}

// Exact mode for V <= kExactLdsV, node-parallel. The walk's work at a node v
// depends only on v's own verify row and its depth's drafting distribution:
// p_v, the acceptance tests of v's children in order with the residual
// update after each rejection, and -- when no child is accepted, or v has
// none -- the draw from the final residual. So one workgroup per (node,
// sequence) does exactly that for every node at once (exact_node_kernel,
// writing (first accepted child or -1, draw) per node), and a small kernel
// follows the accepted children from the root (exact_walk_kernel). Nodes the
// walk never reaches cost only idle compute units.
//
// In a node's workgroup thread t holds the 32 consecutive tokens 32t ..
// 32t + 31 in registers: the target as unnormalised weights p_i with one
// scale factor (p(x) = p_i * scale) and the drafting distribution q_i =
// e^(head logit - lse). Memory is read once, the verify row and the head
// row; every later pass -- the residual's sum, its update (kept when the
// residual is all zero), the CDF's chunk sums (chunks of 8 or 16 consecutive
// tokens, inside one thread) -- runs on registers. An acceptance test reads
// p(x) and q(x) from the thread that holds x, through LDS.
constexpr int kExactLdsV = 32768;
constexpr int kExactPer = kExactLdsV / 1024;   // tokens per thread

// Row values of tokens 32t .. 32t + 31 (clamped indices, so every load is in
// flight before the first is used; values past V are never used).
__device__ __forceinline__ void load_row32(const float* __restrict__ row, int V,
                                           float (&out)[kExactPer]) {
  const int x0 = kExactPer * threadIdx.x;
  if ((V & 3) == 0) {
#pragma unroll
    for (int j = 0; j < kExactPer / 4; ++j) {
      const floatx4_t v =
          *reinterpret_cast<const floatx4_t*>(row + max(min(x0 + 4 * j, V - 4), 0));
#pragma unroll
      for (int i = 0; i < 4; ++i) out[4 * j + i] = v[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kExactPer; ++i) out[i] = row[min(x0 + i, V - 1)];
  }
}

// Rows of V % 4 == 0 tokens, read coalesced: thread T loads float4s
// T + 1024 i of the row (clamped into it, as load_row32 does) into its
// registers r[4 i .. 4 i + 3], and unstage_row32 passes them through LDS
// (float4 column j of thread t's 32 tokens at column j ^ ((t >> 1) & 7),
// which keeps the writes of 16 consecutive threads and the reads of their
// own tokens free of bank conflicts) into the layout of load_row32: thread
// t holds tokens 32 t .. 32 t + 31, in the same registers.
__device__ __forceinline__ void stage_row32(const float* __restrict__ row, int V,
                                            float (&r)[kExactPer]) {
#pragma unroll
  for (int i = 0; i < kExactPer / 4; ++i) {
    const int f = threadIdx.x + 1024 * i;
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(row + max(min(4 * f, V - 4), 0));
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * i + e] = v[e];
  }
}
// Every thread calls it; `buf` (kExactLdsV floats) is free on entry and may
// be written again after a barrier that follows the call.
__device__ __forceinline__ void unstage_row32(float (&r)[kExactPer], floatx4_t* buf) {
  static_assert(kExactPer == 32, "eight float4 columns a thread");
#pragma unroll
  for (int i = 0; i < kExactPer / 4; ++i) {
    const int f = threadIdx.x + 1024 * i, tt = f >> 3, j = f & 7;
    buf[8 * tt + (j ^ ((tt >> 1) & 7))] =
        floatx4_t{r[4 * i], r[4 * i + 1], r[4 * i + 2], r[4 * i + 3]};
  }
  __syncthreads();
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kExactPer / 4; ++j) {
    const floatx4_t v = buf[8 * t + (j ^ ((t >> 1) & 7))];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * j + e] = v[e];
  }
}

// Register i of an array, for a runtime i the same in the whole wave
// (selects, no indexed register access).
__device__ __forceinline__ float pick32(const float (&r)[kExactPer], int i) {
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < kExactPer; ++j) v = j == i ? r[j] : v;
  return v;
}

__global__ __launch_bounds__(1024) void exact_node_kernel(PostArgs a) {
  if (blockIdx.x >= a.T) {
    // workgroups past the nodes (composite step): the row-statistics merge
    // of the LM head's records, 4 rows a workgroup, beside the nodes' work
    __shared__ floatx4_t wr[4][4];
    const int grp = threadIdx.x >> 8, n = 4 * (blockIdx.x - a.T) + grp;
    row_records_merge(a.lm_part, a.lm_G, a.inv_tau, blockIdx.y * a.T + min(n, a.T - 1),
                      threadIdx.x & 255, n < a.T, wr[grp], a.row_stats_out, a.row_argmax_out);
    return;
  }
  const int v = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int T = a.T, V = a.V, K = a.K;
  const int x0 = kExactPer * t;
  __shared__ float red[16];
  __shared__ CdfLds cdf;
  __shared__ int s_par[MAXT], s_tok[MAXT];
  __shared__ float s_ua[MAXT];
  __shared__ float s_pq[2];
  __shared__ int s_next;
  // the rows (V % 4 == 0) are read coalesced and handed out through LDS
  __shared__ floatx4_t rowbuf[kExactLdsV / 4];
  const bool coalesced = (V & 3) == 0;
  float p[kExactPer], q[kExactPer];
  const float* prow = a.verify_logits + ((size_t)b * T + v) * V;
  if (coalesced)
    stage_row32(prow, V, p);
  else
    load_row32(prow, V, p);
  if (t < T) {
    s_par[t] = a.parent[t];
    s_tok[t] = a.tokens[(size_t)b * T + t];
    s_ua[t] = a.u_accept[(size_t)b * T + t];
  }
  if (t == 0) cdf.last_nz = -1;
  __syncthreads();
  int dv = 0;
  for (int x = v; x != 0 && dv < K; x = min(max(s_par[x], 0), T - 1)) ++dv;
  const bool kids = dv < K;
  const float* hl = a.head_logits + ((size_t)b * K + min(dv, K - 1)) * V;
  if (coalesced) {
    if (kids) stage_row32(hl, V, q);   // in flight while p is handed out
    unstage_row32(p, rowbuf);
    if (kids) {
      __syncthreads();   // every thread has its p
      unstage_row32(q, rowbuf);
    }
  } else if (kids) {
    load_row32(hl, V, q);   // in flight during the softmax below
  }
  // p = softmax(l_v / tau): unnormalised weights and their scale
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < kExactPer; ++i) {
    p[i] = p[i] * a.inv_tau;
    if (x0 + i < V) mx = fmaxf(mx, p[i]);
  }
  mx = block_max(mx, red);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kExactPer; ++i) {
    p[i] = x0 + i < V ? exp_e(p[i] - mx) : 0.f;
    s += p[i];
  }
  s = block_sum(s, red);
  float scale = 1.f / s;

  int taken = -1;
  if (kids) {
    const float lse = a.head_lse[(size_t)b * K + dv];
#pragma unroll
    for (int i = 0; i < kExactPer; ++i) q[i] = x0 + i < V ? exp_e(q[i] - lse) : 0.f;
    for (int c = v + 1; c < T; ++c) {
      if (s_par[c] != v) continue;
      const int x = min(max(s_tok[c], 0), V - 1);
      if (t == x / kExactPer) {
        s_pq[0] = pick32(p, x % kExactPer) * scale;
        s_pq[1] = pick32(q, x % kExactPer);
      }
      __syncthreads();
      // every thread takes the same decision from the same values
      if (s_ua[c] * s_pq[1] < s_pq[0]) {
        taken = c;
        break;
      }
      // residual p <- norm(max(0, p - q)); kept when all zero
      float rs = 0.f;
#pragma unroll
      for (int i = 0; i < kExactPer; ++i) rs += fmaxf(p[i] * scale - q[i], 0.f);
      rs = block_sum(rs, red);   // also orders this child's s_pq reads before the next write
      if (rs > 0.f) {
#pragma unroll
        for (int i = 0; i < kExactPer; ++i) p[i] = fmaxf(p[i] * scale - q[i], 0.f);
        scale = 1.f / rs;
      }
    }
  }
  if (taken < 0) {
    // the CDF of p * scale: this thread's chunks, each summed in token order
    const int csz = cdf_chunk_size(V);
    const int nch = (V + csz - 1) / csz;
    int my_last = -1;
    float w[kExactPer];
#pragma unroll
    for (int i = 0; i < kExactPer; ++i) {
      w[i] = p[i] * scale;
      if (w[i] > 0.f) my_last = x0 + i;
    }
    // (csz is 8 or 16: both shapes unrolled, so every register index is fixed)
    const auto chunk_sums = [&](auto csz_c) {
      constexpr int CS = decltype(csz_c)::value;
#pragma unroll
      for (int c0 = 0; c0 < kExactPer; c0 += CS) {
        float cs = 0.f;
#pragma unroll
        for (int i = 0; i < CS; ++i) cs += w[c0 + i];
        const int c = (x0 + c0) / CS;
        if (c < nch) cdf.cs[c] = cs;
      }
    };
    if (csz == 8)
      chunk_sums(std::integral_constant<int, 8>{});
    else
      chunk_sums(std::integral_constant<int, 16>{});
    cdf_prefix(my_last, nch, csz, cdf);
    float target, eg, fc;
    const int c = cdf_locate(a.u_resample[(size_t)b * T + v], cdf, target, eg, fc);
    if (t == 0) s_next = -1;
    __syncthreads();
    if (c >= 0 && t == c * csz / kExactPer) {
      const int i0 = c * csz - x0;
      float local = 0.f;
      int x = -1;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (i < csz) {
          local += pick32(w, i0 + i);
          if (x < 0 && eg + (fc + local) > target) x = c * csz + i;
        }
      s_next = x;
    }
    __syncthreads();
  }
  if (t == 0) {
    int next = -1;
    if (taken < 0) {
      next = s_next;
      if (next < 0 || next > cdf.last_nz) next = cdf.last_nz < 0 ? V - 1 : cdf.last_nz;
    }
    *reinterpret_cast<int2*>(a.exact_dec + ((size_t)b * T + v) * 2) = make_int2(taken, next);
  }
}

// The walk over the nodes' decisions, one wave per sequence: from the root
// along the accepted children; the next root is the draw of the node where
// it stops.
__global__ __launch_bounds__(64) void exact_walk_kernel(PostArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int T = a.T, K = a.K;
  __shared__ int s_par[MAXT], s_tok[MAXT], s_taken[MAXT], s_draw[MAXT];
  __shared__ int s_v;
  for (int x = lane; x < T; x += 64) {
    const int2 dec = *reinterpret_cast<const int2*>(a.exact_dec + ((size_t)b * T + x) * 2);
    s_par[x] = min(max(a.parent[x], 0), T - 1);
    s_tok[x] = a.tokens[(size_t)b * T + x];
    s_taken[x] = dec.x;
    s_draw[x] = dec.y;
  }
  __syncthreads();
  const auto par = [&](int x) { return s_par[x]; };
  if (lane == 0) {
    int v = 0;
    // a taken child is a later node, so the walk ends within T steps
    for (int i = 0; i < T; ++i) {
      const int c = s_taken[v];
      if (c <= v || c >= T) break;
      v = c;
    }
    s_v = v;
  }
  __syncthreads();
  const int v = s_v;
  int depth = 0;
  for (int x = v; x != 0 && depth < K; x = par(x)) ++depth;
  // best path: the lowest path index whose node at this depth is v
  int bp = 0x7fffffff;
  for (int q = lane; q < a.P; q += 64)
    if (a.retrieve[(size_t)q * (K + 1) + depth] == v) bp = min(bp, q);
  bp = -wave_max_i(-bp);
  if (lane != 0) return;
  a.accept_len[b] = depth;
  a.last_node[b] = v;
  int* out = a.out_tokens + (size_t)b * (K + 1);
  for (int j = depth + 1; j <= K; ++j) out[j] = -1;
  int x = v;
  for (int j = depth; j >= 0; --j) {
    out[j] = s_tok[x];
    x = par(x);
  }
  a.next_root[b] = s_draw[v];
  a.best_path[b] = bp == 0x7fffffff ? 0 : bp;
}

// The LDS kernel needs more LDS than older parts give one workgroup; it runs
// where the device's per-workgroup limit holds it.
bool exact_lds_fits() {
  static const bool v = [] {
    int dev = 0, lim = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(exact_node_kernel)) !=
            hipSuccess)
      return false;
    return fa.sharedSizeBytes <= (size_t)lim;
  }();
  return v;
}

// ---- commit ----------------------------------------------------------------------
// One or more workgroups per sequence; the path's K/V rows are copied as
// 16-byte vectors (a node's row [H][Dh] is contiguous in the tree buffers, a
// head's row Dh is contiguous in the cache), together with the committed
// node's output row (h_next), every thread loading all its vectors (up to
// kCopyBatch) before it stores any, so the copy costs one round trip to
// memory.
constexpr int kCopyBatch = 4;

// Commit of sequence b's accepted path ending at node `last`, prefix length
// L, by workgroup `part` of `nparts` (each takes every nparts-th block of the
// vectors); sh.parent holds the tree. Thread 0 writes the advanced length
// when `write_len` (with several workgroups: the one that every other has
// read L before, so that an in-place update races with no read).
template <class ET>
__device__ void commit_lds(const CommitArgs& a, int b, int last_in, int L, TreeLds& sh,
                           int part = 0, int nparts = 1, bool write_len = true) {
  constexpr int PV = ET::kPerVec;
  const int T = a.T, H = a.H, Dh = a.Dh;
  if (threadIdx.x == 0) {
    const int last = min(max(last_in, 0), T - 1);
    int d = 0;
    for (int x = last; x != 0 && d < a.K; x = sh.parent[x]) ++d;
    int x = last;
    for (int j = d; j >= 0; --j) {
      sh.path[j] = x;
      x = sh.parent[x];
    }
    sh.depth = d;
  }
  __syncthreads();
  const int d = sh.depth;
  const bool room = L >= 0 && L + d + 1 <= a.Lmax;
  const u32x4_t* y = reinterpret_cast<const u32x4_t*>(a.y + ((size_t)b * T + sh.path[d]) * a.d);
  u32x4_t* hn = reinterpret_cast<u32x4_t*>(a.h_next + (size_t)b * a.d);
  const int vec_row = H * Dh / PV;          // 16-byte vectors per node row
  const int vec_head = Dh / PV;             // per head
  const int ny = a.d / 4;                   // vectors of the h_next row
  const int total = ny + (room ? (d + 1) * vec_row : 0);   // h_next, then K/V pairs
  const u32x4_t* kt = reinterpret_cast<const u32x4_t*>(a.k_tree);
  const u32x4_t* vt = reinterpret_cast<const u32x4_t*>(a.v_tree);
  u32x4_t* kc = reinterpret_cast<u32x4_t*>(a.k_cache);
  u32x4_t* vc = reinterpret_cast<u32x4_t*>(a.v_cache);
  const int stride = nparts * (int)blockDim.x;
  for (int e0 = part * (int)blockDim.x + (int)threadIdx.x; e0 < total;
       e0 += kCopyBatch * stride) {
    u32x4_t kv[kCopyBatch], vv[kCopyBatch];
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int e = min(e0 + u * stride, total - 1);
      if (e < ny) {
        kv[u] = y[e];
      } else {
        const int i = (e - ny) / vec_row, rem = (e - ny) - i * vec_row;
        const size_t src = ((size_t)b * T + sh.path[i]) * vec_row + rem;
        kv[u] = kt[src];
        vv[u] = vt[src];
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyBatch; ++u) {
      const int e = e0 + u * stride;
      if (e >= total) break;
      if (e < ny) {
        hn[e] = kv[u];
      } else {
        const int i = (e - ny) / vec_row, rem = (e - ny) - i * vec_row;
        const int hh = rem / vec_head, x = rem - hh * vec_head;
        const size_t dst = (((size_t)b * H + hh) * a.Lmax + L + i) * vec_head + x;
        kc[dst] = kv[u];
        vc[dst] = vv[u];
      }
    }
  }
  if (write_len && threadIdx.x == 0)
    (a.kv_len_out ? a.kv_len_out : a.kv_len)[b] = room ? L + d + 1 : -1;
}

template <class ET>
__global__ __launch_bounds__(1024) void commit_kernel(CommitArgs a) {
  const int b = blockIdx.x, c = threadIdx.x;
  __shared__ TreeLds sh;
  const int par = c < a.T ? a.parent[c] : 0;
  if (c == 0) sh.L = a.kv_len[b];
  const int last = a.last_node[b];
  stage_tree(a.T, par, 0, sh);
  __syncthreads();
  commit_lds<ET>(a, b, last, sh.L, sh);
}

// Composite step, greedy / typical: gridDim.x workgroups per sequence
// (blockIdx.y) each evaluate the posterior from the merged row statistics
// -- the same inputs and operations, so the same decision -- and copy their
// share of the accepted path; the first publishes the decision. All the
// loads the decision needs -- row statistics, child logits, tokens,
// parents, path rows, the prefix length -- are issued before any is used.
constexpr int kPostThreads = 256;
static_assert(kPostThreads >= MAXT, "one thread per tree row");
template <class ET>
__global__ __launch_bounds__(kPostThreads) void posterior_commit_kernel(PostArgs a, CommitArgs c) {
  const int b = blockIdx.y, t = threadIdx.x, T = a.T;
  __shared__ TreeLds sh;
  int par = 0, tk = 0;
  float cl = 0.f;
  if (t < T) {
    const size_t r = (size_t)b * T + t;
    par = a.parent[t];
    tk = a.tokens[r];
    cl = a.child_logit[r];
  }
  int ret[MAXK + 1];
  load_path_row(a, ret);
  int L = 0;
  if (t == 0) L = c.kv_len[b];
  if (t < T) {
    const size_t r = (size_t)b * T + t;
    sh.stat[t] = RowStat{a.row_stats[r * 3 + 0], a.row_stats[r * 3 + 1],
                         a.row_stats[r * 3 + 2], a.row_argmax[r]};
  }
  // Workgroups of several count themselves in on c.counters[b] once their
  // read of the prefix length is complete (every load of the wave waited
  // for); the last to count writes the advanced length and leaves the
  // counter at zero. The count is not waited for until the end.
  int before = 0;
  if (t == 0) {
    sh.L = L;
    if (gridDim.x > 1) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      vmcnt<0>();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      before = __hip_atomic_fetch_add(c.counters + b, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  stage_tree(T, par, tk, sh);
  __syncthreads();
  const bool publish = blockIdx.x == 0;
  posterior_det_lds(a, b, cl, sh, publish);
  best_path_lds(a, b, ret, sh, publish);
  const bool last = (int)gridDim.x == 1 || before == (int)gridDim.x - 1;
  commit_lds<ET>(c, b, sh.best, sh.L, sh, blockIdx.x, gridDim.x, last);
  if (t == 0 && gridDim.x > 1 && last) coherent_store(c.counters + b, 0);
}

// Composite step, exact mode, after exact_node_kernel: gridDim.x workgroups
// per sequence (blockIdx.y) each follow the accepted children from the root,
// as exact_walk_kernel does, and copy their share of the accepted path; the
// first publishes the decision. The prefix length is counted in and written
// as in posterior_commit_kernel.
template <class ET>
__global__ __launch_bounds__(kPostThreads) void exact_walk_commit_kernel(PostArgs a,
                                                                         CommitArgs c) {
  const int b = blockIdx.y, t = threadIdx.x, T = a.T, K = a.K;
  __shared__ TreeLds sh;
  __shared__ int s_taken[MAXT], s_draw[MAXT];
  int2 dec = make_int2(0, 0);
  int par = 0, tk = 0;
  if (t < T) {
    dec = *reinterpret_cast<const int2*>(a.exact_dec + ((size_t)b * T + t) * 2);
    par = a.parent[t];
    tk = a.tokens[(size_t)b * T + t];
  }
  int L = 0;
  if (t == 0) L = c.kv_len[b];
  int before = 0;
  if (t == 0) {
    sh.L = L;
    if (gridDim.x > 1) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      vmcnt<0>();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      before = __hip_atomic_fetch_add(c.counters + b, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  stage_tree(T, par, tk, sh);
  if (t < T) {
    s_taken[t] = dec.x;
    s_draw[t] = dec.y;
  }
  __syncthreads();
  if (t == 0) {
    int v = 0;
    // a taken child is a later node, so the walk ends within T steps
    for (int i = 0; i < T; ++i) {
      const int ch = s_taken[v];
      if (ch <= v || ch >= T) break;
      v = ch;
    }
    sh.best = v;
  }
  __syncthreads();
  const int v = sh.best;
  if (blockIdx.x == 0 && t < 64) {
    int depth = 0;
    for (int x = v; x != 0 && depth < K; x = sh.parent[x]) ++depth;
    // best path: the lowest path index whose node at this depth is v
    int bp = 0x7fffffff;
    for (int q = t; q < a.P; q += 64)
      if (a.retrieve[(size_t)q * (K + 1) + depth] == v) bp = min(bp, q);
    bp = -wave_max_i(-bp);
    if (t == 0) {
      a.accept_len[b] = depth;
      a.last_node[b] = v;
      int* out = a.out_tokens + (size_t)b * (K + 1);
      for (int j = depth + 1; j <= K; ++j) out[j] = -1;
      int x = v;
      for (int j = depth; j >= 0; --j) {
        out[j] = sh.tok[x];
        x = sh.parent[x];
      }
      a.next_root[b] = s_draw[v];
      a.best_path[b] = bp == 0x7fffffff ? 0 : bp;
    }
  }
  const bool last = (int)gridDim.x == 1 || before == (int)gridDim.x - 1;
  commit_lds<ET>(c, b, v, sh.L, sh, blockIdx.x, gridDim.x, last);
  if (t == 0 && gridDim.x > 1 && last) coherent_store(c.counters + b, 0);
}

// Workgroups a sequence of the composite posterior + commit kernels: the
// copy spread over up to kCommitParts, about one workgroup per compute unit
// in all.
int commit_parts(int B) { return std::max(1, std::min(kCommitParts, device_cus() / std::max(B, 1))); }

}  // namespace

hipError_t launch_posterior(const PostArgs& a, hipStream_t st) {
  if (a.mode == 2 && a.V <= kExactLdsV && exact_lds_fits()) {
    hipLaunchKernelGGL(exact_node_kernel, dim3(a.T, a.B), dim3(1024), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(exact_walk_kernel, dim3(a.B), dim3(64), 0, st, a);
  }
  else if (a.mode == 2)
    hipLaunchKernelGGL(posterior_exact_kernel, dim3(a.B), dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(posterior_kernel, dim3(a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_posterior_commit(const PostArgs& a, const CommitArgs& c, hipStream_t st) {
  if (a.mode == 2) {
    // exact: the node-parallel posterior, then the walk with the commit;
    // vocabularies past the LDS kernel take the separate kernels
    if (a.V <= kExactLdsV && exact_lds_fits()) {
      const int rx = a.lm_part ? (a.T + 3) / 4 : 0;   // row-statistics workgroups
      hipLaunchKernelGGL(exact_node_kernel, dim3(a.T + rx, a.B), dim3(1024), 0, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const dim3 grid(commit_parts(a.B), a.B);
      if (c.f32)
        hipLaunchKernelGGL(exact_walk_commit_kernel<F32>, grid, dim3(kPostThreads), 0, st, a, c);
      else
        hipLaunchKernelGGL(exact_walk_commit_kernel<BF16>, grid, dim3(kPostThreads), 0, st, a, c);
      return hipGetLastError();
    }
    hipError_t e = hipSuccess;
    if (a.lm_part)
      e = launch_row_stats_merge(a.lm_part, a.lm_G, a.B * a.T, a.inv_tau, a.row_stats_out,
                                 a.row_argmax_out, st);
    if (e != hipSuccess) return e;
    e = launch_posterior(a, st);
    if (e != hipSuccess) return e;
    return launch_commit(c, st);
  }
  const dim3 grid(commit_parts(a.B), a.B);
  if (c.f32)
    hipLaunchKernelGGL(posterior_commit_kernel<F32>, grid, dim3(kPostThreads), 0, st, a, c);
  else
    hipLaunchKernelGGL(posterior_commit_kernel<BF16>, grid, dim3(kPostThreads), 0, st, a, c);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t st) {
  if (a.f32)
    hipLaunchKernelGGL(commit_kernel<F32>, dim3(a.B), dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(commit_kernel<BF16>, dim3(a.B), dim3(1024), 0, st, a);
  return hipGetLastError();
}

}  // namespace medusa
