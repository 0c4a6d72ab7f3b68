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
// Exact: one 1024-thread workgroup per sequence walks the tree; each p/q
// step is a block-wide pass over the vocabulary.
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
// out_tokens and next_root; on return every thread sees sh.best, sh.depth.
__device__ void posterior_det_lds(const PostArgs& a, int b, float cl, TreeLds& sh) {
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
                              TreeLds& sh) {
  const int c = threadIdx.x;
  int r = -1;
#pragma unroll
  for (int j = 0; j <= MAXK; ++j)
    if (j == sh.depth) r = ret[j];
  if (c < a.P && r == sh.best) atomicMin(&sh.bp, c);
  __syncthreads();
  if (c == 0) a.best_path[b] = sh.bp < a.P ? sh.bp : 0;
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

// Exact mode for V <= kExactLdsV: the target distribution lives in LDS as
// unnormalised weights p[x] with one scale factor, p(x) = p[x] * scale, which
// is the product posterior_exact_kernel stores, so every value and decision
// is the same while the normalising passes disappear. Each pass over the
// vocabulary reads its logits from clamped indices, all of a thread's loads
// (32 for V = 32768) in flight before the first is used; the tree, tokens and
// uniforms are staged in LDS.
constexpr int kExactLdsV = 32768;

__global__ __launch_bounds__(1024) void posterior_exact_lds_kernel(PostArgs a) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int T = a.T, V = a.V, K = a.K;
  constexpr int kStride = 1024, kBatch = kExactLdsV / 1024;
  __shared__ float p[kExactLdsV];
  __shared__ float red[16];
  __shared__ CdfLds cdf;
  __shared__ int s_par[MAXT], s_tok[MAXT];
  __shared__ float s_ua[MAXT];
  __shared__ int s_next, s_bp;
  if (t < T) {
    s_par[t] = a.parent[t];
    s_tok[t] = a.tokens[(size_t)b * T + t];
    s_ua[t] = a.u_accept[(size_t)b * T + t];
  }
  if (t == 0) s_bp = 0x7fffffff;
  __syncthreads();
  const auto par = [&](int x) { return min(max(s_par[x], 0), T - 1); };
  // f(x, value of row[x]) for this thread's tokens x = t + 1024 i, in x order
  const auto stream = [&](const float* row, auto&& f) {
    for (int x0 = t; x0 < V; x0 += kStride * kBatch) {
      float lv[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) lv[i] = row[min(x0 + kStride * i, V - 1)];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (x0 + kStride * i < V) f(x0 + kStride * i, lv[i]);
    }
  };
  float scale = 1.f;
  const auto load_p = [&](int v) {
    float mx = kNegInf;
    stream(a.verify_logits + ((size_t)b * T + v) * V, [&](int x, float l) {
      const float z = l * a.inv_tau;
      p[x] = z;
      mx = fmaxf(mx, z);
    });
    mx = block_max(mx, red);
    float s = 0.f;
#pragma unroll 8
    for (int x = t; x < V; x += kStride) {
      const float e = exp_e(p[x] - mx);
      p[x] = e;
      s += e;
    }
    s = block_sum(s, red);   // ends with a barrier: p is complete
    scale = 1.f / s;
  };

  int v = 0;
  int next = -1;
  load_p(0);
  while (true) {
    int dv = 0;
    for (int x = v; x != 0 && dv < K; x = par(x)) ++dv;
    int taken = -1;
    if (dv < K) {
      const float* hl = a.head_logits + ((size_t)b * K + dv) * V;
      const float lse = a.head_lse[(size_t)b * K + dv];
      for (int c = v + 1; c < T; ++c) {
        if (s_par[c] != v) continue;
        const int x = min(max(s_tok[c], 0), V - 1);
        // every thread takes the same decision from the same values
        if (s_ua[c] * exp_e(hl[x] - lse) < p[x] * scale) {
          taken = c;
          break;
        }
        // residual p <- norm(max(0, p - q)); kept when all zero
        float s = 0.f;
        stream(hl, [&](int y, float l) { s += fmaxf(p[y] * scale - exp_e(l - lse), 0.f); });
        s = block_sum(s, red);
        if (s > 0.f) {
          stream(hl, [&](int y, float l) { p[y] = fmaxf(p[y] * scale - exp_e(l - lse), 0.f); });
          scale = 1.f / s;
        }
        __syncthreads();
      }
    }
    if (taken < 0) {
      const ScaledRow w{p, scale, V};
      cdf_build<true>(w, V, cdf);
      if (t == 0) s_next = cdf_draw(w, V, a.u_resample[(size_t)b * T + v], cdf);
      __syncthreads();
      next = s_next;
      break;
    }
    // Every wave has read p[x] for the decision above before any wave
    // overwrites p with the accepted child's row.
    __syncthreads();
    v = taken;
    load_p(v);
  }
  int depth = 0;
  for (int x = v; x != 0 && depth < K; x = par(x)) ++depth;
  // best path: the lowest path index whose node at this depth is v
  if (t < a.P && a.retrieve[(size_t)t * (K + 1) + depth] == v) atomicMin(&s_bp, t);
  __syncthreads();
  if (t != 0) return;
  a.accept_len[b] = depth;
  a.last_node[b] = v;
  int* out = a.out_tokens + (size_t)b * (K + 1);
  for (int j = depth + 1; j <= K; ++j) out[j] = -1;
  int x = v;
  for (int j = depth; j >= 0; --j) {
    out[j] = s_tok[x];
    x = par(x);
  }
  a.next_root[b] = next;
  a.best_path[b] = s_bp == 0x7fffffff ? 0 : s_bp;
}

// The LDS kernel needs more LDS than older parts give one workgroup; it runs
// where the device's per-workgroup limit holds it.
bool exact_lds_fits() {
  static const bool v = [] {
    int dev = 0, lim = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(posterior_exact_lds_kernel)) !=
            hipSuccess)
      return false;
    return fa.sharedSizeBytes <= (size_t)lim;
  }();
  return v;
}

// ---- commit ----------------------------------------------------------------------
// One 1024-thread workgroup per sequence; the path's K/V rows are copied as
// 16-byte vectors (a node's row [H][Dh] is contiguous in the tree buffers, a
// head's row Dh is contiguous in the cache), every thread loading all its
// vectors (up to kCopyBatch per tensor) before it stores any, so the copy
// costs one round trip to memory.
constexpr int kCopyBatch = 4;

// Commit of sequence b's accepted path ending at node `last`, prefix length
// L, over the whole workgroup; sh.parent holds the tree.
template <class ET>
__device__ void commit_lds(const CommitArgs& a, int b, int last_in, int L, TreeLds& sh) {
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
  const float4* y = reinterpret_cast<const float4*>(a.y + ((size_t)b * T + sh.path[d]) * a.d);
  float4* hn = reinterpret_cast<float4*>(a.h_next + (size_t)b * a.d);
  if (room) {
    const int vec_row = H * Dh / PV;          // 16-byte vectors per node row
    const int vec_head = Dh / PV;             // per head
    const int total = (d + 1) * vec_row;
    const u32x4_t* kt = reinterpret_cast<const u32x4_t*>(a.k_tree);
    const u32x4_t* vt = reinterpret_cast<const u32x4_t*>(a.v_tree);
    u32x4_t* kc = reinterpret_cast<u32x4_t*>(a.k_cache);
    u32x4_t* vc = reinterpret_cast<u32x4_t*>(a.v_cache);
    for (int e0 = threadIdx.x; e0 < total; e0 += kCopyBatch * blockDim.x) {
      u32x4_t kv[kCopyBatch], vv[kCopyBatch];
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int e = min(e0 + u * (int)blockDim.x, total - 1);
        const int i = e / vec_row, rem = e - i * vec_row;
        const size_t src = ((size_t)b * T + sh.path[i]) * vec_row + rem;
        kv[u] = kt[src];
        vv[u] = vt[src];
      }
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int e = e0 + u * (int)blockDim.x;
        if (e >= total) break;
        const int i = e / vec_row, rem = e - i * vec_row;
        const int hh = rem / vec_head, x = rem - hh * vec_head;
        const size_t dst = (((size_t)b * H + hh) * a.Lmax + L + i) * vec_head + x;
        kc[dst] = kv[u];
        vc[dst] = vv[u];
      }
    }
  }
  for (int e = threadIdx.x; e < a.d / 4; e += blockDim.x) hn[e] = y[e];
  __syncthreads();
  if (threadIdx.x == 0) (a.kv_len_out ? a.kv_len_out : a.kv_len)[b] = room ? L + d + 1 : -1;
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

// Composite step, greedy / typical: one workgroup per sequence evaluates the
// posterior from the merged row statistics and commits the accepted path.
// All the loads the decision needs -- row statistics, child logits, tokens,
// parents, path rows, the prefix length -- are issued before any is used.
template <class ET>
__global__ __launch_bounds__(1024) void posterior_commit_kernel(PostArgs a, CommitArgs c) {
  const int b = blockIdx.x, t = threadIdx.x, T = a.T;
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
  if (t == 0) sh.L = c.kv_len[b];
  if (t < T) {
    const size_t r = (size_t)b * T + t;
    sh.stat[t] = RowStat{a.row_stats[r * 3 + 0], a.row_stats[r * 3 + 1],
                         a.row_stats[r * 3 + 2], a.row_argmax[r]};
  }
  stage_tree(T, par, tk, sh);
  __syncthreads();
  posterior_det_lds(a, b, cl, sh);
  best_path_lds(a, b, ret, sh);
  commit_lds<ET>(c, b, sh.best, sh.L, sh);
}

}  // namespace

hipError_t launch_posterior(const PostArgs& a, hipStream_t st) {
  if (a.mode == 2 && a.V <= kExactLdsV && exact_lds_fits())
    hipLaunchKernelGGL(posterior_exact_lds_kernel, dim3(a.B), dim3(1024), 0, st, a);
  else if (a.mode == 2)
    hipLaunchKernelGGL(posterior_exact_kernel, dim3(a.B), dim3(1024), 0, st, a);
  else
    hipLaunchKernelGGL(posterior_kernel, dim3(a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_posterior_commit(const PostArgs& a, const CommitArgs& c, hipStream_t st) {
  if (c.f32)
    hipLaunchKernelGGL(posterior_commit_kernel<F32>, dim3(a.B), dim3(1024), 0, st, a, c);
  else
    hipLaunchKernelGGL(posterior_commit_kernel<BF16>, dim3(a.B), dim3(1024), 0, st, a, c);
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
