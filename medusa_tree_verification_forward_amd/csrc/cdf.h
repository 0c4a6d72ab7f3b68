// Inverse-CDF draws over V non-negative weights in one 1024-thread
// workgroup: a drafted token from a head softmax ("Medusa 深读", sampling
// the candidates in the exact acceptance setting) and the next root from the
// target or residual distribution ("Medusa Part I", Part 2, the rejection
// rule's resampling step).
//
// The CDF is a fixed sum that is monotone by construction. Chunks of CS
// consecutive tokens (CS a multiple of 8, at most kCdfChunks chunks) are each
// summed in token order by one lane; groups of 64 consecutive chunks carry
// the running sum F of their chunks, taken in order; group totals are
// combined in order into E. For token x in chunk c of group g,
//   C(x) = E[g] + (F[c] + (w_first(c) + ... + w_x)),
// and every step adds a non-negative weight to the value before it, so C
// never decreases. The last chunk of a group ends at exactly E[g + 1], and
// chunk c ends at exactly E[g] + F[c + 1]. A draw with uniform u is the
// smallest x with C(x) > u * C(V - 1), clamped to the last token with a
// positive weight (reached only when rounding puts u * C(V - 1) at the top).
#pragma once

#include "common.h"

namespace medusa {

constexpr int kCdfThreads = 1024;
constexpr int kCdfChunks = 2048;
constexpr int kCdfGroups = kCdfChunks / 64;

struct CdfLds {
  float cs[kCdfChunks];      // chunk sums
  float F[kCdfChunks];       // running sum of the group's chunks before chunk c
  float E[kCdfGroups + 1];   // running sum of the groups before group g; E[ng] = total
  int ng, nch, csz, last_nz;
};

// Tokens per chunk: 8, doubled until the chunks fit (16 for a 32000 vocabulary).
__host__ __device__ inline int cdf_chunk_size(int V) {
  int cs = 8;
  while ((V + cs - 1) / cs > kCdfChunks) cs *= 2;
  return cs;
}

// Weights of tokens x0 .. x0 + N - 1 (zero past V). The weights are read at
// clamped indices without a condition, so all N loads are in flight before
// the first is used; tokens past V are zeroed afterwards.
template <int N, class Wf>
__device__ __forceinline__ void cdf_weights(const Wf& w, int x0, int V, float (&wv)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) wv[i] = w(max(min(x0 + i, V - 1), 0));
#pragma unroll
  for (int i = 0; i < N; ++i) wv[i] = x0 + i < V ? wv[i] : 0.f;
}

// Sequential sum of chunk c's weights in token order, its last positive
// token in *last; N tokens loaded at a time.
template <int N, class Wf>
__device__ __forceinline__ float cdf_chunk_sum(const Wf& w, int c, int csz, int V, int* last) {
  float s = 0.f;
  for (int i0 = 0; i0 < csz; i0 += N) {
    float wv[N];
    cdf_weights<N>(w, c * csz + i0, V, wv);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      s += wv[i];
      if (wv[i] > 0.f) *last = c * csz + i0 + i;
    }
  }
  return s;
}

// Weights e^(l_x - lse) of a logit row l (16-byte aligned, V a multiple of
// 4): w(x) for one token, w4(x) for tokens x .. x + 3 (x a multiple of 4) in
// one 16-byte load, zero past V.
struct ExpRow {
  const float* l;
  float lse;
  int V;
  __device__ __forceinline__ float operator()(int x) const { return exp_e(l[x] - lse); }
  __device__ __forceinline__ floatx4_t w4(int x) const {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(l + min(x, V - 4));
    floatx4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x + i < V ? exp_e(v[i] - lse) : 0.f;
    return r;
  }
};

// Weights p[x] * scale of a row in LDS or memory (16-byte aligned, V a
// multiple of 4): w(x) for one token, w4(x) for four, zero past V.
struct ScaledRow {
  const float* p;
  float scale;
  int V;
  __device__ __forceinline__ float operator()(int x) const { return p[x] * scale; }
  __device__ __forceinline__ floatx4_t w4(int x) const {
    const floatx4_t v = *reinterpret_cast<const floatx4_t*>(p + min(x, V - 4));
    floatx4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x + i < V ? v[i] * scale : 0.f;
    return r;
  }
};

// Chunk c's sequential sum with the weights read four at a time (Wf::w4).
template <class Wf>
__device__ __forceinline__ float cdf_chunk_sum_v4(const Wf& w, int c, int csz, int* last) {
  float s = 0.f;
  for (int i0 = 0; i0 < csz; i0 += 16) {
    floatx4_t q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = w.w4(c * csz + i0 + 4 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s += q[u][i];
        if (q[u][i] > 0.f) *last = c * csz + i0 + 4 * u + i;
      }
  }
  return s;
}

// The rest of a build once sh.cs holds the chunk sums (written by every
// thread before the call, which every thread makes): the last token with a
// positive weight (the maximum of the threads' my_last), the groups'
// running sums F and the group totals E. Ends with a barrier.
__device__ inline void cdf_prefix(int my_last, int nch, int csz, CdfLds& sh) {
  const int t = threadIdx.x, lane = t & 63;
  const int ng = (nch + 63) / 64;
  {
    // token indices are exact in float (V < 2^24)
    const int wl = (int)wave_max((float)my_last);
    if (lane == 0) atomicMax(&sh.last_nz, wl);   // LDS atomic, one per wave
  }
  __syncthreads();
  if (t < ng) {
    float f = 0.f;
    const int end = min(64 * t + 64, nch);
#pragma unroll 8
    for (int c = 64 * t; c < end; ++c) {
      sh.F[c] = f;
      f = f + sh.cs[c];
    }
    sh.E[t + 1] = f;   // the group's total, until the pass below
  }
  __syncthreads();
  if (t == 0) {
    float e = 0.f;
    for (int g = 0; g < ng; ++g) {
      const float gt = sh.E[g + 1];
      sh.E[g] = e;
      e = e + gt;
    }
    sh.E[ng] = e;
    sh.ng = ng;
    sh.nch = nch;
    sh.csz = csz;
  }
  __syncthreads();
}

// Build the CDF of w(0 .. V-1) into sh. Every thread of the workgroup calls
// it; ends with a barrier. kVec4: chunks of 16 or more tokens read through
// Wf::w4 (16-byte loads) when V is a multiple of 4; the sums are the same.
template <bool kVec4 = false, class Wf>
__device__ void cdf_build(const Wf& w, int V, CdfLds& sh) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int csz = cdf_chunk_size(V);
  const int nch = (V + csz - 1) / csz;
  if (t == 0) sh.last_nz = -1;
  __syncthreads();
  int my_last = -1;
  // wave w sums the rows of 64 chunks w, w + 16, ...; lane l chunk 64 r + l
  for (int c0 = 64 * wave; c0 < nch; c0 += 64 * (kCdfThreads / 64)) {
    const int c = c0 + lane;
    float s;
    if constexpr (kVec4) {
      s = csz >= 16 && (V & 3) == 0 ? cdf_chunk_sum_v4(w, c, csz, &my_last)
          : csz == 8               ? cdf_chunk_sum<8>(w, c, csz, V, &my_last)
                                   : cdf_chunk_sum<16>(w, c, csz, V, &my_last);
    } else {
      s = csz == 8 ? cdf_chunk_sum<8>(w, c, csz, V, &my_last)
                   : cdf_chunk_sum<16>(w, c, csz, V, &my_last);
    }
    if (c < nch) sh.cs[c] = s;   // chunks past nch hold only tokens >= V
  }
  cdf_prefix(my_last, nch, csz, sh);
}

// The chunk in which a draw with uniform u lands: the first group, then the
// first chunk of it, whose end lies above target = u * total; returns the
// chunk (-1 when no group does, only for a target at the top) and the CDF
// before its first token, E[g] + F[c], as eg and fc.
__device__ inline int cdf_locate(float u, const CdfLds& sh, float& target, float& eg,
                                 float& fc) {
  const int ng = sh.ng, nch = sh.nch;
  target = u * sh.E[ng];
  int lo = 0, hi = ng;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (sh.E[mid + 1] > target)
      hi = mid;
    else
      lo = mid + 1;
  }
  if (lo >= ng) return -1;
  const int g = lo;
  eg = sh.E[g];
  // first chunk of the group ending above the target (its last chunk does)
  int a = 64 * g, bnd = min(64 * g + 64, nch) - 1;
  while (a < bnd) {
    const int mid = (a + bnd) >> 1;
    if (eg + (sh.F[mid] + sh.cs[mid]) > target)
      bnd = mid;
    else
      a = mid + 1;
  }
  fc = sh.F[a];
  return a;
}

// One draw with uniform u from a built CDF (any single thread).
template <class Wf>
__device__ int cdf_draw(const Wf& w, int V, float u, const CdfLds& sh) {
  const int csz = sh.csz;
  float target, eg, fc;
  const int c = cdf_locate(u, sh, target, eg, fc);
  int x = -1;
  if (c >= 0) {
    float local = 0.f;
    for (int i0 = 0; i0 < csz && x < 0; i0 += 8) {
      float wv[8];
      cdf_weights<8>(w, c * csz + i0, V, wv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        local += wv[i];
        if (x < 0 && eg + (fc + local) > target) x = c * csz + i0 + i;
      }
    }
  }
  if (x < 0 || x > sh.last_nz) x = sh.last_nz < 0 ? V - 1 : sh.last_nz;
  return x;
}

}  // namespace medusa
