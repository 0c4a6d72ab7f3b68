// Top-s selection and log-sum-exp of the heads' vocabulary projections
// ("Medusa 深读", §3.1: each head's candidates are its top-s tokens; the
// head softmax needs the log-sum-exp of its logits).
//
// Candidates are (logit, token id) pairs ordered by `better` (higher logit
// first, equal logits: lower id first); ids are unique, so the top-s set and
// its order do not depend on the order candidates are visited in. The
// log-sum-exp of G partial (max, sum) records is reduced in a fixed order.
#pragma once

#include "common.h"

namespace medusa {

constexpr int kNoId = 0x7fffffff;

// Best (value desc, id asc) over the wave, returned to every lane.
__device__ __forceinline__ void wave_best(float& bv, int& bi) {
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    float ov;
    int oi;
    if (step == 0) { ov = dpp<kDppQuadXor1>(bv); oi = dppi<kDppQuadXor1>(bi); }
    else if (step == 1) { ov = dpp<kDppQuadXor2>(bv); oi = dppi<kDppQuadXor2>(bi); }
    else if (step == 2) { ov = dpp<kDppRowRor4>(bv); oi = dppi<kDppRowRor4>(bi); }
    else { ov = dpp<kDppRowRor8>(bv); oi = dppi<kDppRowRor8>(bi); }
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  float wv = readlane_f(bv, 0);
  int wi = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int row = 16; row < 64; row += 16) {
    const float ov = readlane_f(bv, row);
    const int oi = __builtin_amdgcn_readlane(bi, row);
    if (better(ov, oi, wv, wi)) {
      wv = ov;
      wi = oi;
    }
  }
  bv = wv;
  bi = wi;
}

// Insert (v, id) into a lane's sorted list of the S best (SMAX >= S slots).
template <int SMAX>
__device__ __forceinline__ void reg_insert(float (&lv)[SMAX], int (&li)[SMAX], float v, int id,
                                           int S) {
#pragma unroll
  for (int j = SMAX - 1; j >= 0; --j) {
    if (j >= S) continue;
    if (!better(v, id, lv[j], li[j])) continue;
    if (j > 0 && better(v, id, lv[j - 1], li[j - 1])) {
      lv[j] = lv[j - 1];
      li[j] = li[j - 1];
    } else {
      lv[j] = v;
      li[j] = id;
    }
  }
}

// S rounds of selection over the lanes' sorted lists; lane r < S receives
// the r-th best of the wave.
template <int SMAX>
__device__ __forceinline__ void wave_select(float (&lv)[SMAX], int (&li)[SMAX], int S,
                                            float& out_v, int& out_i) {
  const int lane = threadIdx.x & 63;
  out_v = -__builtin_huge_valf();
  out_i = kNoId;
  for (int r = 0; r < S; ++r) {
    float bv = lv[0];
    int bi = li[0];
    wave_best(bv, bi);
    if (lane == r) {
      out_v = bv;
      out_i = bi;
    }
    // pop the winner from the lane that holds it (ids are unique)
    if (li[0] == bi && bi != kNoId) {
#pragma unroll
      for (int j = 0; j < SMAX - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[SMAX - 1] = -__builtin_huge_valf();
      li[SMAX - 1] = kNoId;
    }
  }
}

// The S best of n candidates (val[i], id[i]) in one wave: lane r < S
// receives the r-th best. Candidates are read kBatch per lane at a time,
// every load of a batch issued before any is compared.
template <int SMAX>
__device__ __forceinline__ void wave_topk(const float* __restrict__ val,
                                          const int* __restrict__ id, int n, int S,
                                          float& out_v, int& out_i) {
  constexpr int kBatch = 8;
  const int lane = threadIdx.x & 63;
  float lv[SMAX];
  int li[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    lv[j] = -__builtin_huge_valf();
    li[j] = kNoId;
  }
  for (int base = 0; base < n; base += 64 * kBatch) {
    float v[kBatch];
    int x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int c = min(base + lane + 64 * u, n - 1);
      v[u] = val[c];
      x[u] = id[c];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (base + lane + 64 * u < n) reg_insert<SMAX>(lv, li, v[u], x[u], S);
  }
  wave_select<SMAX>(lv, li, S, out_v, out_i);
}

// log sum_g s_g e^{m_g} of G partial records (m_g, s_g) in one wave
// (natural log), returned to every lane: lane l takes records l + 64 u in
// u order, then a fixed-order wave maximum and sum.
constexpr int kLseRegs = 4;   // records per lane held in registers (G <= 256)
__device__ __forceinline__ void lse_load(const float* __restrict__ pm,
                                         const float* __restrict__ ps, int G,
                                         float (&m)[kLseRegs], float (&sv)[kLseRegs]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < kLseRegs; ++u) {
    const int g = min(lane + 64 * u, G - 1);
    m[u] = pm[g];
    sv[u] = ps[g];
  }
}
__device__ __forceinline__ float lse_of(const float (&m)[kLseRegs], const float (&sv)[kLseRegs],
                                        int G) {
  const int lane = threadIdx.x & 63;
  float mx = -__builtin_huge_valf();
#pragma unroll
  for (int u = 0; u < kLseRegs; ++u)
    if (lane + 64 * u < G) mx = fmaxf(mx, m[u]);
  mx = wave_max(mx);
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kLseRegs; ++u)
    if (lane + 64 * u < G && m[u] != -__builtin_huge_valf()) s += sv[u] * exp_e(m[u] - mx);
  return mx + __logf(wave_sum(s));
}
__device__ __forceinline__ float wave_lse(const float* __restrict__ pm,
                                          const float* __restrict__ ps, int G) {
  if (G <= 64 * kLseRegs) {
    float m[kLseRegs], sv[kLseRegs];
    lse_load(pm, ps, G, m, sv);
    return lse_of(m, sv, G);
  }
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63;
  float mx = -__builtin_huge_valf();
  for (int g0 = 0; g0 < G; g0 += 64 * kBatch) {
    float m[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) m[u] = pm[min(g0 + lane + 64 * u, G - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (g0 + lane + 64 * u < G) mx = fmaxf(mx, m[u]);
  }
  mx = wave_max(mx);
  float s = 0.f;
  for (int g0 = 0; g0 < G; g0 += 64 * kBatch) {
    float m[kBatch], sv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int g = min(g0 + lane + 64 * u, G - 1);
      m[u] = pm[g];
      sv[u] = ps[g];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (g0 + lane + 64 * u < G && m[u] != -__builtin_huge_valf()) s += sv[u] * exp_e(m[u] - mx);
  }
  return mx + __logf(wave_sum(s));
}

}  // namespace medusa
