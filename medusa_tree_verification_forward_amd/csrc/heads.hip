// Medusa heads on gfx950 ("Medusa 深读", §3.1, head equation):
//   z_k = h + SiLU(W1_k h + b1_k),  l_k = W2_k z_k,  top-s of l_k,  lse of l_k.
//
// Both products are matrix-vector streams over bf16 (or fp32) weights, bound
// by HBM bandwidth. A wavefront owns ROWS weight rows at a time; each lane
// reads 16-byte vectors along the row (consecutive lanes, consecutive
// vectors), multiplies them with the activation held in LDS, and the row sums
// are finished with DPP reductions. The W2 pass never writes the V logits
// unless asked: each wave keeps a running top-s list spread over lanes 0..s-1
// (one entry per lane, best first) plus online softmax statistics, and a
// workgroup leaves one partial record per (sequence, head, row block). A small
// merge kernel reduces the records of one (sequence, head) in a fixed order.
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kNoId = 0x7fffffff;

// Partial dot products of ROWS consecutive weight rows with NB activation
// vectors (fp32 in LDS, row stride ldx). acc[b][r] holds this lane's share.
// Rows past `nrows` read the last valid row and are ignored by the caller.
template <class ET, int NB, int ROWS>
__device__ __forceinline__ void dot_rows(const typename ET::storage* __restrict__ W,
                                         size_t row0, int nrows, int d,
                                         const float* __restrict__ xs, int ldx,
                                         float (&acc)[NB][ROWS]) {
  constexpr int PV = ET::kPerVec;
  const int lane = threadIdx.x & 63;
  const int nvec = d / PV;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[b][r] = 0.f;
  const typename ET::storage* rowp[ROWS];
#pragma unroll
  for (int r = 0; r < ROWS; ++r) rowp[r] = W + (row0 + (size_t)(r < nrows ? r : nrows - 1)) * d;

  int c = lane;
  // two vectors per row in flight per iteration
  for (; c + 64 < nvec; c += 128) {
    u32x4_t w0[ROWS], w1[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
      w0[r] = load16_stream(rowp[r] + (size_t)c * PV);
      w1[r] = load16_stream(rowp[r] + (size_t)(c + 64) * PV);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float x0[PV], x1[PV];
#pragma unroll
      for (int e = 0; e < PV; ++e) {
        x0[e] = xs[b * ldx + c * PV + e];
        x1[e] = xs[b * ldx + (c + 64) * PV + e];
      }
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float f0[PV], f1[PV];
        ET::widen(w0[r], f0);
        ET::widen(w1[r], f1);
        float a = acc[b][r];
#pragma unroll
        for (int e = 0; e < PV; ++e) a = fmaf(f0[e], x0[e], a);
#pragma unroll
        for (int e = 0; e < PV; ++e) a = fmaf(f1[e], x1[e], a);
        acc[b][r] = a;
      }
    }
  }
  if (c < nvec) {
    u32x4_t w0[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) w0[r] = load16_stream(rowp[r] + (size_t)c * PV);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float x0[PV];
#pragma unroll
      for (int e = 0; e < PV; ++e) x0[e] = xs[b * ldx + c * PV + e];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        float f0[PV];
        ET::widen(w0[r], f0);
        float a = acc[b][r];
#pragma unroll
        for (int e = 0; e < PV; ++e) a = fmaf(f0[e], x0[e], a);
        acc[b][r] = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// z[b][k][i] = h[b][i] + silu(sum_j W1[k][i][j] h[b][j] + b1[k][i])
// grid.x: blocks of `rows_per_wg` rows over the K*d rows of all heads.
template <class ET, int NB, int ROWS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void heads_w1_kernel(
    const float* __restrict__ h, int B, int b0, int K, int d,
    const typename ET::storage* __restrict__ W1, const float* __restrict__ b1,
    float* __restrict__ z, int rows_per_wg) {
  extern __shared__ float xs[];   // [NB][d]
  const int nb = min(NB, B - b0);
  for (int i = threadIdx.x; i < NB * d; i += blockDim.x) {
    const int b = i / d, j = i - b * d;
    xs[i] = b < nb ? h[(size_t)(b0 + b) * d + j] : 0.f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int total = K * d;
  const int rbeg = blockIdx.x * rows_per_wg;
  const int rend = min(total, rbeg + rows_per_wg);
  for (int r0 = rbeg + wave * ROWS; r0 < rend; r0 += WAVES * ROWS) {
    const int nrows = min(ROWS, rend - r0);
    float acc[NB][ROWS];
    dot_rows<ET, NB, ROWS>(W1, (size_t)r0, nrows, d, xs, d, acc);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float u = wave_sum(acc[b][r]);
        if (lane == r && r < nrows && b < nb) {
          const int row = r0 + r;          // row = k*d + i
          const int k = row / d, i = row - k * d;
          const float uu = u + (b1 ? b1[row] : 0.f);
          const float sig = 1.f / (1.f + exp_e(-uu));
          z[((size_t)(b0 + b) * K + k) * d + i] = xs[b * d + i] + uu * sig;
        }
      }
    }
  }
}

// Lane-parallel sorted list: lane i (< S) holds entry i, best first.
// Insert (v, id) known to beat the current S-th entry.
__device__ __forceinline__ void list_insert(float& tv, int& ti, float v, int id, int S) {
  const int lane = threadIdx.x & 63;
  const bool ahead = lane < S && better(tv, ti, v, id);
  const int pos = __popcll(__ballot(ahead));
  // entry of lane-1 (row_shr:1 within the 16-lane row holding the list)
  const float pv = __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(tv), __float_as_int(tv), 0x111, 0xf, 0xf, false));
  const int pi = __builtin_amdgcn_update_dpp(ti, ti, 0x111, 0xf, 0xf, false);
  if (lane == pos) {
    tv = v;
    ti = id;
  } else if (lane > pos) {
    tv = pv;
    ti = pi;
  }
}

// Merge of online softmax statistics (m, s): s = sum exp(l - m).
__device__ __forceinline__ void stats_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == kNegInf) return;
  s = s * exp_e(m - mn) + s2 * exp_e(m2 - mn);
  m = mn;
}

// ---------------------------------------------------------------------------
// l = W2_k z_k for the rows of one block; running top-S and (max, sum exp).
// grid = (G, K): block g of head k covers rows [g*rows_per_wg, ...).
// Partial records: part_val/part_id [B][K][G][S], part_m/part_s [B][K][G].
template <class ET, int NB, int ROWS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void heads_w2_kernel(
    const float* __restrict__ z, int B, int b0, int K, int V, int d,
    const typename ET::storage* __restrict__ W2, int rows_per_wg, int S,
    float* __restrict__ head_logits, float* __restrict__ part_val, int* __restrict__ part_id,
    float* __restrict__ part_m, float* __restrict__ part_s, int G) {
  extern __shared__ float xs[];   // [NB][d], then per-wave list exchange
  const int k = blockIdx.y, g = blockIdx.x;
  const int nb = min(NB, B - b0);
  for (int i = threadIdx.x; i < NB * d; i += blockDim.x) {
    const int b = i / d, j = i - b * d;
    xs[i] = b < nb ? z[((size_t)(b0 + b) * K + k) * d + j] : 0.f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rbeg = g * rows_per_wg;
  const int rend = min(V, rbeg + rows_per_wg);
  const typename ET::storage* Wk = W2 + (size_t)k * V * d;

  float tv[NB], m[NB], s[NB];
  int ti[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    tv[b] = kNegInf;
    ti[b] = kNoId;
    m[b] = kNegInf;
    s[b] = 0.f;
  }
  for (int r0 = rbeg + wave * ROWS; r0 < rend; r0 += WAVES * ROWS) {
    const int nrows = min(ROWS, rend - r0);
    float acc[NB][ROWS];
    dot_rows<ET, NB, ROWS>(Wk, (size_t)r0, nrows, d, xs, d, acc);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v[ROWS];
#pragma unroll
      for (int r = 0; r < ROWS; ++r) v[r] = wave_sum(acc[b][r]);
      if (head_logits && b < nb && lane < nrows) {
        float mine = v[0];
#pragma unroll
        for (int r = 1; r < ROWS; ++r)
          if (lane == r) mine = v[r];
        head_logits[((size_t)(b0 + b) * K + k) * V + r0 + lane] = mine;
      }
      // online statistics over the valid rows
      float bm = v[0];
#pragma unroll
      for (int r = 1; r < ROWS; ++r)
        if (r < nrows) bm = fmaxf(bm, v[r]);
      float bs = 0.f;
#pragma unroll
      for (int r = 0; r < ROWS; ++r)
        if (r < nrows) bs += exp_e(v[r] - bm);
      stats_merge(m[b], s[b], bm, bs);
      // top-S insertion, gated by the current S-th entry
      float thv = readlane_f(tv[b], S - 1);
      int thi = __builtin_amdgcn_readlane(ti[b], S - 1);
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        if (r < nrows && better(v[r], r0 + r, thv, thi)) {
          list_insert(tv[b], ti[b], v[r], r0 + r, S);
          thv = readlane_f(tv[b], S - 1);
          thi = __builtin_amdgcn_readlane(ti[b], S - 1);
        }
      }
    }
  }
  // merge the waves of this block through LDS (after the activation is no
  // longer needed)
  __syncthreads();
  float* lv = xs;                                        // [WAVES][NB][S]
  int* li = reinterpret_cast<int*>(xs + WAVES * NB * MAXS_LDS);
  float* lm = xs + 2 * WAVES * NB * MAXS_LDS;            // [WAVES][NB]
  float* ls = lm + WAVES * NB;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (lane < S) {
      lv[(wave * NB + b) * MAXS_LDS + lane] = tv[b];
      li[(wave * NB + b) * MAXS_LDS + lane] = ti[b];
    }
    if (lane == 0) {
      lm[wave * NB + b] = m[b];
      ls[wave * NB + b] = s[b];
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    for (int w = 1; w < WAVES; ++w) {
      for (int e = 0; e < S; ++e) {
        const float v = lv[(w * NB + b) * MAXS_LDS + e];
        const int id = li[(w * NB + b) * MAXS_LDS + e];
        const float thv = readlane_f(tv[b], S - 1);
        const int thi = __builtin_amdgcn_readlane(ti[b], S - 1);
        if (better(v, id, thv, thi)) list_insert(tv[b], ti[b], v, id, S);
      }
      stats_merge(m[b], s[b], lm[w * NB + b], ls[w * NB + b]);
    }
    if (b < nb) {
      const size_t rec = ((size_t)(b0 + b) * K + k) * G + g;
      if (lane < S) {
        part_val[rec * S + lane] = tv[b];
        part_id[rec * S + lane] = ti[b];
      }
      if (lane == 0) {
        part_m[rec] = m[b];
        part_s[rec] = s[b];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge the G partial records of one (sequence, head): one wavefront.
// grid = (K, B). Each lane keeps a private sorted list of its candidates in
// registers (a candidate that does not beat the lane's S-th entry costs one
// compare); then S selection rounds take the best lane head with a DPP
// (value desc, id asc) reduction and pop it from its lane.
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

template <int SMAX>
__global__ __launch_bounds__(64) void heads_merge_kernel(
    int K, int G, int S, const float* __restrict__ part_val, const int* __restrict__ part_id,
    const float* __restrict__ part_m, const float* __restrict__ part_s,
    int* __restrict__ topk_ids, float* __restrict__ topk_logits, float* __restrict__ lse) {
  const int k = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const size_t rec0 = ((size_t)b * K + k) * G;
  float lv[SMAX];
  int li[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    lv[j] = kNegInf;
    li[j] = kNoId;
  }
  const int ncand = G * S;
  for (int c = lane; c < ncand; c += 64) {
    const float v = part_val[rec0 * S + c];
    const int id = part_id[rec0 * S + c];
    // the S-th entry sits at a runtime index: select it with an unrolled scan
    float tv = kNegInf;
    int ti = kNoId;
#pragma unroll
    for (int j = 0; j < SMAX; ++j)
      if (j == S - 1) {
        tv = lv[j];
        ti = li[j];
      }
    if (better(v, id, tv, ti)) reg_insert<SMAX>(lv, li, v, id, S);
  }
  float out_v = kNegInf;
  int out_i = kNoId;
  for (int r = 0; r < S; ++r) {
    float bv = lv[0];
    int bi = li[0];
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
    // best of the four 16-lane rows (uniform)
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
    if (lane == r) {
      out_v = bv;
      out_i = bi;
    }
    // pop the winner from the lane that holds it (ids are unique)
    if (li[0] == bi) {
#pragma unroll
      for (int j = 0; j < SMAX - 1; ++j) {
        lv[j] = lv[j + 1];
        li[j] = li[j + 1];
      }
      lv[SMAX - 1] = kNegInf;
      li[SMAX - 1] = kNoId;
    }
  }
  const size_t out = ((size_t)b * K + k) * S;
  if (lane < S) {
    topk_ids[out + lane] = out_i;
    topk_logits[out + lane] = out_v;
  }
  if (lse) {
    float mm = kNegInf;
    for (int g = lane; g < G; g += 64) mm = fmaxf(mm, part_m[rec0 + g]);
    mm = wave_max(mm);
    float ss = 0.f;
    for (int g = lane; g < G; g += 64) {
      const float pm = part_m[rec0 + g];
      if (pm != kNegInf) ss += part_s[rec0 + g] * exp_e(pm - mm);
    }
    ss = wave_sum(ss);
    if (lane == 0) lse[(size_t)b * K + k] = mm + __logf(ss);
  }
}

template <class ET, int NB>
hipError_t launch_heads_nb(const HeadsArgs& a, int b0, hipStream_t st) {
  constexpr int ROWS = NB <= 2 ? 4 : (NB == 4 ? 2 : 1);
  constexpr int WAVES = NB <= 2 ? 4 : (NB == 4 ? 8 : 16);
  const size_t lds_x = (size_t)NB * a.d * sizeof(float);
  const int total1 = a.K * a.d;
  const int g1 = (total1 + a.w1_rows_per_wg - 1) / a.w1_rows_per_wg;
  hipLaunchKernelGGL((heads_w1_kernel<ET, NB, ROWS, WAVES>), dim3(g1), dim3(WAVES * 64), lds_x,
                     st, a.h, a.B, b0, a.K, a.d,
                     reinterpret_cast<const typename ET::storage*>(a.W1), a.b1, a.z,
                     a.w1_rows_per_wg);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_list = (size_t)WAVES * NB * (2 * MAXS_LDS + 2) * sizeof(float);
  const size_t lds2 = lds_x > lds_list ? lds_x : lds_list;
  if (a.ev_before) {
    e = hipEventRecord(a.ev_before, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((heads_w2_kernel<ET, NB, ROWS, WAVES>), dim3(a.G, a.K), dim3(WAVES * 64),
                     lds2, st, a.z, a.B, b0, a.K, a.V, a.d,
                     reinterpret_cast<const typename ET::storage*>(a.W2), a.w2_rows_per_wg,
                     a.S, a.head_logits, a.part_val, a.part_id, a.part_m, a.part_s, a.G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_after) e = hipEventRecord(a.ev_after, st);
  return e;
}

template <class ET>
hipError_t launch_heads_et(const HeadsArgs& a, hipStream_t st) {
  for (int b0 = 0; b0 < a.B; b0 += 8) {
    const int nb = a.B - b0;
    hipError_t e;
    if (nb == 1)
      e = launch_heads_nb<ET, 1>(a, b0, st);
    else if (nb == 2)
      e = launch_heads_nb<ET, 2>(a, b0, st);
    else if (nb <= 4)
      e = launch_heads_nb<ET, 4>(a, b0, st);
    else
      e = launch_heads_nb<ET, 8>(a, b0, st);
    if (e != hipSuccess) return e;
  }
#define MERGE_LAUNCH(SM)                                                                    \
  hipLaunchKernelGGL(heads_merge_kernel<SM>, dim3(a.K, a.B), dim3(64), 0, st, a.K, a.G, a.S, \
                     a.part_val, a.part_id, a.part_m, a.part_s, a.topk_ids, a.topk_logits,   \
                     a.lse)
  if (a.S <= 4)
    MERGE_LAUNCH(4);
  else if (a.S <= 8)
    MERGE_LAUNCH(8);
  else
    MERGE_LAUNCH(16);
#undef MERGE_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_heads(const HeadsArgs& a, hipStream_t st) {
  return a.f32 ? launch_heads_et<F32>(a, st) : launch_heads_et<BF16>(a, st);
}

}  // namespace medusa
