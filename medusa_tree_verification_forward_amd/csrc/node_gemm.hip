// Skinny node GEMMs of the verify pass on gfx950 MFMA:
//   C[M][N] = A[M][K] * W[N][K]^T,  M = B*T tree rows (tens to a few hundred),
//   N = 3d (QKV), d (output projection) or V (verification LM head).
//
// The weights stream from HBM once; A (a few hundred KB) stays in L2.
// A workgroup of 8 waves owns 128 output columns (16 per wave), all M rows
// (in passes of 16*MT rows) and one of KS slices of K. K advances in
// k-blocks of 128 bytes per row. Both operands of a k-block -- the 128
// weight rows and the 16*MT A rows -- are copied by direct global->LDS
// loads (each lane names one 16-byte piece; a wave's 64 pieces land
// lane-major) into a ring of S stages, so up to S-1 k-blocks are in flight
// per workgroup without holding registers. One barrier per stage: every
// wave waits for its own loads of the stage (vmcnt), then s_barrier, then
// refills the slot freed by the previous stage. A lane then reads back
// exactly the MFMA fragments it needs: for weights its own two pieces, for
// A the pieces of each m-tile. Per 16-byte piece that is one
// v_mfma_f32_16x16x32_bf16 per m-tile, or four v_mfma_f32_16x16x4_f32 for
// fp32 storage (the k index inside a piece is permuted identically for
// both operands, which does not change the sum).
//
// With KS > 1 the workgroup writes fp32 partial tiles; an elementwise
// epilogue kernel sums the KS partials in order and applies
//   QKV  : RoPE on q and k (pairs i, i+Dh/2; angle pos * theta^(-2i/Dh)),
//          rounding to the storage type, scatter to [B][T][H][Dh];
//   OPROJ: y = x + acc with x = E[token], written as fp32 and storage type.
// The LM head runs with KS = 1 and reduces in-kernel: per row and 128-column
// block (max, argmax, S, W) at temperature tau with S = sum e^{(l-m)/tau},
// W = sum e^{(l-m)/tau} (l-m)/tau; the logit of every tree node's token
// under its parent's row; optional full logits. A merge kernel combines the
// column blocks of a row.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kGemmWaves = 8;
constexpr int kGemmCols = 16 * kGemmWaves;   // output columns per workgroup

// Merge of (max, S, W, argmax) records at temperature tau (see header).
__device__ __forceinline__ void rec_merge(float& m, float& s, float& w, int& a, float m2,
                                          float s2, float w2, int a2, float inv_tau) {
  if (m2 == kNegInf) return;
  if (m == kNegInf) {
    m = m2; s = s2; w = w2; a = a2;
    return;
  }
  const float mn = fmaxf(m, m2);
  const float d1 = (m - mn) * inv_tau, d2 = (m2 - mn) * inv_tau;
  const float c1 = exp_e(d1), c2 = exp_e(d2);
  const int an = better(m, a, m2, a2) ? a : a2;
  w = c1 * (w + s * d1) + c2 * (w2 + s2 * d2);
  s = c1 * s + c2 * s2;
  m = mn;
  a = an;
}

template <class ET, int MT, int S, bool LM>
__global__ __launch_bounds__(512) void node_gemm_kernel(GemmParams p) {
  using St = typename ET::storage;
  constexpr int PV = ET::kPerVec;   // elements per 16-byte piece
  constexpr int KB = 8 * PV;        // k elements per k-block (128 bytes of a row)
  constexpr int WV = kGemmWaves;
  constexpr int NA = 2 * MT;        // A pieces per lane per k-block
  constexpr int NAW = (NA + WV - 1) / WV;   // A load instructions per wave (max)
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int g = blockIdx.x, ks = blockIdx.y, KS = gridDim.y;
  const St* __restrict__ A = reinterpret_cast<const St*>(p.A);
  const St* __restrict__ W = reinterpret_cast<const St*>(p.W);

  const int n0 = g * kGemmCols;
  const int col = n0 + 16 * wave + li;
  const St* wrow = W + (size_t)min(col, p.N - 1) * p.K + PV * lq;
  const int nkb = p.K / KB;
  const int kb_lo = (int)((long)nkb * ks / KS), kb_hi = (int)((long)nkb * (ks + 1) / KS);
  const int nloc = kb_hi - kb_lo;
  const int na_w = wave < NA ? (NA - wave + WV - 1) / WV : 0;
  const int ops = 2 + na_w;         // load instructions this wave issues per stage

  __shared__ u32x4_t ringW[S][WV][2][64];
  __shared__ u32x4_t ringA[S][MT][2][64];
  __shared__ float stat[LM ? WV : 1][LM ? 16 * MT : 1][4];

  for (int m0 = 0; m0 < p.M; m0 += 16 * MT) {
    if (m0 > 0) __syncthreads();   // previous pass's readers are done
    const St* arow[NAW];
#pragma unroll
    for (int j = 0; j < NAW; ++j) {
      const int idx = min(wave + WV * j, NA - 1);
      const int r = min(m0 + 16 * (idx >> 1) + li, p.M - 1);
      const int src = p.a_rows ? min(max(p.a_rows[r], 0), p.a_nrows - 1) : r;
      arow[j] = A + (size_t)src * p.lda + PV * lq + 4 * PV * (idx & 1);
    }
    auto issue = [&](int i) {
      const int slot = i % S;
      const size_t off = (size_t)(kb_lo + i) * KB;
      dma16(wrow + off, &ringW[slot][wave][0][0]);
      dma16(wrow + off + 4 * PV, &ringW[slot][wave][1][0]);
#pragma unroll
      for (int j = 0; j < NAW; ++j) {
        const int idx = wave + WV * j;
        if (idx < NA) dma16(arow[j] + off, &ringA[slot][idx >> 1][idx & 1][0]);
      }
    };
    floatx4_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int i = 0; i < S - 1 && i < nloc; ++i) issue(i);
    for (int i = 0; i < nloc; ++i) {
      vmcnt_rt(min(S - 2, nloc - 1 - i) * ops);   // this wave's loads of stage i landed
      stage_barrier();                            // ... and everyone else's
      if (i + S - 1 < nloc) issue(i + S - 1);     // refill the slot stage i-1 used
      const int slot = i % S;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t b = ringW[slot][wave][h][lane];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4_t a = ringA[slot][mt][h][lane];
          if constexpr (PV == 8) {
            acc[mt] = mfma16x16x32_bf16(a, b, acc[mt]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mt] = mfma16x16x4_f32(__uint_as_float(a[j]), __uint_as_float(b[j]), acc[mt]);
          }
        }
      }
    }

    if constexpr (!LM) {
      // partial tile of slice ks: part[ks][r][n]
      float* part = p.part + (size_t)ks * p.M * p.N;
      if (col < p.N) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = m0 + 16 * mt + 4 * lq + j;
            if (r < p.M) part[(size_t)r * p.N + col] = acc[mt][j];
          }
      }
    } else {
      const bool cv = col < p.N;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * mt + 4 * lq + j;
          const int r = m0 + rr;
          // (max, lowest argmax) over this wave's 16 columns of the row
          float bv = cv ? acc[mt][j] : kNegInf;
          int bi = cv ? col : 0x7fffffff;
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
          float sv = 0.f, wv = 0.f;
          if (cv) {
            const float z = (acc[mt][j] - bv) * p.inv_tau;
            const float e = exp_e(z);
            sv = e;
            wv = e * z;
          }
          sv = row16_sum(sv);
          wv = row16_sum(wv);
          if (li == 0) {
            stat[wave][rr][0] = bv;
            stat[wave][rr][1] = sv;
            stat[wave][rr][2] = wv;
            stat[wave][rr][3] = __int_as_float(bi);
          }
          if (p.logits_out && cv && r < p.M) p.logits_out[(size_t)r * p.N + col] = acc[mt][j];
        }
      // logit of each tree node's token under its parent's row (this wave's columns)
      const int rows_hi = min(p.M, m0 + 16 * MT);
      const int c0 = n0 + 16 * wave;
      const int bl = m0 / p.T, bh = (rows_hi - 1) / p.T;
      const int nchild = (bh - bl + 1) * p.T;
      for (int e0 = 0; e0 < nchild; e0 += 64) {
        const int e = e0 + lane;
        int r = -1, tok = -1, node = -1;
        bool hit = false;
        if (e < nchild) {
          const int b = bl + e / p.T, cnode = e % p.T;
          if (cnode >= 1) {
            node = b * p.T + cnode;
            tok = p.tokens[node];
            r = b * p.T + min(max(p.parent[cnode], 0), p.T - 1);
            hit = tok >= c0 && tok < c0 + 16 && r >= m0 && r < rows_hi;
          }
        }
        uint64_t mask = __ballot(hit);
        while (mask) {
          const int src = __ffsll((unsigned long long)mask) - 1;
          mask &= mask - 1;
          const int hr = __builtin_amdgcn_readlane(r, src);
          const int ht = __builtin_amdgcn_readlane(tok, src);
          const int hn = __builtin_amdgcn_readlane(node, src);
          const int rr = hr - m0;
          const int want_li = ht - c0, want_mt = rr >> 4, want_lq = (rr & 15) >> 2,
                    want_j = rr & 3;
          float v = 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (mt == want_mt && j == want_j) v = acc[mt][j];
          if (li == want_li && lq == want_lq) p.child_logit[hn] = v;
        }
      }
      __syncthreads();
      // one record per (row, column block): merge the 8 waves in order
      for (int rr = threadIdx.x; rr < 16 * MT; rr += blockDim.x) {
        const int r = m0 + rr;
        if (r >= p.M) continue;
        float m = kNegInf, sv = 0.f, wv = 0.f;
        int a = 0x7fffffff;
        for (int w = 0; w < WV; ++w)
          rec_merge(m, sv, wv, a, stat[w][rr][0], stat[w][rr][1], stat[w][rr][2],
                    __float_as_int(stat[w][rr][3]), p.inv_tau);
        float* rec = p.part + ((size_t)r * gridDim.x + g) * 4;
        rec[0] = m;
        rec[1] = sv;
        rec[2] = wv;
        rec[3] = __int_as_float(a);
      }
    }
  }
}

// QKV epilogue: sum the KS partials of (row r, column pair i, i+Dh/2) in
// order, rotate q and k by the RoPE angle of the row's position (reduced
// to one turn in double precision), round, scatter to [M][H][Dh].
// grid = (M, 3H), block = Dh/2 threads.
template <class ET>
__global__ void qkv_epilogue_kernel(GemmParams p, int KS) {
  using S = typename ET::storage;
  const int r = blockIdx.x, hp = blockIdx.y, i = threadIdx.x;
  const int Dh = p.Dh, half = Dh / 2, H = p.H;
  const int which = hp / H, h = hp - which * H;
  const int c1 = hp * Dh + i, c2 = c1 + half;
  float x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < KS; ++s) {
    const float* part = p.part + ((size_t)s * p.M + r) * p.N;
    x1 += part[c1];
    x2 += part[c2];
  }
  if (which < 2) {
    const double inv_freq = exp(-(2.0 * i / Dh) * p.log_theta);
    const double turns = (double)p.pos[r] * inv_freq * 0.15915494309189535;   // 1/(2 pi)
    const float ang = (float)((turns - rint(turns)) * 6.283185307179586);
    float sn, cs;
    __sincosf(ang, &sn, &cs);
    const float y1 = x1 * cs - x2 * sn;
    const float y2 = x2 * cs + x1 * sn;
    x1 = y1;
    x2 = y2;
  }
  S* dst = reinterpret_cast<S*>(which == 0 ? p.q_out : (which == 1 ? p.k_out : p.v_out));
  S* o = dst + ((size_t)r * H + h) * Dh + i;
  o[0] = ET::from_float(x1);
  o[half] = ET::from_float(x2);
}

// Output-projection epilogue: y = E[token] + sum of partials, fp32 and
// storage type. grid = (M, ceil(N/256)), block 256.
template <class ET>
__global__ void oproj_epilogue_kernel(GemmParams p, int KS) {
  using S = typename ET::storage;
  const int r = blockIdx.x, n = blockIdx.y * 256 + threadIdx.x;
  if (n >= p.N) return;
  float acc = 0.f;
  for (int s = 0; s < KS; ++s) acc += p.part[((size_t)s * p.M + r) * p.N + n];
  const S* x = reinterpret_cast<const S*>(p.E) +
               (size_t)min(max(p.tokens[r], 0), p.a_nrows - 1) * p.N;
  const float y = ET::load1(x + n) + acc;
  p.y_out[(size_t)r * p.N + n] = y;
  reinterpret_cast<S*>(p.y_elem)[(size_t)r * p.N + n] = ET::from_float(y);
}

__global__ __launch_bounds__(64) void row_stats_merge_kernel(const float* __restrict__ part,
                                                             int G, float inv_tau,
                                                             float* __restrict__ row_stats,
                                                             int* __restrict__ row_argmax) {
  const int r = blockIdx.x, lane = threadIdx.x;
  float m = kNegInf, s = 0.f, w = 0.f;
  int a = 0x7fffffff;
  for (int g = lane; g < G; g += 64) {
    const float* rec = part + ((size_t)r * G + g) * 4;
    rec_merge(m, s, w, a, rec[0], rec[1], rec[2], __float_as_int(rec[3]), inv_tau);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off), w2 = __shfl_xor(w, off);
    const int a2 = __shfl_xor(a, off);
    rec_merge(m, s, w, a, m2, s2, w2, a2, inv_tau);
  }
  if (lane == 0) {
    row_stats[(size_t)r * 3 + 0] = m;
    row_stats[(size_t)r * 3 + 1] = s;
    row_stats[(size_t)r * 3 + 2] = w;
    row_argmax[r] = a;
  }
}

template <class ET, bool LM>
hipError_t launch_main(const GemmParams& p, int groups, int KS, hipStream_t st) {
  const int mt_needed = (p.M + 15) / 16;
  dim3 grid(groups, KS), block(64 * kGemmWaves);
  // stages: as many as fit in LDS next to the A tiles
  if (mt_needed <= 3)
    hipLaunchKernelGGL((node_gemm_kernel<ET, 3, LM ? 6 : 7, LM>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((node_gemm_kernel<ET, 9, 4, LM>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

int lm_head_blocks(int N) { return (N + kGemmCols - 1) / kGemmCols; }

// Slices of K so that the grid has at least ~512 workgroups while every
// wave keeps at least one k-block per slice.
int gemm_splits(int N, int K, bool f32) {
  static const int min_wgs = [] {
    const char* s = getenv("MEDUSA_GEMM_MIN_WGS");
    const int v = s && *s ? atoi(s) : 384;
    return v < 1 ? 1 : (v > 4096 ? 4096 : v);
  }();
  const int groups = (N + kGemmCols - 1) / kGemmCols;
  const int nkb = K / (f32 ? 32 : 64);
  int ks = 1;
  while (groups * ks < min_wgs && ks * 2 * 4 <= nkb && ks < 32) ks *= 2;
  return ks;
}

hipError_t launch_qkv(const GemmParams& p, hipStream_t st) {
  const int KS = gemm_splits(p.N, p.K, p.f32);
  const int groups = (p.N + kGemmCols - 1) / kGemmCols;
  hipError_t e = p.f32 ? launch_main<F32, false>(p, groups, KS, st)
                       : launch_main<BF16, false>(p, groups, KS, st);
  if (e != hipSuccess) return e;
  dim3 grid(p.M, 3 * p.H);
  if (p.f32)
    hipLaunchKernelGGL(qkv_epilogue_kernel<F32>, grid, dim3(p.Dh / 2), 0, st, p, KS);
  else
    hipLaunchKernelGGL(qkv_epilogue_kernel<BF16>, grid, dim3(p.Dh / 2), 0, st, p, KS);
  return hipGetLastError();
}

hipError_t launch_oproj(const GemmParams& p, hipStream_t st) {
  const int KS = gemm_splits(p.N, p.K, p.f32);
  const int groups = (p.N + kGemmCols - 1) / kGemmCols;
  hipError_t e = p.f32 ? launch_main<F32, false>(p, groups, KS, st)
                       : launch_main<BF16, false>(p, groups, KS, st);
  if (e != hipSuccess) return e;
  dim3 grid(p.M, (p.N + 255) / 256);
  if (p.f32)
    hipLaunchKernelGGL(oproj_epilogue_kernel<F32>, grid, dim3(256), 0, st, p, KS);
  else
    hipLaunchKernelGGL(oproj_epilogue_kernel<BF16>, grid, dim3(256), 0, st, p, KS);
  return hipGetLastError();
}

hipError_t launch_lm_head(const GemmParams& p, float* row_stats, int* row_argmax,
                          hipStream_t st) {
  const int groups = lm_head_blocks(p.N);
  hipError_t e = p.f32 ? launch_main<F32, true>(p, groups, 1, st)
                       : launch_main<BF16, true>(p, groups, 1, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_stats_merge_kernel, dim3(p.M), dim3(64), 0, st, p.part, groups,
                     p.inv_tau, row_stats, row_argmax);
  return hipGetLastError();
}

}  // namespace medusa
