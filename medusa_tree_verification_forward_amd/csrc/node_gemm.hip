// Skinny node GEMMs of the verify pass on gfx950 MFMA:
//   C[M][N] = A[M][K] * W[N][K]^T,  M = B*T tree rows (tens to a few hundred),
//   N = 3d (QKV), d (output projection) or V (verification LM head).
//
// The weights stream from HBM once; A (a few hundred KB) stays in L2. A
// workgroup owns 16*NT output columns and all M rows (in passes of 16*MT
// rows); its four waves split K (chunk c goes to wave c mod 4, so together
// they read 4 consecutive chunks of every weight row) and are summed in a
// fixed order through LDS. Each lane loads 16 bytes of a weight row and 16
// bytes of an A row per chunk: that is one v_mfma_f32_16x16x32_bf16 per
// (m-tile, n-tile), or four v_mfma_f32_16x16x4_f32 for fp32 storage (the k
// index inside a chunk is permuted identically for both operands, which does
// not change the sum).
//
// Epilogues:
//   QKV  : RoPE on q and k (pairs i, i+Dh/2; angle pos * theta^(-2i/Dh)),
//          rounding to the storage type, scatter to [B][T][H][Dh].
//   OPROJ: y = x + acc with x = E[token], written as fp32 and as storage type.
//   LM   : per row and column block, (max, argmax, S, W) at temperature tau
//          with S = sum e^{(l-m)/tau}, W = sum e^{(l-m)/tau} (l-m)/tau; the
//          logit of every tree node's token under its parent's row; optional
//          full logits. A merge kernel combines the column blocks.
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

template <class ET, int MT, int NT, int EPI>
__global__ __launch_bounds__(256) void node_gemm_kernel(GemmParams p) {
  using S = typename ET::storage;
  constexpr int PV = ET::kPerVec;   // elements per 16-byte vector
  constexpr int KC = 4 * PV;        // k elements per chunk
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int g = blockIdx.x;
  const S* __restrict__ A = reinterpret_cast<const S*>(p.A);
  const S* __restrict__ W = reinterpret_cast<const S*>(p.W);

  // ---- columns of this workgroup ----
  int col[NT];
  int n0 = 0;
  if (EPI == EPI_QKV) {
    // 32 RoPE pairs of one (q|k|v, head) block: tiles 0,1 low half, 2,3 high
    const int half = p.Dh / 2;
    const int per = half / 32;
    const int hp = g / per, i0 = (g % per) * 32;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      col[nt] = hp * p.Dh + (nt >= 2 ? half : 0) + i0 + 16 * (nt & 1) + li;
  } else {
    n0 = g * 16 * NT;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) col[nt] = n0 + 16 * nt + li;
  }
  const S* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wrow[nt] = W + (size_t)min(col[nt], p.N - 1) * p.K + PV * lq;

  __shared__ float red[3][MT][64][4];
  __shared__ float rope_cs[EPI == EPI_QKV ? 16 * MT : 1][32][2];

  const int nch = p.K / KC;
  for (int m0 = 0; m0 < p.M; m0 += 16 * MT) {
    // the previous pass's epilogue (wave 0) may still read rope_cs / red
    if (m0 > 0) __syncthreads();
    const S* arow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int r = min(m0 + 16 * mt + li, p.M - 1);
      const int src = p.a_rows ? min(max(p.a_rows[r], 0), p.a_nrows - 1) : r;
      arow[mt] = A + (size_t)src * p.lda + PV * lq;
    }
    floatx4_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wb[2][NT], ab[2][MT];
    auto load = [&](int c, u32x4_t(&w)[NT], u32x4_t(&a)[MT]) {
      const size_t off = (size_t)c * KC;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[nt] = load16_stream(wrow[nt] + off);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = load16(arow[mt] + off);
    };
    auto mma = [&](const u32x4_t(&w)[NT], const u32x4_t(&a)[MT]) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (PV == 8) {
            acc[mt][nt] = mfma16x16x32_bf16(a[mt], w[nt], acc[mt][nt]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[mt][nt] = mfma16x16x4_f32(__uint_as_float(a[mt][j]), __uint_as_float(w[nt][j]),
                                            acc[mt][nt]);
          }
        }
    };
    int c = wave;
    if (c < nch) load(c, wb[0], ab[0]);

    if (EPI == EPI_QKV) {
      // cos/sin of this block's 32 pair indices for the rows of the pass,
      // angle reduced to one turn in double precision
      const int half = p.Dh / 2;
      const int i0 = (g % (half / 32)) * 32;
      for (int e = threadIdx.x; e < 16 * MT * 32; e += 256) {
        const int rr = e >> 5, ii = e & 31;
        const int r = min(m0 + rr, p.M - 1);
        const double inv_freq = exp(-(2.0 * (i0 + ii) / p.Dh) * p.log_theta);
        const double turns = (double)p.pos[r] * inv_freq * 0.15915494309189535;  // 1/(2 pi)
        const float ang = (float)((turns - rint(turns)) * 6.283185307179586);
        float sn, cs;
        __sincosf(ang, &sn, &cs);
        rope_cs[rr][ii][0] = cs;
        rope_cs[rr][ii][1] = sn;
      }
    }

    for (; c < nch; c += 8) {
      if (c + 4 < nch) load(c + 4, wb[1], ab[1]);
      mma(wb[0], ab[0]);
      if (c + 4 >= nch) break;
      if (c + 8 < nch) load(c + 8, wb[0], ab[0]);
      mma(wb[1], ab[1]);
    }

    // ---- fixed-order sum of the four waves' partial tiles ----
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) red[wave - 1][mt][lane][j] = acc[mt][nt][j];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[mt][nt][j] = ((acc[mt][nt][j] + red[0][mt][lane][j]) + red[1][mt][lane][j]) +
                             red[2][mt][lane][j];
      }
      __syncthreads();
    }
    if (wave != 0) continue;

    // ---- epilogues (wave 0) ----
    if constexpr (EPI == EPI_QKV) {
      const int half = p.Dh / 2;
      const int hp = g / (half / 32);
      const int which = hp / p.H, h = hp - which * p.H;
      S* dst = reinterpret_cast<S*>(which == 0 ? p.q_out : (which == 1 ? p.k_out : p.v_out));
      const int i0 = (g % (half / 32)) * 32;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * mt + 4 * lq + j;
          const int r = m0 + rr;
          if (r >= p.M) continue;
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int ii = 16 * nt + li;
            float x1 = acc[mt][nt][j], x2 = acc[mt][nt + 2][j];
            if (which < 2) {
              const float cs = rope_cs[rr][ii][0], sn = rope_cs[rr][ii][1];
              const float y1 = x1 * cs - x2 * sn;
              const float y2 = x2 * cs + x1 * sn;
              x1 = y1;
              x2 = y2;
            }
            S* o = dst + (size_t)r * p.H * p.Dh + (size_t)h * p.Dh + i0 + ii;
            o[0] = ET::from_float(x1);
            o[half] = ET::from_float(x2);
          }
        }
    } else if constexpr (EPI == EPI_OPROJ) {
      const S* E = reinterpret_cast<const S*>(p.E);
      S* ye = reinterpret_cast<S*>(p.y_elem);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m0 + 16 * mt + 4 * lq + j;
          if (r >= p.M) continue;
          const S* x = E + (size_t)min(max(p.tokens[r], 0), p.a_nrows - 1) * p.N;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int n = col[nt];
            if (n >= p.N) continue;
            const float y = ET::load1(x + n) + acc[mt][nt][j];
            p.y_out[(size_t)r * p.N + n] = y;
            ye[(size_t)r * p.N + n] = ET::from_float(y);
          }
        }
    } else {   // EPI_LM
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m0 + 16 * mt + 4 * lq + j;
          // lane-local best over this lane's columns (increasing with nt)
          float bv = kNegInf;
          int bi = 0x7fffffff;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const float v = acc[mt][nt][j];
            if (col[nt] < p.N && v > bv) {
              bv = v;
              bi = col[nt];
            }
          }
          // (max, lowest argmax) over the 16 lanes sharing this row
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
          float s = 0.f, w = 0.f;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if (col[nt] < p.N) {
              const float z = (acc[mt][nt][j] - bv) * p.inv_tau;
              const float e = exp_e(z);
              s += e;
              w += e * z;
            }
          }
          s = row16_sum(s);
          w = row16_sum(w);
          if (li == 0 && r < p.M) {
            float* rec = p.part + ((size_t)r * gridDim.x + g) * 4;
            rec[0] = bv;
            rec[1] = s;
            rec[2] = w;
            rec[3] = __int_as_float(bi);
          }
          if (p.logits_out && r < p.M) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if (col[nt] < p.N) p.logits_out[(size_t)r * p.N + col[nt]] = acc[mt][nt][j];
          }
        }
      // logit of each tree node's token under its parent's row
      const int ncol = 16 * NT;
      const int rows_hi = min(p.M, m0 + 16 * MT);
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
            hit = tok >= n0 && tok < n0 + ncol && r >= m0 && r < rows_hi;
          }
        }
        uint64_t mask = __ballot(hit);
        while (mask) {
          const int src = __ffsll((unsigned long long)mask) - 1;
          mask &= mask - 1;
          const int hr = __builtin_amdgcn_readlane(r, src);
          const int ht = __builtin_amdgcn_readlane(tok, src);
          const int hn = __builtin_amdgcn_readlane(node, src);
          const int cc = ht - n0, rr = hr - m0;
          const int want_li = cc & 15, want_nt = cc >> 4;
          const int want_mt = rr >> 4, want_lq = (rr & 15) >> 2, want_j = rr & 3;
          float v = 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (mt == want_mt && nt == want_nt && j == want_j) v = acc[mt][nt][j];
          if (li == want_li && lq == want_lq) p.child_logit[hn] = v;
        }
      }
    }
  }
}

// Merge the column-block records of one row: (max, S, W, argmax).
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

template <class ET, int EPI>
hipError_t launch_gemm_et(const GemmParams& p, int mt_needed, hipStream_t st) {
  // QKV needs four column tiles (two RoPE halves); other epilogues pick the
  // tile count that gives the grid enough workgroups.
  dim3 block(256);
  if (EPI == EPI_QKV) {
    const int grid = 3 * p.H * (p.Dh / 64);
    if (mt_needed <= 3)
      hipLaunchKernelGGL((node_gemm_kernel<ET, 3, 4, EPI>), dim3(grid), block, 0, st, p);
    else
      hipLaunchKernelGGL((node_gemm_kernel<ET, 8, 4, EPI>), dim3(grid), block, 0, st, p);
  } else {
    const int nt = p.N / 64 >= 256 ? 4 : (p.N / 32 >= 256 ? 2 : 1);
    const int grid = (p.N + 16 * nt - 1) / (16 * nt);
#define GEMM_LAUNCH(MT_, NT_) \
  hipLaunchKernelGGL((node_gemm_kernel<ET, MT_, NT_, EPI>), dim3(grid), block, 0, st, p)
    if (mt_needed <= 3) {
      if (nt == 4) GEMM_LAUNCH(3, 4); else if (nt == 2) GEMM_LAUNCH(3, 2); else GEMM_LAUNCH(3, 1);
    } else {
      if (nt == 4) GEMM_LAUNCH(8, 4); else if (nt == 2) GEMM_LAUNCH(8, 2); else GEMM_LAUNCH(8, 1);
    }
#undef GEMM_LAUNCH
  }
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_gemm(const GemmParams& p, hipStream_t st) {
  const int mt_needed = (p.M + 15) / 16;
  return p.f32 ? launch_gemm_et<F32, EPI>(p, mt_needed, st)
               : launch_gemm_et<BF16, EPI>(p, mt_needed, st);
}

}  // namespace

int lm_head_blocks(int N) {
  const int nt = N / 64 >= 256 ? 4 : (N / 32 >= 256 ? 2 : 1);
  return (N + 16 * nt - 1) / (16 * nt);
}

hipError_t launch_qkv(const GemmParams& p, hipStream_t st) { return launch_gemm<EPI_QKV>(p, st); }
hipError_t launch_oproj(const GemmParams& p, hipStream_t st) {
  return launch_gemm<EPI_OPROJ>(p, st);
}
hipError_t launch_lm_head(const GemmParams& p, float* row_stats, int* row_argmax,
                          hipStream_t st) {
  hipError_t e = launch_gemm<EPI_LM>(p, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(row_stats_merge_kernel, dim3(p.M), dim3(64), 0, st, p.part,
                     lm_head_blocks(p.N), p.inv_tau, row_stats, row_argmax);
  return hipGetLastError();
}

}  // namespace medusa
