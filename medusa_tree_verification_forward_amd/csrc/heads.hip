// Medusa heads on gfx950 ("Medusa 深读", §3.1, head equation):
//   z_k = h + SiLU(W1_k h + b1_k),  l_k = W2_k z_k,  top-s of l_k,  lse of l_k.
//
// Both products are matrix-vector streams over bf16 (or fp32) weights, bound
// by HBM bandwidth. A wavefront owns up to 64 consecutive weight rows and
// streams them as 1 KB wave loads with a fixed number in flight (each lane
// reads 16 bytes of a row, consecutive lanes consecutive bytes), multiplies
// them with the activation held in LDS and finishes each row sum with a DPP
// reduction; lane l keeps row l's result. The W2 pass never writes the V
// logits unless asked: after its stream a wave takes the top-s of its rows
// (lanes 0..s-1, best first) and their softmax statistics, and a workgroup
// leaves one partial record per (sequence, head, row block). A small merge
// kernel reduces the records of one (sequence, head) in a fixed order.
#include <algorithm>
#include <type_traits>

#include "cdf.h"
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

constexpr int kHeadWaves = 4;   // waves per workgroup
constexpr int kRing = 8;        // weight loads in flight per wave

// Weight-row stream of one wave: rows [rb, rb + nrows) of W ([*][d], row-major),
// nrows <= 64. Step t is one 1 KB wave load: chunk sg of row r covers
// elements [sg*CW, sg*CW + CW) of the row (CW = 64 PV, lane l takes PV of
// them at sg*CW + PV*l); a row has SPR = ceil(d / CW) chunks. kRing loads
// are in flight; refills past the end re-read the last chunk (never used),
// so every step issues exactly one load and the pipeline depth is fixed.
// The activation xs (fp32 in LDS, NB vectors of stride ldx, zero past d)
// is read at the same positions; lanes past the end of a row read a valid
// weight and a zero activation.
//
// bf16 weights with one or two activation vectors take the dot products on
// the matrix cores: lane l gives its 8 weights as its B fragment and the 8
// activations they multiply as its A fragment of a v_mfma_f32_16x16x32_bf16,
// so the diagonal entry (n, n) of the product is the sum of the dot products
// of lanes n, n + 16, n + 32, n + 48, and the trace over a row's chunks is
// the row's dot product. The activation enters as two bf16 parts, x = hi +
// lo (hi = bf16(x), lo = bf16(x - hi), together within 2^-17 |x|), one
// product each; the vector ALUs then only keep the stream going.
template <class ET, int NB>
struct RowStream {
  using St = typename ET::storage;
  static constexpr int PV = ET::kPerVec;
  static constexpr int CW = 64 * PV;
  static constexpr bool kMfma = std::is_same<ET, BF16>::value && NB <= 2;
  using Acc = typename std::conditional<kMfma, floatx4_t, float>::type;
  const St* __restrict__ W;
  int rb, rstride, nrows, d, SPR, lane;
  int fr, fs;   // row / chunk of the next refill
  u32x4_t wr[kRing];

  __device__ __forceinline__ const St* chunk_ptr(int r, int sg) const {
    return W + (size_t)(rb + r * rstride) * d + min(sg * CW + PV * lane, d - PV);
  }
  __device__ __forceinline__ void refill(int j) {
    const bool past = fr >= nrows;
    wr[j] = load16_stream(chunk_ptr(past ? nrows - 1 : fr, past ? SPR - 1 : fs));
    if (++fs == SPR) {
      fs = 0;
      ++fr;
    }
  }
  // Issue the first kRing loads (a wave without rows reads row rb_ok, a
  // valid row, and never consumes the results).
  __device__ __forceinline__ void start(const St* W_, int rb_, int rstride_, int nrows_, int d_,
                                        int rb_ok) {
    W = W_;
    rstride = rstride_;
    rb = nrows_ > 0 ? rb_ : rb_ok;
    nrows = nrows_ > 0 ? nrows_ : 1;
    d = d_;
    SPR = (d + CW - 1) / CW;
    lane = threadIdx.x & 63;
    fr = 0;
    fs = 0;
#pragma unroll
    for (int j = 0; j < kRing; ++j) refill(j);
  }
  // Row value from the accumulated product: the sum of its diagonal, whose
  // entry (n, n) sits in lane 20 q + j (n = 4 q + j) as element j.
  __device__ __forceinline__ static float trace(const floatx4_t& c) {
    const int l = threadIdx.x & 63, dj = (l & 15) - 4 * (l >> 4);
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) v = dj == j ? c[j] : v;
    return wave_sum(v);
  }
  template <bool GUARD>
  __device__ __forceinline__ void step(int t, int j, int total, const float* xs, int ldx,
                                       Acc (&acc)[NB], float (&win)[NB], int& cr, int& cs) {
    if constexpr (kMfma) {
      if (!GUARD || t < total) {
        // activation parts: hi plane [NB][ldx] then lo plane, bf16
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs) + cs * CW + PV * lane;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(xh + b * ldx);
          const u32x4_t al = *reinterpret_cast<const u32x4_t*>(xh + (NB + b) * ldx);
          acc[b] = mfma16x16x32_bf16(ah, wr[j], acc[b]);
          acc[b] = mfma16x16x32_bf16(al, wr[j], acc[b]);
        }
        if (++cs == SPR) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float v = trace(acc[b]);
            win[b] = lane == cr ? v : win[b];
            acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
          }
          cs = 0;
          ++cr;
        }
      }
      if (!GUARD || t + kRing < total) refill(j);
    } else {
    if (!GUARD || t < total) {
      float wf[PV];
      ET::widen(wr[j], wf);
      const float* xp = xs + cs * CW + PV * lane;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float a = acc[b];
#pragma unroll
        for (int e = 0; e < PV; e += 4) {
          const floatx4_t xv = *reinterpret_cast<const floatx4_t*>(xp + b * ldx + e);
          a = fmaf(wf[e], xv[0], a);
          a = fmaf(wf[e + 1], xv[1], a);
          a = fmaf(wf[e + 2], xv[2], a);
          a = fmaf(wf[e + 3], xv[3], a);
        }
        acc[b] = a;
      }
      if (++cs == SPR) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float v = wave_sum(acc[b]);
          win[b] = lane == cr ? v : win[b];
          acc[b] = 0.f;
        }
        cs = 0;
        ++cr;
      }
    }
    if (!GUARD || t + kRing < total) refill(j);
    }
  }
  // Consume the stream; lane l of win[b] receives row rb + l's dot product
  // with activation b (lanes >= nrows keep their old value). The steady
  // loop has every step and refill in range, so it keeps exactly kRing
  // loads in flight; the last two rounds check their bounds.
  __device__ __forceinline__ void run(const float* xs, int ldx, float (&win)[NB]) {
    const int total = nrows * SPR;
    Acc acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = Acc{};
    int cr = 0, cs = 0;   // row / chunk being consumed
    int t0 = 0;
    for (; t0 + 2 * kRing <= total; t0 += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) step<false>(t0 + j, j, total, xs, ldx, acc, win, cr, cs);
    }
    for (; t0 < total; t0 += kRing) {
#pragma unroll
      for (int j = 0; j < kRing; ++j) step<true>(t0 + j, j, total, xs, ldx, acc, win, cr, cs);
    }
  }
};

// Row stream for rows of exactly SPR chunks (d a multiple of CW): the ring
// holds one row, so chunk s of the next row refills slot s as soon as chunk
// s of the current row is consumed; addresses advance by one add per row and
// the row's dot product is reduced once, after its last chunk. Same contract
// as RowStream (lane l of win[b] receives the wave's row l).
template <class ET, int NB, int SPR>
struct RowStreamRows {
  using St = typename ET::storage;
  static constexpr int PV = ET::kPerVec;
  static constexpr int CW = 64 * PV;
  static constexpr bool kMfma = RowStream<ET, NB>::kMfma;
  using Acc = typename RowStream<ET, NB>::Acc;
  const St* __restrict__ p;   // this lane's piece of the row being consumed
  size_t rstep;               // elements from one of the wave's rows to the next
  int nrows;
  u32x4_t wr[SPR];

  __device__ __forceinline__ void start(const St* W, int rb, int rstride, int nrows_, int d,
                                        int /*rb_ok*/) {
    nrows = nrows_;
    p = W + (size_t)rb * d + PV * (threadIdx.x & 63);
    rstep = (size_t)rstride * d;
    if (nrows > 0) {
#pragma unroll
      for (int s = 0; s < SPR; ++s) wr[s] = load16_stream(p + s * CW);
    }
  }
  template <bool REFILL>
  __device__ __forceinline__ void row(int i, const float* xs, int ldx, float (&win)[NB]) {
    const int lane = threadIdx.x & 63;
    const St* pn = p + rstep;
    Acc acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = Acc{};
#pragma unroll
    for (int s = 0; s < SPR; ++s) {
      if constexpr (kMfma) {
        const uint16_t* xh = reinterpret_cast<const uint16_t*>(xs) + s * CW + PV * lane;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const u32x4_t ah = *reinterpret_cast<const u32x4_t*>(xh + b * ldx);
          const u32x4_t al = *reinterpret_cast<const u32x4_t*>(xh + (NB + b) * ldx);
          acc[b] = mfma16x16x32_bf16(ah, wr[s], acc[b]);
          acc[b] = mfma16x16x32_bf16(al, wr[s], acc[b]);
        }
      } else {
        float wf[PV];
        ET::widen(wr[s], wf);
        const float* xp = xs + s * CW + PV * lane;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float a = acc[b];
#pragma unroll
          for (int e = 0; e < PV; e += 4) {
            const floatx4_t xv = *reinterpret_cast<const floatx4_t*>(xp + b * ldx + e);
            a = fmaf(wf[e], xv[0], a);
            a = fmaf(wf[e + 1], xv[1], a);
            a = fmaf(wf[e + 2], xv[2], a);
            a = fmaf(wf[e + 3], xv[3], a);
          }
          acc[b] = a;
        }
      }
      if (REFILL) wr[s] = load16_stream(pn + s * CW);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v;
      if constexpr (kMfma)
        v = RowStream<ET, NB>::trace(acc[b]);
      else
        v = wave_sum(acc[b]);
      win[b] = lane == i ? v : win[b];
    }
    p = pn;
  }
  __device__ __forceinline__ void run(const float* xs, int ldx, float (&win)[NB]) {
    int i = 0;
    for (; i + 1 < nrows; ++i) row<true>(i, xs, ldx, win);
    if (i < nrows) row<false>(i, xs, ldx, win);
  }
};

// Stage NB activation vectors (src + b * src_stride, d floats each) into LDS
// as xs[b][0 .. ldx), zero past d. The first round of activation loads is
// issued before the weight stream starts, so it is not queued behind it.
// Ends with a barrier that leaves the weight loads in flight.
template <class ET, int NB, class Stream>
__device__ __forceinline__ void stage_and_start(Stream& rs, const float* __restrict__ src,
                                                size_t src_stride, int nb, int d, float* xs,
                                                int ldx, const typename ET::storage* W, int rb,
                                                int rstride, int nrows, int rb_ok) {
  constexpr int XR = 8;   // float4 loads per thread per round
  const int n4 = NB * ldx / 4;
  auto load_round = [&](int base, floatx4_t (&v)[XR]) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int i4 = min(base + u * (int)blockDim.x + (int)threadIdx.x, n4 - 1);
      const int b = (4 * i4) / ldx, j = 4 * i4 - b * ldx;
      const int bb = min(b, nb - 1), jj = min(j, d - 4);
      v[u] = *reinterpret_cast<const floatx4_t*>(src + bb * src_stride + jj);
      if (b >= nb || j >= d) v[u] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_round = [&](int base, const floatx4_t (&v)[XR]) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int i4 = base + u * (int)blockDim.x + (int)threadIdx.x;
      if (i4 >= n4) continue;
      if constexpr (Stream::kMfma) {
        // bf16 parts: hi = bf16(x), lo = bf16(x - hi)
        uint32_t hb[4], lb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hb[e] = f32_to_bf16_bits(v[u][e]);
          lb[e] = f32_to_bf16_bits(v[u][e] - __uint_as_float(hb[e] << 16));
        }
        uint16_t* xh = reinterpret_cast<uint16_t*>(xs);
        *reinterpret_cast<uint2*>(xh + 4 * i4) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        *reinterpret_cast<uint2*>(xh + NB * ldx + 4 * i4) =
            make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
      } else {
        *reinterpret_cast<floatx4_t*>(xs + 4 * i4) = v[u];
      }
    }
  };
  floatx4_t v[XR];
  load_round(0, v);
  rs.start(W, rb, rstride, nrows, d, rb_ok);
  store_round(0, v);
  const int per_round = XR * (int)blockDim.x;
  for (int base = per_round; base < n4; base += per_round) {
    load_round(base, v);
    store_round(base, v);
  }
  lds_barrier();
}

// Rows of wave wi out of nw waves streaming `total` rows, at most rpw each,
// interleaved (rows wi, wi + nw, wi + 2 nw, ...), so the waves of a launch
// advance through memory side by side (blocks of consecutive rows a wave
// measured slower).
__device__ __forceinline__ void wave_rows(int wi, int nw, int rpw, int total, int& rb,
                                          int& rstride, int& nrows) {
  rb = wi;
  rstride = nw;
  nrows = wi < total ? min(rpw, (total - wi + nw - 1) / nw) : 0;
}

// ---------------------------------------------------------------------------
// z[b][k][i] = h[b][i] + silu(sum_j W1[k][i][j] h[b][j] + b1[k][i])
// Rows are numbered k*d + i over all heads; wave w of workgroup g streams
// rows [(g*4 + w) * rpw, ... + rpw).
template <class ET, int NB, int SPR>
using HeadStream =
    typename std::conditional<SPR == 0, RowStream<ET, NB>, RowStreamRows<ET, NB, SPR>>::type;

// Resident workgroups per compute unit the head kernels are compiled for:
// four (128 registers) where the stream fits them, fewer where a whole-row
// ring of 10 or 16 chunks, or two activation vectors, needs more registers —
// at four those spilled (two vectors at d = 4096: a 770 us step at batch 2
// against 420; one vector at d = 5120: 597 against 556 us).
template <int NB, int SPR>
constexpr int head_min_blocks() {
  return (SPR == 0 || (NB == 1 && SPR <= 8)) ? 4 : ((NB == 1 && SPR <= 10) ? 3 : 2);
}

template <class ET, int NB, int SPR>
__global__ __launch_bounds__(kHeadWaves * 64, (head_min_blocks<NB, SPR>())) void heads_w1_kernel(
    const float* __restrict__ h, int B, int b0, int K, int d,
    const typename ET::storage* __restrict__ W1, const float* __restrict__ b1,
    float* __restrict__ z, int rpw) {
  extern __shared__ float xs[];   // [NB][ldx]
  constexpr int CW = RowStream<ET, NB>::CW;
  const int ldx = (d + CW - 1) / CW * CW;
  const int nb = min(NB, B - b0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int total = K * d;
  int rb, rstride, nrows;
  wave_rows(blockIdx.x * kHeadWaves + wave, gridDim.x * kHeadWaves, rpw, total,
            rb, rstride, nrows);
  // the residual h of the lane's row, read before the stream
  float hres[NB];
  {
    const int row = min(rb + min(lane, max(nrows - 1, 0)) * rstride, total - 1);
    const int i = row - (row / d) * d;
#pragma unroll
    for (int b = 0; b < NB; ++b) hres[b] = h[(size_t)(b0 + min(b, nb - 1)) * d + i];
  }
  HeadStream<ET, NB, SPR> rs;
  stage_and_start<ET, NB>(rs, h + (size_t)b0 * d, d, nb, d, xs, ldx, W1, rb, rstride, nrows, 0);
  if (nrows == 0) return;
  float win[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) win[b] = 0.f;
  rs.run(xs, ldx, win);
  if (lane < nrows) {
    const int row = rb + lane * rstride;   // row = k*d + i
    const int k = row / d, i = row - k * d;
    const float bias = b1 ? b1[row] : 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < nb) {
        const float u = win[b] + bias;
        const float sig = 1.f / (1.f + exp_e(-u));
        z[((size_t)(b0 + b) * K + k) * d + i] = hres[b] + u * sig;
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

// Per-wave top-S and softmax statistics of the rows in win (lane l: row
// rb + l rstride, valid below nrows), merged over the workgroup's waves
// through LDS (xs, at least kHeadWaves NB (2 MAXS_LDS + 2) floats; the
// caller's last use of it must be done) into one partial record per vector.
template <int NB>
__device__ __forceinline__ void w2_finish(const float (&win)[NB], int nb, int b0, int K, int k,
                                          int V, int G, int g, int rb, int rstride, int nrows,
                                          int S, float* xs, float* __restrict__ head_logits,
                                          float* __restrict__ part_val, int* __restrict__ part_id,
                                          float* __restrict__ part_m, float* __restrict__ part_s) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float tv[NB], m[NB], s[NB];
  int ti[NB];
  const bool valid = lane < nrows;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float v = valid ? win[b] : kNegInf;
    if (head_logits && b < nb && valid)
      head_logits[((size_t)(b0 + b) * K + k) * V + rb + lane * rstride] = v;
    // statistics of this wave's rows
    const float mx = wave_max(v);
    m[b] = mx;
    s[b] = mx == kNegInf ? 0.f : wave_sum(valid ? exp_e(v - mx) : 0.f);
    // top-S of this wave's rows, best first in lanes 0..S-1
    float cv = v;
    int ci = valid ? rb + lane * rstride : kNoId;
    tv[b] = kNegInf;
    ti[b] = kNoId;
    for (int r = 0; r < S; ++r) {
      float bv = cv;
      int bi = ci;
      wave_best(bv, bi);
      if (lane == r) {
        tv[b] = bv;
        ti[b] = bi;
      }
      if (ci == bi) {
        cv = kNegInf;
        ci = kNoId;
      }
    }
  }
  // merge the waves of this block through LDS (after the activation is no
  // longer needed)
  __syncthreads();
  float* lv = xs;                                        // [WAVES][NB][S]
  int* li = reinterpret_cast<int*>(xs + kHeadWaves * NB * MAXS_LDS);
  float* lm = xs + 2 * kHeadWaves * NB * MAXS_LDS;       // [WAVES][NB]
  float* ls = lm + kHeadWaves * NB;
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
    for (int w = 1; w < kHeadWaves; ++w) {
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
// l = W2_k z_k for the rows of one block; top-S and (max, sum exp) of them.
// grid = (G, K): wave w of block g of head k streams rows
// [(g*4 + w) * rpw, ... + rpw) of head k.
// Partial records: part_val/part_id [B][K][G][S], part_m/part_s [B][K][G].
template <class ET, int NB, int SPR>
__global__ __launch_bounds__(kHeadWaves * 64, (head_min_blocks<NB, SPR>())) void heads_w2_kernel(
    const float* __restrict__ z, int B, int b0, int K, int V, int d,
    const typename ET::storage* __restrict__ W2, int rpw, int S,
    float* __restrict__ head_logits, float* __restrict__ part_val, int* __restrict__ part_id,
    float* __restrict__ part_m, float* __restrict__ part_s, int G) {
  extern __shared__ float xs[];   // [NB][ldx], then per-wave list exchange
  constexpr int CW = RowStream<ET, NB>::CW;
  const int ldx = (d + CW - 1) / CW * CW;
  const int k = blockIdx.y, g = blockIdx.x;
  const int nb = min(NB, B - b0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int rb, rstride, nrows;
  wave_rows(g * kHeadWaves + wave, gridDim.x * kHeadWaves, rpw, V, rb, rstride,
            nrows);
  HeadStream<ET, NB, SPR> rs;
  stage_and_start<ET, NB>(rs, z + ((size_t)b0 * K + k) * d, (size_t)K * d, nb, d, xs, ldx,
                          W2 + (size_t)k * V * d, rb, rstride, nrows, 0);
  float win[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) win[b] = kNegInf;
  if (nrows > 0) rs.run(xs, ldx, win);

  w2_finish<NB>(win, nb, b0, K, k, V, G, g, rb, rstride, nrows, S, xs, head_logits, part_val,
                part_id, part_m, part_s);
}

// ---------------------------------------------------------------------------
// Batched head streams: 3 to 8 activation vectors over bf16 weights.
//
// With several vectors the weights are multiplied in the plain MFMA product
// layout. Weight tile (rows r_0..r_15, column block t) is 16 rows by 32
// columns: lane (j, q) = (l % 16, l / 16) takes the 16 bytes of row r_j at
// column 32 t + 8 q as its B fragment (64 contiguous bytes of each row). The
// A fragment of column block t holds the same columns for 16 operand rows,
// row 2 s + p being part p (bf16 hi, lo as above) of vector s, so one
// v_mfma_f32_16x16x32_bf16 per 1 KB tile accumulates the partial sums of
// every vector for 16 weight rows. Entry (i, j) of the product sits in lane
// j + 16 (i / 4) as element i % 4: lane (j, q) holds vectors 2 q (elements
// 0 + 1) and 2 q + 1 (elements 2 + 3) of row r_j. The A fragments of a
// vector set (32 d bytes) are built once and read from global memory, where
// they stay in L2, so the LDS holds nothing per vector and several
// workgroups share a compute unit.
constexpr int kTileVecs = 8;   // vectors per batched pass

__device__ __forceinline__ uint32_t bf16_part_bits(float x, int p) {
  const uint32_t hi = f32_to_bf16_bits(x);
  return p ? f32_to_bf16_bits(x - __uint_as_float(hi << 16)) : hi;
}

// A fragments of nb <= 8 fp32 vectors (src + s * stride, d values each; zero
// rows for s >= nb): frag[64 t + l] is part l % 2 of vector (l % 16) / 2 at
// columns 32 t + 8 (l / 16) .. + 7. One thread per fragment.
__global__ __launch_bounds__(256) void act_frag_kernel(const float* __restrict__ src,
                                                       size_t stride, int nb, int d,
                                                       u32x4_t* __restrict__ frag) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= (d / 32) * 64) return;
  const int t = idx >> 6, l = idx & 63, i = l & 15, v = i >> 1;
  u32x4_t out = {0u, 0u, 0u, 0u};
  if (v < nb) {
    const float* p = src + (size_t)v * stride + 32 * t + 8 * (l >> 4);
    const floatx4_t x0 = *reinterpret_cast<const floatx4_t*>(p);
    const floatx4_t x1 = *reinterpret_cast<const floatx4_t*>(p + 4);
    const int part = i & 1;
    out[0] = bf16_part_bits(x0[0], part) | (bf16_part_bits(x0[1], part) << 16);
    out[1] = bf16_part_bits(x0[2], part) | (bf16_part_bits(x0[3], part) << 16);
    out[2] = bf16_part_bits(x1[0], part) | (bf16_part_bits(x1[1], part) << 16);
    out[3] = bf16_part_bits(x1[2], part) | (bf16_part_bits(x1[3], part) << 16);
  }
  frag[idx] = out;
}

// NG tile rows of one wave over nt column blocks, DS blocks (NG DS tiles and
// DS A fragments) in flight: wp[g] points at the lane's 8 weights of the
// first block in group g, ap at its A fragment of the first block. Requires
// nt a positive multiple of DS. STREAM: the weight loads carry the
// non-temporal hint -- for packed weights, whose tiles are whole 1 KB runs
// (batch of 8: W2 236 -> 210 us, W1 34.8 -> 30.3). From a row-major W the
// loads are plain (cached): there a tile reads half of each 128-byte line and
// the next block the other half, and with the hint the line was often gone
// by then (37% more HBM traffic).
// `step`: elements from one column block of a lane's row piece to the next
// (32 in a row-major W, ntiles * 512 in a packed one).
template <int NG, int DS, bool STREAM = false>
__device__ __forceinline__ void tile_stream(const uint16_t* const (&wp)[NG], size_t step,
                                            const u32x4_t* __restrict__ ap, int nt,
                                            floatx4_t (&acc)[NG]) {
  auto wload = [](const uint16_t* q) { return STREAM ? load16_stream(q) : load16(q); };
  u32x4_t wr[DS][NG], ar[DS];
#pragma unroll
  for (int j = 0; j < DS; ++j) {
#pragma unroll
    for (int g = 0; g < NG; ++g) wr[j][g] = wload(wp[g] + step * j);
    ar[j] = load16(ap + 64 * j);
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  int t = 0;
  for (; t + DS < nt; t += DS) {
#pragma unroll
    for (int j = 0; j < DS; ++j) {
      const int tn = t + DS + j;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        acc[g] = mfma16x16x32_bf16(ar[j], wr[j][g], acc[g]);
        wr[j][g] = wload(wp[g] + step * tn);
      }
      ar[j] = load16(ap + 64 * tn);
    }
  }
#pragma unroll
  for (int j = 0; j < DS; ++j)
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = mfma16x16x32_bf16(ar[j], wr[j][g], acc[g]);
}

// W1 over 3..8 vectors: z[b][k][i] as heads_w1_kernel computes it, plus the
// A fragments of z for the W2 pass (zfrag[k], layout as act_frag_kernel's).
// A workgroup takes 16 (4 / KS) consecutive rows of the K d rows: wave w
// streams rows 16 (w / KS) .. + 15 over column blocks of part w % KS of d,
// and the KS partial tiles are summed through LDS in part order.
template <int KS, int DS, bool PACKED>
__global__ __launch_bounds__(kHeadWaves * 64, 4) void heads_w1_tile_kernel(
    const float* __restrict__ h, int B, int b0, int K, int d, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W1p, const float* __restrict__ b1,
    const u32x4_t* __restrict__ hfrag, float* __restrict__ z,
    uint16_t* __restrict__ zfrag) {
  constexpr int RS = kHeadWaves / KS;   // row sets of 16 per workgroup
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int set = wave / KS, part = wave % KS;
  const int nb = min(kTileVecs, B - b0);
  const int total = K * d;
  const int row = min((blockIdx.x * RS + set) * 16 + j, total - 1);
  const int k = row / d, i = row - k * d;
  const int nblk = d / 32, per = nblk / KS;
  // residuals h[b0 + 2 q + e][i] and the bias, read before the stream
  float hres[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) hres[e] = h[(size_t)(b0 + min(2 * q + e, nb - 1)) * d + i];
  const float bias = b1 ? b1[row] : 0.f;
  // row-major W1, or W1 packed as one [K d][d] matrix (tile (nt, kt) at
  // kt * ntiles + nt, lane (j, q)'s piece = row j, columns 32 kt + 8 q ..)
  const uint16_t* wp[1];
  size_t step = 32;
  if constexpr (PACKED) {
    const int ntiles = total / 16;
    const int nt = min((int)(blockIdx.x * RS + set), ntiles - 1);
    step = (size_t)ntiles * 512;
    wp[0] = W1p + (((size_t)per * part * ntiles + nt) * 64 + lane) * 8;
  } else {
    wp[0] = W1 + (size_t)row * d + 32 * per * part + 8 * q;
  }
  floatx4_t acc[1];
  tile_stream<1, DS, PACKED>(wp, step, hfrag + (size_t)per * part * 64 + lane, per, acc);
  if constexpr (KS > 1) {
    __shared__ floatx4_t red[RS][KS - 1][64];
    if (part > 0) red[set][part - 1][lane] = acc[0];
    __syncthreads();
    if (part > 0) return;
#pragma unroll
    for (int u = 0; u < KS - 1; ++u) acc[0] += red[set][u][lane];
  }
  if ((blockIdx.x * RS + set) * 16 + j >= total) return;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int v = 2 * q + e;
    float zv = 0.f;
    if (v < nb) {
      const float u = acc[0][2 * e] + acc[0][2 * e + 1] + bias;
      zv = hres[e] + u * (1.f / (1.f + exp_e(-u)));
      z[((size_t)(b0 + v) * K + k) * d + i] = zv;
    }
    // operand rows 2 v (hi) and 2 v + 1 (lo) of column i in head k's fragments
    uint16_t* f = zfrag + ((((size_t)k * nblk + (i >> 5)) * 64 + 16 * ((i & 31) >> 3) + 2 * v) * 8 +
                           (i & 7));
    f[0] = (uint16_t)bf16_part_bits(zv, 0);
    f[8] = (uint16_t)bf16_part_bits(zv, 1);
  }
}

// W2 over 3..8 vectors: the records of heads_w2_kernel. Wave w of block g of
// head k streams 16 NG consecutive rows as NG tile rows over all of d (the
// rows of a wave stay within a few pages; rows interleaved over the waves
// spread every wave over the whole head); the values are moved to lane = row
// (lane 16 g + j takes row j of tile row g) for the shared top-S epilogue.
// three resident workgroups a compute unit: registers for 8 column blocks in flight
constexpr int kW2TileMinBlocks = 3;
template <int NG, int DS, bool PACKED>
__global__ __launch_bounds__(kHeadWaves * 64, kW2TileMinBlocks) void heads_w2_tile_kernel(
    int B, int b0, int K, int V, int d, const uint16_t* __restrict__ W2,
    const uint16_t* __restrict__ W2p, const u32x4_t* __restrict__ zfrag, int S,
    float* __restrict__ head_logits,
    float* __restrict__ part_val, int* __restrict__ part_id, float* __restrict__ part_m,
    float* __restrict__ part_s, int G) {
  __shared__ float xs[kHeadWaves * kTileVecs * (2 * MAXS_LDS + 2)];
  const int k = blockIdx.y, g = blockIdx.x;
  const int nb = min(kTileVecs, B - b0);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  // a wave's 16 NG rows are consecutive (interleaved rows measured slower here)
  const int rstride = 1, rb = (g * kHeadWaves + wave) * 16 * NG;
  const int nrows = max(0, min(16 * NG, V - rb));
  float win[kTileVecs];
#pragma unroll
  for (int b = 0; b < kTileVecs; ++b) win[b] = kNegInf;
  if (nrows > 0) {
    const uint16_t* wp[NG];
    size_t step = 32;
    if constexpr (PACKED) {
      // packed tiles (16 rows x 32 columns, 64 lane pieces, k-major within
      // each head): lane (j, q)'s piece of tile (row block, column block t)
      // is row j, columns 32 t + 8 q .. + 7 -- the same fragment
      const int ntiles = (V + 15) / 16;
      const uint16_t* head = W2p + (size_t)k * ntiles * 16 * d;
      step = (size_t)ntiles * 512;
#pragma unroll
      for (int tg = 0; tg < NG; ++tg)
        wp[tg] = head + ((size_t)min(rb / 16 + tg, ntiles - 1) * 64 + lane) * 8;
    } else {
#pragma unroll
      for (int tg = 0; tg < NG; ++tg)
        wp[tg] = W2 + ((size_t)k * V + rb + (size_t)min(16 * tg + j, nrows - 1) * rstride) * d +
                 8 * q;
    }
    floatx4_t acc[NG];
    tile_stream<NG, DS, PACKED>(wp, step, zfrag + (size_t)k * (d / 32) * 64 + lane, d / 32, acc);
#pragma unroll
    for (int tg = 0; tg < NG; ++tg) {
      const float v0 = acc[tg][0] + acc[tg][1], v1 = acc[tg][2] + acc[tg][3];
#pragma unroll
      for (int b = 0; b < kTileVecs; ++b) {
        const float x = __shfl(b & 1 ? v1 : v0, j + 16 * (b >> 1));
        if (q == tg) win[b] = x;
      }
    }
  }
  w2_finish<kTileVecs>(win, nb, b0, K, k, V, G, g, rb, rstride, nrows, S, xs, head_logits,
                       part_val, part_id, part_m, part_s);
}

// ---------------------------------------------------------------------------
// Merge the G partial records of one (sequence, head): one workgroup of
// kMergeThreads. grid = (K, B). Every thread loads its share of the G*S
// candidates at once (kMergeBatch per round) and keeps a private sorted
// list in registers; each wave then takes its top S in S rounds of a
// wave-wide (value desc, id asc) selection, and wave 0 selects the final S
// from the waves' lists. Wave 0 also takes the log-sum-exp of the G (max,
// sum) records (wave_lse, fixed order).
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 4;

// Tree tokens and positions written by the merge (composite step): top-s
// drafting (u_draft null), the merge of head k writes the depth-(k+1) nodes'
// tokens; sampled drafting, workgroups of their own draw them (below).
struct MergeTree {
  int on;
  TreePlan plan;
  const int32_t* root_tok;
  const int32_t* kv_len;
  int32_t* tokens;
  int32_t* position_ids;
  const float* u_draft;       // [B][T] (sampled drafting) or null
  const float* head_logits;   // [B][K][V] (sampled drafting)
  int V;
};

// The merge of head k of sequence b. Threads past the first kMergeThreads
// (in a larger workgroup) take no part but meet its barrier; `tree`: write
// the top-s tree tokens and positions.
template <int SMAX>
__device__ __forceinline__ void merge_head(
    int k, int b, int K, int G, int S, const float* __restrict__ part_val,
    const int* __restrict__ part_id, const float* __restrict__ part_m,
    const float* __restrict__ part_s, int* __restrict__ topk_ids,
    float* __restrict__ topk_logits, float* __restrict__ lse, const MergeTree& tr, bool tree) {
  constexpr int NW = kMergeThreads / 64;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const bool act = t < kMergeThreads;   // wave-uniform
  const size_t rec0 = ((size_t)b * K + k) * G;
  __shared__ float sv[NW][MAXS_LDS];
  __shared__ int si[NW][MAXS_LDS];

  // wave 0's log-sum-exp records, loaded with the candidates when they fit
  // in registers
  const bool lse_early = lse != nullptr && wave == 0 && G <= 64 * kLseRegs;
  float lm[kLseRegs], ls[kLseRegs];
  if (lse_early) lse_load(part_m + rec0, part_s + rec0, G, lm, ls);
  // wave 0's tree data (plan rows lane + 64 i, all inside the plan's arrays;
  // the plan is a kernel argument), loaded now and used at the end
  constexpr int NQ = MAXT / 64;
  int pdep[NQ], prank[NQ], pkv = 0, proot = 0;
  if (tree && wave == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      pdep[q] = tr.plan.depth[lane + 64 * q];
      prank[q] = tr.plan.last_rank[lane + 64 * q];
    }
    pkv = tr.kv_len[b];
    proot = tr.root_tok[b];
  }

  float lv[SMAX];
  int li[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    lv[j] = kNegInf;
    li[j] = kNoId;
  }
  const int ncand = act ? G * S : 0;
  for (int base = 0; base < ncand; base += kMergeThreads * kMergeBatch) {
    float v[kMergeBatch];
    int id[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int c = base + t + kMergeThreads * u;
      const int cc = min(c, ncand - 1);
      v[u] = part_val[rec0 * S + cc];
      id[u] = part_id[rec0 * S + cc];
      if (c >= ncand) {
        v[u] = kNegInf;
        id[u] = kNoId;
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      // the S-th entry sits at a runtime index: select it with an unrolled scan
      float tv = kNegInf;
      int ti = kNoId;
#pragma unroll
      for (int j = 0; j < SMAX; ++j)
        if (j == S - 1) {
          tv = lv[j];
          ti = li[j];
        }
      if (better(v[u], id[u], tv, ti)) reg_insert<SMAX>(lv, li, v[u], id[u], S);
    }
  }
  float wv;
  int wi;
  if (act) {
    wave_select<SMAX>(lv, li, S, wv, wi);
    if (lane < S) {
      sv[wave][lane] = wv;
      si[wave][lane] = wi;
    }
  }

  // log-sum-exp of the G (max, sum) records: wave 0, fixed order
  if (lse != nullptr && wave == 0) {
    const float v = lse_early ? lse_of(lm, ls, G) : wave_lse(part_m + rec0, part_s + rec0, G);
    if (lane == 0) lse[(size_t)b * K + k] = v;
  }
  __syncthreads();
  if (wave != 0) return;
  // final selection over the waves' lists: lane l < NW*S holds one entry
  float fv[SMAX];
  int fi[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; ++j) {
    fv[j] = kNegInf;
    fi[j] = kNoId;
  }
  if (lane < NW * S) {
    fv[0] = sv[lane / S][lane % S];
    fi[0] = si[lane / S][lane % S];
  }
  wave_select<SMAX>(fv, fi, S, wv, wi);
  const size_t out = ((size_t)b * K + k) * S;
  if (lane < S) {
    topk_ids[out + lane] = wi;
    topk_logits[out + lane] = wv;
  }
  if (!tree) return;
  // nodes of depth k+1 take rank r's token of this head (held by lane r)
  const int T = tr.plan.T;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int n = 64 * q + lane;
    if (64 * q >= T) break;
    const int dep = opaque(pdep[q]), rk = opaque(prank[q]);
    const bool mine = n < T && n >= 1 && dep == k + 1;
    const int tok = __shfl(wi, min(n < T ? rk : 0, S - 1));
    if (mine) tr.tokens[(size_t)b * T + n] = tok;
    if (k == 0 && n < T) {
      tr.position_ids[(size_t)b * T + n] = opaque(pkv) + dep;
      if (n == 0) tr.tokens[(size_t)b * T] = opaque(proot);
    }
  }
}

template <int SMAX>
__global__ __launch_bounds__(kMergeThreads) void heads_merge_kernel(
    int K, int G, int S, const float* __restrict__ part_val, const int* __restrict__ part_id,
    const float* __restrict__ part_m, const float* __restrict__ part_s,
    int* __restrict__ topk_ids, float* __restrict__ topk_logits, float* __restrict__ lse,
    MergeTree tr) {
  merge_head<SMAX>(blockIdx.x, blockIdx.y, K, G, S, part_val, part_id, part_m, part_s, topk_ids,
                   topk_logits, lse, tr, tr.on != 0);
}

// Sampled drafting (composite step): the draws of the depth-(kd+1) nodes of
// sequence b from head kd's softmax, as the tree sampler makes them, by one
// kCdfThreads workgroup. The weights are e^(l - m) with m the row's maximum
// -- the largest of the W2 workgroups' maxima, an exact maximum -- instead
// of e^(l - lse): an inverse-CDF draw scales its target by the weights'
// total, so it needs no log-sum-exp and does not wait for the merge. Depth 1
// also writes the position ids and the root token.
__device__ __forceinline__ void sample_head(int kd, int b, int K, int G,
                                            const float* __restrict__ part_m,
                                            const MergeTree& tr) {
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int T = tr.plan.T, V = tr.V;
  __shared__ CdfLds sh;
  __shared__ float s_mx;
  const int dep = tr.plan.depth[min(t, MAXT - 1)];
  const bool mine = t >= 1 && t < T && dep == kd + 1;
  const float u = mine ? tr.u_draft[(size_t)b * T + t] : 0.f;
  if (wave == 0) {
    const float* pm = part_m + ((size_t)b * K + kd) * G;
    float m = kNegInf;
    for (int g = lane; g < G; g += 64) m = fmaxf(m, pm[g]);
    m = wave_max(m);
    if (lane == 0) s_mx = m;
  }
  if (kd == 0 && t < T) {
    tr.position_ids[(size_t)b * T + t] = tr.kv_len[b] + dep;
    if (t == 0) tr.tokens[(size_t)b * T] = tr.root_tok[b];
  }
  __syncthreads();
  const ExpRow w{tr.head_logits + ((size_t)b * K + kd) * V, s_mx, V};
  cdf_build<true>(w, V, sh);
  if (mine) tr.tokens[(size_t)b * T + t] = cdf_draw(w, V, u, sh);
}

// Composite step with sampled drafting: workgroups (k, b), k < K, merge head
// k (on their first kMergeThreads threads); workgroups (K + kd, b) draw the
// depth-(kd+1) nodes. Neither waits for the other.
template <int SMAX>
__global__ __launch_bounds__(kCdfThreads) void heads_merge_sample_kernel(
    int K, int G, int S, const float* __restrict__ part_val, const int* __restrict__ part_id,
    const float* __restrict__ part_m, const float* __restrict__ part_s,
    int* __restrict__ topk_ids, float* __restrict__ topk_logits, float* __restrict__ lse,
    MergeTree tr) {
  if ((int)blockIdx.x < K)
    merge_head<SMAX>(blockIdx.x, blockIdx.y, K, G, S, part_val, part_id, part_m, part_s,
                     topk_ids, topk_logits, lse, tr, false);
  else
    sample_head(blockIdx.x - K, blockIdx.y, K, G, part_m, tr);
}

template <class ET, int NB, int SPR>
hipError_t launch_heads_spr(const HeadsArgs& a, int b0, hipStream_t st) {
  constexpr int CW = RowStream<ET, NB>::CW;
  const int ldx = (a.d + CW - 1) / CW * CW;
  const size_t lds_x = (size_t)NB * ldx * sizeof(float);
  // rows per wave: as given, or the fewest that let all K d rows run as one
  // wave of four workgroups per compute unit (also where the kernel fits
  // fewer: the larger grid measured as fast or faster, 417-421 against
  // 423 us a step at batch 2)
  int rpw1 = a.w1_rows_per_wave;
  if (rpw1 <= 0) {
    const int slots = kHeadWaves * 4 * device_cus();
    rpw1 = std::min(64, std::max(1, (a.K * a.d + slots - 1) / slots));
  }
  const int rows1 = kHeadWaves * rpw1;
  const int g1 = (a.K * a.d + rows1 - 1) / rows1;
  hipLaunchKernelGGL((heads_w1_kernel<ET, NB, SPR>), dim3(g1), dim3(kHeadWaves * 64), lds_x, st, a.h,
                     a.B, b0, a.K, a.d, reinterpret_cast<const typename ET::storage*>(a.W1),
                     a.b1, a.z, rpw1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds_list = (size_t)kHeadWaves * NB * (2 * MAXS_LDS + 2) * sizeof(float);
  const size_t lds2 = lds_x > lds_list ? lds_x : lds_list;
  if (a.ev_before) {
    e = hipEventRecord(a.ev_before, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((heads_w2_kernel<ET, NB, SPR>), dim3(a.G, a.K), dim3(kHeadWaves * 64), lds2, st,
                     a.z, a.B, b0, a.K, a.V, a.d,
                     reinterpret_cast<const typename ET::storage*>(a.W2), a.w2_rows_per_wave,
                     a.S, a.head_logits, a.part_val, a.part_id, a.part_m, a.part_s, a.G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_after) e = hipEventRecord(a.ev_after, st);
  return e;
}

// Whole-row streams for bf16 rows of 8, 10 or 16 chunks (d = 4096, 5120,
// 8192) and one or two activation vectors; the generic stream otherwise.
template <class ET, int NB>
hipError_t launch_heads_nb(const HeadsArgs& a, int b0, hipStream_t st) {
  constexpr int CW = RowStream<ET, NB>::CW;
  if (std::is_same<ET, BF16>::value && NB <= 2 && a.d % CW == 0) {
    switch (a.d / CW) {
      case 8: return launch_heads_spr<ET, NB, (NB <= 2 ? 8 : 0)>(a, b0, st);
      case 10: return launch_heads_spr<ET, NB, (NB <= 2 ? 10 : 0)>(a, b0, st);
      case 16: return launch_heads_spr<ET, NB, (NB == 1 ? 16 : 0)>(a, b0, st);   // two spill
      default: break;
    }
  }
  return launch_heads_spr<ET, NB, 0>(a, b0, st);
}

// Batched passes (3 or more vectors, bf16): W1 split over 4 waves (fewer
// where d does not allow) with 8 column blocks in flight, W2 in tile rows of
// two (32 rows a wave) with 8 column blocks in flight (4 or 2 where d does
// not allow; 8 at three workgroups a unit against 4 at four: 206.5 against
// 208.9 us at a batch of 8). From a row-major W2 the batch-8 step took 746 us with these
// against 755-779 for 16-64 rows a wave and 4-16 tiles in flight:
// fragment-shaped reads lose DRAM locality as more of them are outstanding.
// From packed tiles the W2 pass takes 237 us against 286 (row-major); 3
// tile rows a wave (835 workgroups) took 254, 4 spill registers (305).
constexpr int kW2TileNg = 2;
// rows per W2 workgroup of the batched pass
int w2_tile_rows() { return kHeadWaves * 16 * kW2TileNg; }

hipError_t launch_heads_tile(const HeadsArgs& a, int b0, int G, hipStream_t st) {
  const int nb = std::min(kTileVecs, a.B - b0);
  const int d = a.d, nblk = d / 32;
  u32x4_t* hfrag = reinterpret_cast<u32x4_t*>(a.afrag);
  u32x4_t* zfrag = hfrag + (size_t)nblk * 64;
  hipLaunchKernelGGL(act_frag_kernel, dim3((nblk * 64 + 255) / 256), dim3(256), 0, st,
                     a.h + (size_t)b0 * d, (size_t)d, nb, d, hfrag);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint16_t* W1 = reinterpret_cast<const uint16_t*>(a.W1);
  uint16_t* zf16 = reinterpret_cast<uint16_t*>(zfrag);
  const int total = a.K * d;
  const uint16_t* W1p = reinterpret_cast<const uint16_t*>(a.W1_packed);
#define W1_TILE_P(KS, DS, P)                                                                   \
  hipLaunchKernelGGL((heads_w1_tile_kernel<KS, DS, P>),                                        \
                     dim3((total + 16 * (kHeadWaves / KS) - 1) / (16 * (kHeadWaves / KS))),    \
                     dim3(kHeadWaves * 64), 0, st, a.h, a.B, b0, a.K, d, W1, W1p, a.b1, hfrag,  \
                     a.z, zf16)
#define W1_TILE(KS, DS)     \
  if (W1p)                  \
    W1_TILE_P(KS, DS, true); \
  else                      \
    W1_TILE_P(KS, DS, false)
  if (nblk % 32 == 0)
    W1_TILE(4, 8);
  else if (nblk % 16 == 0)
    W1_TILE(2, 8);
  else if (nblk % 8 == 0)
    W1_TILE(1, 8);
  else
    W1_TILE(1, 2);
#undef W1_TILE
#undef W1_TILE_P
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_before) {
    e = hipEventRecord(a.ev_before, st);
    if (e != hipSuccess) return e;
  }
  const uint16_t* W2 = reinterpret_cast<const uint16_t*>(a.W2);
  const uint16_t* W2p = reinterpret_cast<const uint16_t*>(a.W2_packed);
#define W2_TILE_P(NG, DS, P)                                                                    \
  hipLaunchKernelGGL((heads_w2_tile_kernel<NG, DS, P>), dim3(G, a.K), dim3(kHeadWaves * 64), 0, \
                     st, a.B, b0, a.K, a.V, d, W2, W2p, zfrag, a.S, a.head_logits, a.part_val,   \
                     a.part_id, a.part_m, a.part_s, G)
#define W2_TILE(NG, DS)     \
  if (W2p)                  \
    W2_TILE_P(NG, DS, true); \
  else                      \
    W2_TILE_P(NG, DS, false)
  // d is a multiple of 64: nblk is even
  if (nblk % 8 == 0)
    W2_TILE(kW2TileNg, 8);
  else if (nblk % 4 == 0)
    W2_TILE(kW2TileNg, 4);
  else
    W2_TILE(kW2TileNg, 2);
#undef W2_TILE
#undef W2_TILE_P
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.ev_after) e = hipEventRecord(a.ev_after, st);
  return e;
}

template <class ET>
hipError_t launch_heads_et(const HeadsArgs& a, hipStream_t st) {
  // Three or more bf16 vectors go through the batched passes, all of them
  // (the merge reads every sequence's records with one row-block count).
  const bool tile = std::is_same<ET, BF16>::value && a.B >= 3 && a.afrag;
  const int G = tile ? (a.V + w2_tile_rows() - 1) / w2_tile_rows() : a.G;
  for (int b0 = 0; b0 < a.B; b0 += 8) {
    const int nb = a.B - b0;
    hipError_t e;
    if (tile)
      e = launch_heads_tile(a, b0, G, st);
    else if (nb == 1)
      e = launch_heads_nb<ET, 1>(a, b0, st);
    else if (nb == 2)
      e = launch_heads_nb<ET, 2>(a, b0, st);
    else if (nb <= 4)
      e = launch_heads_nb<ET, 4>(a, b0, st);
    else
      e = launch_heads_nb<ET, 8>(a, b0, st);
    if (e != hipSuccess) return e;
  }
  MergeTree tr{};
  tr.on = a.fuse_tree ? 1 : 0;
  if (a.fuse_tree) {
    tr.plan = a.plan;
    tr.root_tok = a.root_tok;
    tr.kv_len = a.kv_len;
    tr.tokens = a.tree_tokens;
    tr.position_ids = a.position_ids;
    tr.u_draft = a.u_draft;
    tr.head_logits = a.head_logits;
    tr.V = a.V;
  }
  // sampled drafting: the merge and the draws in one launch
  const bool sample = a.fuse_tree && a.u_draft;
#define MERGE_LAUNCH(SM)                                                                       \
  if (sample)                                                                                  \
    hipLaunchKernelGGL(heads_merge_sample_kernel<SM>, dim3(2 * a.K, a.B), dim3(kCdfThreads), 0, \
                       st, a.K, G, a.S, a.part_val, a.part_id, a.part_m, a.part_s, a.topk_ids, \
                       a.topk_logits, a.lse, tr);                                              \
  else                                                                                         \
    hipLaunchKernelGGL(heads_merge_kernel<SM>, dim3(a.K, a.B), dim3(kMergeThreads), 0, st,     \
                       a.K, G, a.S, a.part_val, a.part_id, a.part_m, a.part_s, a.topk_ids,     \
                       a.topk_logits, a.lse, tr)
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

int heads_row_blocks_max(int V, int rows_per_wave) {
  const int per_row = (V + 4 * rows_per_wave - 1) / (4 * rows_per_wave);
  const int batched = (V + w2_tile_rows() - 1) / w2_tile_rows();
  return std::max(per_row, batched);
}

hipError_t launch_heads(const HeadsArgs& a, hipStream_t st) {
  return a.f32 ? launch_heads_et<F32>(a, st) : launch_heads_et<BF16>(a, st);
}

}  // namespace medusa
