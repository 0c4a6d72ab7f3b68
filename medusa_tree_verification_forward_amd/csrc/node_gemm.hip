// Skinny node GEMMs of the verify pass on gfx950 MFMA:
//   C[M][N] = A[M][K] * W[N][K]^T,  M = B*T tree rows (tens to a few hundred),
//   N = 3d (QKV), d (output projection) or V (verification LM head).
//
// The weights are read exactly once and dominate the traffic, so the kernel
// is built around streaming them at full HBM rate:
//  * W is pre-packed into MFMA operand tiles (launch_pack_weight): a tile is
//    16 rows x 64 bytes of k, stored as 64 lane-ordered 16-byte pieces, so
//    the B fragment of one v_mfma_f32_16x16x32_bf16 is a single 1 KB
//    contiguous wave load, and a 16-row stripe of W is one contiguous run.
//  * Each wave owns one 16-column stripe and streams its k-tiles through a
//    ring of D registers (D loads in flight per wave).
//  * A (the tree rows, a few hundred KB, L2-resident) is shared by the WV
//    waves of a workgroup: it moves in chunks of CH k-tiles, loaded into
//    registers one chunk ahead and written to one of two LDS buffers; one
//    barrier per chunk publishes the next buffer.
//  * fp32 storage uses v_mfma_f32_16x16x4_f32, four per 16-byte piece (the
//    k order inside a piece is permuted identically for both operands,
//    which leaves the dot products unchanged).
//  * Rows beyond one pass of 16*MT go to further workgroups (grid z).
//
// QKV and the output projection split K over KS workgroups per column group
// and write fp32 partials part[g][ks][r][c]; an epilogue sums the KS slices
// of each output in slice order and applies
//   QKV  : RoPE on q and k (pairs i, i+Dh/2; angle pos * theta^(-2i/Dh)),
//          rounding to the storage type, scatter to [B][T][H][Dh];
//   OPROJ: y = x + acc with x = E[token], written as fp32 and storage type.
// W_qkv is packed with the rows of every head reordered so that each
// 16-column tile holds 8 whole rotation pairs (columns j and j+8 of the tile
// are rows i and i+Dh/2 of the head, i = 8*(tile in head) + j).
// With KS = 1 the epilogue runs on the accumulators themselves (the rotation
// partner of a lane's column is in lane li ^ 8). Otherwise it runs in the last
// of the KS workgroups of a group to finish (found with a device-scope
// counter that it leaves at zero for the next launch; the partials travel
// through agent-coherent stores and loads, no fence).
// The LM head (never split over K) reduces in-kernel:
// per row and 16-column stripe (max, argmax, S, W) at temperature tau with
// S = sum e^{(l-m)/tau}, W = sum e^{(l-m)/tau} (l-m)/tau, one record per
// (row, stripe) written by the wave that owns the stripe; the logit of every
// tree node's token under its parent's row; optional full logits. A merge
// kernel combines the stripes of a row in order.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSplits = 16;


// One A fragment times one W fragment (16-byte pieces of both operands).
template <class ET>
__device__ __forceinline__ floatx4_t frag_mfma(const u32x4_t& a, const u32x4_t& b,
                                               floatx4_t c) {
  if constexpr (ET::kPerVec == 8) {
    return mfma16x16x32_bf16(a, b, c);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = mfma16x16x4_f32(__uint_as_float(a[j]), __uint_as_float(b[j]), c);
    return c;
  }
}

// Row of W held by packed row n: identity, or the rotation-pair order of
// W_qkv (within each block of Dh rows, tile tt, lane column li: rows
// 8 tt + li for li < 8, Dh/2 + 8 tt + li - 8 otherwise).
__device__ __forceinline__ int packed_source_row(int n, int pair_dh) {
  if (pair_dh == 0) return n;
  const int blk = n / pair_dh, nl = n - blk * pair_dh;
  const int tt = nl >> 4, li = nl & 15;
  return blk * pair_dh + (li < 8 ? 8 * tt + li : (pair_dh >> 1) + 8 * tt + li - 8);
}

// Tile order: k-major -- tile (nt, kt) at kt * ntiles + nt, so the stripes
// that the waves of a launch stream side by side are adjacent in memory
// (stripe-major order, and runs of 2-16 k-tiles a stripe, measured no
// faster).
__device__ __forceinline__ size_t packed_tile(int nt, int kt, int ntiles) {
  return (size_t)kt * ntiles + nt;
}

// Packing: piece q of the output is lane l = q % 64 of tile q / 64; tile
// (nt, kt) (order above) holds packed rows 16 nt + l % 16, k elements
// KT kt + PV (l / 16) .. + PV - 1 (KT = 4 PV). Rows >= rows are 0.
template <class ET>
__global__ void pack_weight_kernel(const typename ET::storage* __restrict__ W, int rows, int K,
                                   int pair_dh, u32x4_t* __restrict__ out, size_t pieces) {
  constexpr int PV = ET::kPerVec, KT = 4 * PV;
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= pieces) return;
  const int ntiles = (rows + 15) / 16;
  const size_t tile = q >> 6;
  const int l = (int)(q & 63);
  const int kt = (int)(tile / ntiles), nt = (int)(tile - (size_t)kt * ntiles);
  const int n = 16 * nt + (l & 15);
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < rows) {
    const int r = packed_source_row(n, pair_dh);
    v = load16(W + (size_t)r * K + (size_t)KT * kt + PV * (l >> 4));
  }
  out[q] = v;
}

// QKV epilogue of packed column c1 (a rotation pair: columns c1 and c1 + 8
// of the tile are elements i and i + Dh/2 of head h of q, k or v). What
// depends on the column alone is computed once per lane: the destination of
// row 0, the RoPE frequency theta^(-2i/Dh) in fp64, and whether to rotate
// (q and k). The three output addresses go through opaque(): a
// lane-dependent choice among kernel arguments would otherwise become a load
// from the argument segment at every use; the chosen one is used as a global
// (address space 1) pointer.
template <class ET>
struct QkvColumn {
  using St = typename ET::storage;
  typedef __attribute__((address_space(1))) St GSt;
  GSt* o;         // element (row 0, i) of the destination
  int rstride;    // elements per row: H * Dh
  int half;       // Dh / 2
  bool rope;
  double inv_freq;
  __device__ __forceinline__ QkvColumn(const GemmParams& p, int c1) {
    const int Dh = p.Dh;
    const int blk = c1 / Dh, nl = c1 - blk * Dh;
    const int i = 8 * (nl >> 4) + (nl & 7);
    const int which = blk / p.H, h = blk - which * p.H;
    const uint64_t q = opaque((uint64_t)(uintptr_t)p.q_out);
    const uint64_t k = opaque((uint64_t)(uintptr_t)p.k_out);
    const uint64_t v = opaque((uint64_t)(uintptr_t)p.v_out);
    o = (GSt*)(which == 0 ? q : (which == 1 ? k : v)) + (size_t)h * Dh + i;
    rstride = p.H * Dh;
    half = Dh >> 1;
    rope = which < 2;
    inv_freq = exp(-(2.0 * i / Dh) * p.log_theta);
  }
  // cos and sin of the rotation at position pos
  __device__ __forceinline__ void angle(int pos, float& cs, float& sn) const {
    const double turns = (double)pos * inv_freq * 0.15915494309189535;   // 1/(2 pi)
    const float ang = (float)((turns - rint(turns)) * 6.283185307179586);
    __sincosf(ang, &sn, &cs);
  }
  // row r at position pos: rotate (x1, x2), round, store both elements
  __device__ __forceinline__ void store(int r, int pos, float x1, float x2) const {
    if (rope) {
      float cs, sn;
      angle(pos, cs, sn);
      const float y1 = x1 * cs - x2 * sn;
      const float y2 = x2 * cs + x1 * sn;
      x1 = y1;
      x2 = y2;
    }
    GSt* const d = o + (size_t)r * rstride;
    d[0] = ET::from_float(x1);
    d[half] = ET::from_float(x2);
  }
  // One element of the pair: the first (second = false: x1 own, x2 the
  // partner's) or the second (x2 own, x1 the partner's); the same rounding
  // as store().
  __device__ __forceinline__ void store_one(int r, int pos, float own, float partner,
                                            bool second) const {
    float y = own;
    if (rope) {
      float cs, sn;
      angle(pos, cs, sn);
      y = second ? own * cs + partner * sn : own * cs - partner * sn;
    }
    o[(size_t)r * rstride + (second ? half : 0)] = ET::from_float(y);
  }
};

// y = x + acc, x = E[token of row r]: written as fp32 and, in the LM head's
// A-fragment order, as storage type. Rows M .. 16 a_mtiles - 1 of the
// fragment-ordered copy (the padding of its last m-tile) are written as zero.
template <class ET>
__device__ __forceinline__ void oproj_store(const GemmParams& p, int r, int n, float y) {
  using St = typename ET::storage;
  if (r >= 16 * p.a_mtiles) return;
  const bool live = r < p.M;
  if (live) p.y_out[(size_t)r * p.N + n] = y;
  reinterpret_cast<St*>(p.y_elem)[frag_index(r, n, p.a_mtiles, ET::kPerVec)] =
      ET::from_float(live ? y : 0.f);
}

// Workgroup coordinates: column group g, K slice ks, row pass pz. With one
// row pass they are the block indices. With several, the passes of one
// (group, slice) get linear ids 8 apart: linear id mod 8 picks the XCD, so
// they run on the same XCD at about the same time and stream the same
// weight tiles through its L2 instead of each from HBM.
__device__ __forceinline__ void wg_coords(int& g, int& ks, int& pz) {
  const int P = gridDim.z;
  if (P == 1) {
    g = blockIdx.x;
    ks = blockIdx.y;
    pz = 0;
    return;
  }
  const int units = gridDim.x * gridDim.y;
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int full = units & ~7;
  int u;
  if (lin < full * P) {
    u = 8 * (lin / (8 * P)) + (lin & 7);
    pz = (lin >> 3) % P;
  } else {
    const int rest = units - full, l2 = lin - full * P;
    u = full + l2 % rest;
    pz = l2 / rest;
  }
  g = u % gridDim.x;
  ks = u / gridDim.x;
}

// Row data and outputs of the one-slice QKV / output-projection epilogue:
// lane (li, lq) holds column col and rows m0 + 16 mt + 4 lq + j of the
// accumulators. QKV: the rows' positions; output projection: the rows'
// residual elements E[token], raw bits. Loads
// are issued by load() and used only in finish() (opaque() keeps the
// arithmetic on them there, so that a load issued early does not stall).
template <class ET, int MT, int EPI>
struct SliceRows {
  int rv[MT][4];
  uint32_t xr[MT][4];
  __device__ __forceinline__ void load(const GemmParams& p, int m0, int lq, int col) {
    using St = typename ET::storage;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = min(m0 + 16 * mt + 4 * lq + j, p.M - 1);
        rv[mt][j] = EPI == EPI_QKV ? p.pos[r] : min(max(p.tokens[r], 0), p.a_nrows - 1);
      }
    if constexpr (EPI != EPI_QKV) {
      const int cc = min(col, p.N - 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xr[mt][j] = ET::load_raw(reinterpret_cast<const St*>(p.E) + (size_t)rv[mt][j] * p.N + cc);
    }
  }
  __device__ __forceinline__ void finish(const GemmParams& p, const floatx4_t (&acc)[MT], int m0,
                                         int li, int lq, int col) const {
    if constexpr (EPI == EPI_QKV) {
      // lanes li and li ^ 8 hold the two elements of a rotation pair: each
      // rotates and stores its own (the pair's column constants are the same
      // for both)
      const QkvColumn<ET> cq(p, min(col, p.N - 1));
      const bool second = li >= 8;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float other = __shfl_xor(acc[mt][j], 8);
          const int r = m0 + 16 * mt + 4 * lq + j;
          if (r < p.M && col < p.N) cq.store_one(r, opaque(rv[mt][j]), acc[mt][j], other, second);
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m0 + 16 * mt + 4 * lq + j;
          if (col < p.N)
            oproj_store<ET>(p, r, col, ET::from_raw(opaque(xr[mt][j])) + acc[mt][j]);
        }
    }
  }
};

// LDS slot of the 16-byte A piece of fragment lane (lq, li) in k-tile kt of
// a chunk (chunks start at even k-tiles): the lane's own slot within its lq
// quarter, rotated by 2 lq + 8 (kt % 2). Sixteen consecutive lanes of a
// fragment read (fixed lq, kt) hit 16 distinct slots mod 16, and so do
// sixteen consecutive lanes of a row-contiguous store (two rows, both
// k-tiles of a pair, four pieces).
__device__ __forceinline__ int a_slot(int kt, int lq, int li) {
  return 16 * lq + ((li + 2 * lq + 8 * (kt & 1)) & 15);
}

template <class ET, int WV, int MT, int CH, int D, int EPI>
__global__ __launch_bounds__(64 * WV, WV <= 3 ? 1 : 2) void node_gemm_kernel(
    GemmParams p) {
  using St = typename ET::storage;
  constexpr int PV = ET::kPerVec, KT = 4 * PV;   // k elements per tile
  constexpr int GC = 16 * WV;                     // output columns per workgroup
  static_assert((CH * MT) % WV == 0, "A fragments of a chunk must divide over the waves");
  static_assert((2 * CH) % D == 0, "the weight ring must divide a pair of chunks");
  constexpr int NAW = CH * MT / WV;               // A loads per wave per chunk
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  int g, ks, pz;
  wg_coords(g, ks, pz);
  const int KS = gridDim.y;
  const int m0 = pz * 16 * MT;
  const St* __restrict__ A = reinterpret_cast<const St*>(p.A);
  const int nkt = p.K / KT;
  const int kt_lo = (int)((long)nkt * ks / KS), kt_hi = (int)((long)nkt * (ks + 1) / KS);
  const int nloc = kt_hi - kt_lo;
  const int ntiles = (p.N + 15) >> 4;
  const int n0 = g * GC;
  const int col = n0 + 16 * wave + li;
  // this wave's stripe (wave-uniform) and its k-tile s of the slice
  const int nt = min(g * WV + __builtin_amdgcn_readfirstlane(wave), ntiles - 1);
  const u32x4_t* __restrict__ W4 = reinterpret_cast<const u32x4_t*>(p.W) + lane;
  auto wtile = [&](int s) { return W4 + packed_tile(nt, kt_lo + s, ntiles) * 64; };

  __shared__ u32x4_t sA0[CH][MT][64];
  __shared__ u32x4_t sA1[CH][MT][64];

  // LM head: node e of the pass's sequences (-1 for roots and past the end),
  // its token and the row of its parent. The token and parent loads are in
  // range for every e; what is computed from them is computed where used.
  const int rows_hi = min(p.M, m0 + 16 * MT);
  const int bl = m0 / max(p.T, 1), bh = (rows_hi - 1) / max(p.T, 1);
  const int nchild = EPI == EPI_LM ? (bh - bl + 1) * p.T : 0;
  auto child_node = [&](int e) {
    const int cnode = e % p.T;
    return e < nchild && cnode >= 1 ? (bl + e / p.T) * p.T + cnode : -1;
  };
  auto child_raw = [&](int node, int& tok_raw, int& par_raw) {
    const int nd = max(node, 0);   // node < M = B T for every e < nchild
    tok_raw = p.tokens[nd];
    par_raw = p.parent[nd % p.T];
  };
  // the first 64 nodes' loads go out before the stream (not with twelve
  // m-tiles, whose registers are taken)
  constexpr bool kEarlyChild = EPI == EPI_LM && MT <= 3;
  int ch_node = -1, ch_tok_raw = 0, ch_par_raw = 0;
  if constexpr (kEarlyChild) {
    ch_node = child_node(lane);
    child_raw(ch_node, ch_tok_raw, ch_par_raw);
  }

  // A moves in units of 1 KB, unit f = wave + WV i of a chunk covering rows
  // 8 h .. 8 h + 7 of m-tile mt over the k-tile pair 2 pr, 2 pr + 1, with
  // (h, mt, pr) = (f % 2, f / 2 % MT, f / (2 MT)): each row's 128 bytes are
  // read by 8 lanes (row 8 h + ar, k-tile 2 pr + ak, piece ap), so a unit
  // touches 8 whole cache lines where a fragment-shaped load touches 16
  // halves. In LDS the fragments are stored with the 16-byte slot of lane
  // (lq, li) of k-tile kt at a_slot(kt, lq, li), which keeps both the
  // scattered stores and the fragment reads free of bank conflicts.
  // Gathered rows: every index load is issued before any is used (a load
  // and its clamp per unit would put one memory latency per unit in front
  // of the weight stream).
  // The LM head's A (the output projection's y) comes in A-fragment order
  // (frag_index): there unit f is fragment (k-tile f / MT, m-tile f % MT),
  // one contiguous 1 KB, stored at its lanes' own slots.
  static_assert(CH % 2 == 0, "A units cover k-tile pairs");
  constexpr bool kFragA = EPI == EPI_LM;
  const int ar = lane >> 3, ak = (lane >> 2) & 1, ap = lane & 3;
  const St* asrc[NAW];
  if constexpr (kFragA) {
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
      const int mt = min(m0 / 16 + (wave + WV * i) % MT, p.a_mtiles - 1);
      asrc[i] = A + ((size_t)kt_lo * p.a_mtiles * 64 + (size_t)mt * 64 + lane) * PV;
    }
  } else {
    int src[NAW];
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
      const int f = wave + WV * i;
      src[i] = min(m0 + 16 * (f / 2 % MT) + 8 * (f % 2) + ar, p.M - 1);
    }
    if (p.a_rows) {
      int raw[NAW];
#pragma unroll
      for (int i = 0; i < NAW; ++i) raw[i] = p.a_rows[src[i]];
#pragma unroll
      for (int i = 0; i < NAW; ++i) src[i] = min(max(raw[i], 0), p.a_nrows - 1);
    }
#pragma unroll
    for (int i = 0; i < NAW; ++i)
      asrc[i] = A + (size_t)src[i] * p.lda + (size_t)kt_lo * KT + PV * ap;
  }
  // A units of chunks c+1 and c+2 are in flight in two register sets
  u32x4_t ra0[NAW], ra1[NAW];
  // Past the slice end the k-tile index is clamped (those values are never read).
  auto load_a = [&](int c, u32x4_t(&ra)[NAW]) {
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
      const int f = wave + WV * i;
      if constexpr (kFragA) {
        const int kt = min(c * CH + f / MT, nloc - 1);
        ra[i] = load16(asrc[i] + (size_t)kt * p.a_mtiles * 64 * PV);
      } else {
        const int kt = min(c * CH + 2 * (f / (2 * MT)) + ak, nloc - 1);
        ra[i] = load16(asrc[i] + (size_t)kt * KT);
      }
    }
  };
  auto store_a = [&](u32x4_t(&buf)[CH][MT][64], const u32x4_t(&ra)[NAW]) {
#pragma unroll
    for (int i = 0; i < NAW; ++i) {
      const int f = wave + WV * i;
      if constexpr (kFragA) {
        buf[f / MT][f % MT][a_slot(f / MT, lq, li)] = ra[i];
      } else {
        const int j = 2 * (f / (2 * MT)) + ak;
        buf[j][f / 2 % MT][a_slot(j, ap, 8 * (f % 2) + ar)] = ra[i];
      }
    }
  };
  floatx4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wr[D];

  // Row data of the one-slice epilogue. Configurations with at most three
  // waves run one workgroup per compute unit and hold it through the stream.
  constexpr bool kEarlyRows = (EPI == EPI_QKV || EPI == EPI_OPROJ) && WV <= 3;
  SliceRows<ET, MT, EPI> rows;

  const int nch = (nloc + CH - 1) / CH;
  load_a(0, ra0);
  load_a(1, ra1);
#pragma unroll
  for (int j = 0; j < D; ++j) wr[j] = load16_stream(wtile(min(j, nloc - 1)));
  // row data held through the stream: loaded once the stream is under way
  if constexpr (kEarlyRows) {
    if (KS == 1) rows.load(p, m0, lq, col);
  }
  store_a(sA0, ra0);
  load_a(2, ra0);
  lds_barrier();

  // Chunk c: CH k-tiles from the weight registers against the A fragments
  // in `cur`; each consumed register is refilled D k-tiles ahead. Then the
  // A fragments of chunk c+1 (loaded two chunks earlier, in `ra`) go to
  // `nxt`, the loads of chunk c+3 start in `ra`, and one barrier publishes
  // `nxt`. Loading A two chunks ahead keeps its wait from draining the
  // weight ring (D = 2 CH loads stay in flight across the barrier). A steady
  // chunk has every step and every refill in range, so the loop keeps a fixed
  // number of loads in flight; the last chunks check their bounds.
  auto chunk = [&](int c, u32x4_t(&cur)[CH][MT][64], u32x4_t(&nxt)[CH][MT][64],
                   u32x4_t(&ra)[NAW], auto steady, auto odd) {
    constexpr bool S = decltype(steady)::value;
    constexpr int R0 = decltype(odd)::value ? CH : 0;   // ring slot of the chunk's first step
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int s = c * CH + j;
      if (S || s < nloc) {
        const u32x4_t b = wr[(R0 + j) % D];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = frag_mfma<ET>(cur[j][mt][a_slot(j, lq, li)], b, acc[mt]);
        if (S || s + D < nloc) wr[(R0 + j) % D] = load16_stream(wtile(s + D));
      }
      // one k-tile at a time: hoisting later LDS reads only raises pressure
      __builtin_amdgcn_sched_barrier(0);
    }
    if (S || c + 1 < nch) {
      store_a(nxt, ra);
      load_a(c + 3, ra);
      lds_barrier();
    }
  };
  const std::integral_constant<bool, true> steady{};
  const std::integral_constant<bool, false> guarded{};
  const std::integral_constant<bool, false> even{};
  const std::integral_constant<bool, true> odd{};
  int c = 0;
  for (; (c + 2) * CH + D <= nloc; c += 2) {
    chunk(c, sA0, sA1, ra1, steady, even);
    chunk(c + 1, sA1, sA0, ra0, steady, odd);
  }
  for (; c < nch; ++c) {
    if (c & 1)
      chunk(c, sA1, sA0, ra0, guarded, odd);
    else
      chunk(c, sA0, sA1, ra1, guarded, even);
  }

  if constexpr (EPI == EPI_QKV || EPI == EPI_OPROJ) {
    if (KS == 1) {
      // One slice: finish straight from the accumulators.
      if constexpr (!kEarlyRows) rows.load(p, m0, lq, col);
      rows.finish(p, acc, m0, li, lq, col);
      return;
    }
  }
  if constexpr (EPI != EPI_LM) {
    // slice ks of the partials: part[g][ks][r][c] (a workgroup's slice is one
    // contiguous [M][GC] block)
    float* part = p.part + (size_t)(g * KS + ks) * p.M * GC + 16 * wave + li;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = m0 + 16 * mt + 4 * lq + j;
        if (r < p.M) coherent_store(part + (size_t)r * GC, acc[mt][j]);
      }
    // The last of the KS workgroups of this (group, pass) finishes it: every
    // thread loads all the slices of its outputs before it uses any, then
    // sums them in slice order. The row data of a thread's first batch of
    // rows (positions, residual rows) is loaded before the hand-off, so its
    // latency overlaps the count; workgroups that turn out not to be last
    // drop it.
    constexpr int NT = 64 * WV;
    const size_t sstride = (size_t)p.M * GC;
    const float* gpart = p.part + (size_t)g * KS * p.M * GC;
    if constexpr (EPI == EPI_QKV) {
      // thread: rotation pair pi of the group (packed columns c1, c1 + 8),
      // rows m0 + rl + RL i, in batches of RB rows
      constexpr int PG = 8 * WV, RL = NT / PG, RPT = 16 * MT / RL;
      constexpr int RB = RPT < 6 ? RPT : 6;
      static_assert(RPT % RB == 0, "row batches");
      const int pi = threadIdx.x % PG, rl = threadIdx.x / PG;
      const int cl = 16 * (pi >> 3) + (pi & 7), c1 = n0 + cl;
      int pos[RB];
      auto load_pos = [&](int i0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) pos[i] = p.pos[min(m0 + rl + RL * (i0 + i), p.M - 1)];
      };
      load_pos(0);
      const QkvColumn<ET> cq(p, min(c1, p.N - 1));
      if (!last_to_arrive(p.counters + g * gridDim.z + pz, KS)) return;
#pragma unroll 1
      for (int i0 = 0; i0 < RPT; i0 += RB) {
        if (i0 > 0) load_pos(i0);
        float x1[RB], x2[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) x1[i] = x2[i] = 0.f;
        for (int s0 = 0; s0 < KS; s0 += 2) {
          float v1[2][RB], v2[2][RB];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < RB; ++i) {
              const int r = min(m0 + rl + RL * (i0 + i), p.M - 1);
              const float* q = gpart + min(s0 + u, KS - 1) * sstride + (size_t)r * GC + cl;
              v1[u][i] = coherent_load(q);
              v2[u][i] = coherent_load(q + 8);
            }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (s0 + u < KS)
#pragma unroll
              for (int i = 0; i < RB; ++i) {
                x1[i] += v1[u][i];
                x2[i] += v2[u][i];
              }
        }
        if (c1 < p.N)
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const int r = m0 + rl + RL * (i0 + i);
            if (r < p.M) cq.store(r, pos[i], x1[i], x2[i]);
          }
      }
    } else if constexpr (EPI == EPI_OPROJ) {
      // thread: column cl of the group, rows m0 + rl + RL i, in batches of RB
      constexpr int RL = NT / GC, RPT = 16 * MT / RL;
      constexpr int RB = RPT < 12 ? RPT : 12;
      static_assert(RPT % RB == 0, "row batches");
      const int cl = threadIdx.x % GC, rl = threadIdx.x / GC;
      const int n = min(n0 + cl, p.N - 1);
      float x[RB];
      auto load_x = [&](int i0) {
        int tok[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i)
          tok[i] = min(max(p.tokens[min(m0 + rl + RL * (i0 + i), p.M - 1)], 0), p.a_nrows - 1);
#pragma unroll
        for (int i = 0; i < RB; ++i)
          x[i] = ET::load1(reinterpret_cast<const St*>(p.E) + (size_t)tok[i] * p.N + n);
      };
      load_x(0);
      if (!last_to_arrive(p.counters + g * gridDim.z + pz, KS)) return;
#pragma unroll 1
      for (int i0 = 0; i0 < RPT; i0 += RB) {
        if (i0 > 0) load_x(i0);
        float acc_s[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) acc_s[i] = 0.f;
        for (int s0 = 0; s0 < KS; s0 += 4) {
          float v[4][RB];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < RB; ++i) {
              const int r = min(m0 + rl + RL * (i0 + i), p.M - 1);
              v[u][i] =
                  coherent_load(gpart + min(s0 + u, KS - 1) * sstride + (size_t)r * GC + cl);
            }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (s0 + u < KS)
#pragma unroll
              for (int i = 0; i < RB; ++i) acc_s[i] += v[u][i];
        }
        if (n0 + cl < p.N)
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            oproj_store<ET>(p, m0 + rl + RL * (i0 + i), n, x[i] + acc_s[i]);
          }
      }
    }
  } else {
    // The wave's logit tile goes through LDS, 48 rows (MG m-tiles) at a time,
    // so that lane r owns row r of the group: per row and 16-column stripe
    // (max, lowest argmax, S, W) scanned over the columns in order, one
    // record per row; then the tree nodes whose parent row is in the group.
    constexpr int MG = MT < 3 ? MT : 3;
    static_assert(MT % MG == 0, "row groups");
    constexpr int LTS = 20;   // row stride (floats) of the tile: 16-byte rows
    // the tiles take the A buffers' LDS when they fit there (every wave is
    // past its last chunk after the barrier), else LDS of their own
    constexpr int kLtFloats = WV * 16 * MG * LTS;
    constexpr bool kLtInA = kLtFloats * 4 <= (int)sizeof(sA0);
    __shared__ float lt_own[kLtInA ? 1 : kLtFloats];
    float* lt_base = lt_own;
    if constexpr (kLtInA) {
      __syncthreads();
      lt_base = reinterpret_cast<float*>(&sA0[0][0][0]);
    }
    const auto lt = [&](int r, int c) -> float& {
      return lt_base[(wave * 16 * MG + r) * LTS + c];
    };
    const int c0 = n0 + 16 * wave;
    const int nv = min(16, p.N - c0);   // valid columns of the stripe
    const int stripes = gridDim.x * WV;
#pragma unroll
    for (int mq = 0; mq < MT; mq += MG) {
      if (mq > 0) wave_lds_sync();   // the previous group's reads are done
#pragma unroll
      for (int mt = 0; mt < MG; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) lt(16 * mt + 4 * lq + j, li) = acc[mq + mt][j];
      wave_lds_sync();
      const int g0 = m0 + 16 * mq;   // first row of the group
      if (lane < 16 * MG) {
        const int r = g0 + lane;
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 x = *reinterpret_cast<const float4*>(&lt(lane, 4 * q));
          v[4 * q] = x.x;
          v[4 * q + 1] = x.y;
          v[4 * q + 2] = x.z;
          v[4 * q + 3] = x.w;
        }
        float bv = kNegInf;
        int bi = 0x7fffffff;
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (c < nv && v[c] > bv) {
            bv = v[c];
            bi = c0 + c;
          }
        float sv = 0.f, wv = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c)
          if (c < nv) {
            const float z = (v[c] - bv) * p.inv_tau;
            const float e = exp_e(z);
            sv += e;
            wv += e * z;
          }
        if (r < p.M)
          *reinterpret_cast<float4*>(p.part + ((size_t)r * stripes + g * WV + wave) * 4) =
              make_float4(bv, sv, wv, __int_as_float(bi));
      }
      // logit of each tree node's token under its parent's row (this wave's
      // columns), 64 nodes at a time
      const int g1 = min(rows_hi, g0 + 16 * MG);
      for (int e0 = 0; e0 < nchild; e0 += 64) {
        int node = ch_node, tok = opaque(ch_tok_raw), par = opaque(ch_par_raw);
        if (!kEarlyChild || e0 > 0) {
          node = child_node(e0 + lane);
          child_raw(node, tok, par);
        }
        const int r = (max(node, 0) / p.T) * p.T + min(max(par, 0), p.T - 1);
        if (node >= 0 && tok >= c0 && tok < c0 + 16 && r >= g0 && r < g1)
          p.child_logit[node] = lt(r - g0, tok - c0);
      }
    }
    if (p.logits_out && col < p.N)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = m0 + 16 * mt + 4 * lq + j;
          if (r < p.M) p.logits_out[(size_t)r * p.N + col] = acc[mt][j];
        }
  }
}

// f(integral_constant<int, J>) for J = 0, 1, ... in order, unrolled
template <class F, int... J>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// ---------------------------------------------------------------------------
// QKV projection and LM head of more than 48 tree rows (13B trees, batches),
// bf16. The WV waves of a workgroup split the rows -- wave w takes rows
// m0 + 48 w .. + 48 (MW = 3 m-tiles) -- and share the weight tiles of the
// workgroup's NS stripes: each k-tile's NS tiles are loaded once per
// workgroup (wave w loads tiles w, w + WV, ...), written to one of two LDS
// slots and read by every wave after one barrier per k-tile. Each wave
// loads its own A fragments (its rows are nobody else's) straight from
// global memory. Per k-tile a wave does MW x NS MFMAs: a B fragment read
// from LDS feeds MW products and an A fragment NS.
// Weights and A fragments are both loaded D k-tiles ahead: vector loads
// complete in issue order, so waiting for an A fragment also waits for
// every weight load issued before it, and the weight prefetch is only as
// deep as the A prefetch. The LDS holds four k-tiles of weights: a step
// publishes k-tile s + 2 and reads k-tile s + 1's B fragments into
// registers before it multiplies k-tile s, so the one barrier per step
// separates writes from reads two steps later and the LDS latency hides
// behind the MFMAs instead of sitting between the barrier and them.
//
// LM epilogue: per m-tile the wave's 16 x 16 NS logit tile goes through LDS;
// lane (r, part) = (lane % 16, lane / 16) scans row r's columns
// part 4 NS .. + 4 NS in order, the four parts are merged in a fixed order
// (rec_merge is commutative), and one record per (row, workgroup) is
// written: the row-statistics merge reads ceil(stripes / NS) records a row.
template <int WV, int NS, int EPI>
__global__ __launch_bounds__(64 * WV, 1) void node_gemm_rows_kernel(GemmParams p) {
  using ET = BF16;
  using St = typename ET::storage;
  static_assert(EPI == EPI_QKV || EPI == EPI_LM, "QKV projection or LM head");
  constexpr int PV = ET::kPerVec, KT = 4 * PV;
  constexpr int MW = 3;                    // m-tiles a wave
  constexpr int NPW = (NS + WV - 1) / WV;  // weight tiles a wave loads per k-tile
  constexpr int D = WV == 4 ? (NS <= 4 ? 12 : 8) : (NS <= 4 ? 8 : 4);   // k-tiles in flight
  static_assert(D % 4 == 0, "ring depth (a multiple of the 4 LDS slots)");
  constexpr int DW = D, DA = D;
  // (the wave index through readfirstlane: its rows, their pointers and the
  // live-rows test stay scalar, 2-12 fewer VGPRs; batch of 8: QKV 55.6 ->
  // 53.5 us; 13B LM head 75.5 -> 74.4 on one box, unchanged on another)
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  int g, ks, pz;
  wg_coords(g, ks, pz);
  const int m0 = pz * 16 * MW * WV;
  const int mw = m0 + 16 * MW * wave;      // the wave's first row
  const bool rows_live = mw < p.M;         // wave-uniform
  const int nkt = p.K / KT, ntiles = (p.N + 15) >> 4;
  const int n0 = g * 16 * NS;

  // A of the wave: its m-tiles' fragments (LM head: A in A-fragment order,
  // frag_index) or its rows (gathered rows: every index load before any use)
  const St* arow[MW];
  if constexpr (EPI == EPI_LM) {
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
      arow[mt] = reinterpret_cast<const St*>(p.A) +
                 ((size_t)min(mw / 16 + mt, p.a_mtiles - 1) * 64 + lane) * PV;
  } else {
    int src[MW];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) src[mt] = min(mw + 16 * mt + li, p.M - 1);
    if (p.a_rows) {
      int raw[MW];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) raw[mt] = p.a_rows[src[mt]];
#pragma unroll
      for (int mt = 0; mt < MW; ++mt) src[mt] = min(max(raw[mt], 0), p.a_nrows - 1);
    }
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
      arow[mt] = reinterpret_cast<const St*>(p.A) + (size_t)src[mt] * p.lda + PV * lq;
  }
  // the wave's weight tiles: t = wave + WV u of the group (loads of t >= NS
  // are clamped and never published); tile (nt, kt) is at kt * ntiles + nt
  const u32x4_t* wbase[NPW];
#pragma unroll
  for (int u = 0; u < NPW; ++u) {
    const int t = min(wave + WV * u, NS - 1);
    wbase[u] = reinterpret_cast<const u32x4_t*>(p.W) + (size_t)min(g * NS + t, ntiles - 1) * 64 +
               lane;
  }
  const size_t kstride = (size_t)ntiles * 64;
  // k-tiles past the end are clamped: every step issues the same loads, and
  // what they bring past the end is never used
  auto load_w = [&](int kt, u32x4_t(&w)[NPW]) {
    const size_t off = (size_t)min(kt, nkt - 1) * kstride;
#pragma unroll
    for (int u = 0; u < NPW; ++u) w[u] = load16_stream(wbase[u] + off);
  };
  auto load_a = [&](int kt, u32x4_t(&a)[MW]) {
    const size_t off = (size_t)min(kt, nkt - 1) * (EPI == EPI_LM ? (size_t)p.a_mtiles * 64 * PV : KT);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) a[mt] = load16(arow[mt] + off);
  };
  __shared__ u32x4_t sW[4][NS][64];
  auto publish = [&](int slot, const u32x4_t(&w)[NPW]) {
#pragma unroll
    for (int u = 0; u < NPW; ++u)
      if (wave + WV * u < NS) sW[slot][wave + WV * u][lane] = w[u];
  };

  floatx4_t acc[MW][NS];
#pragma unroll
  for (int mt = 0; mt < MW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) acc[mt][nt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  u32x4_t wq[DW][NPW], aq[DA][MW];
#pragma unroll
  for (int j = 0; j < DW; ++j) load_w(j, wq[j]);
#pragma unroll
  for (int j = 0; j < DA; ++j) load_a(j, aq[j]);
  // k-tiles 0 and 1 into slots 0 and 1, their registers refilled with
  // k-tiles D and D + 1; then k-tile 0's B fragments
  publish(0, wq[0]);
  load_w(DW, wq[0]);
  publish(1, wq[1]);
  load_w(DW + 1, wq[1]);
  lds_barrier();
  u32x4_t b[NS];
#pragma unroll
  for (int nt = 0; nt < NS; ++nt) b[nt] = sW[0][nt][lane];

  // Step s (j = s mod D): publish k-tile s + 2 (loaded D steps earlier) to
  // slot (s + 2) & 3, last read two barriers ago, and refill its registers
  // with k-tile s + 2 + D; read k-tile s + 1's B fragments (slot (s + 1) & 3,
  // published before the last barrier); multiply k-tile s with the
  // fragments read in the previous step (A from aq[s mod D]); refill aq
  // with k-tile s + D; one barrier.
  auto step = [&](int s, auto jc) {
    constexpr int j = decltype(jc)::value;
    publish((j + 2) & 3, wq[(j + 2) % DW]);
    load_w(s + 2 + DW, wq[(j + 2) % DW]);
    u32x4_t bn[NS];
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) bn[nt] = sW[(j + 1) & 3][nt][lane];
    if (rows_live) {
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NS; ++nt)
          acc[mt][nt] = mfma16x16x32_bf16(aq[j % DA][mt], b[nt], acc[mt][nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) b[nt] = bn[nt];
    load_a(s + DA, aq[j % DA]);
    lds_barrier();
  };
  int s0 = 0;
  for (; s0 + DW <= nkt; s0 += DW)
    unroll_seq([&](auto jc) { step(s0 + decltype(jc)::value, jc); },
               std::make_integer_sequence<int, DW>{});
  if (s0 < nkt)
    unroll_seq(
        [&](auto jc) {
          if (s0 + decltype(jc)::value < nkt) step(s0 + decltype(jc)::value, jc);
        },
        std::make_integer_sequence<int, DW>{});

  if constexpr (EPI == EPI_QKV) {
    // lanes li and li ^ 8 hold the two elements of a rotation pair; each
    // rotates and stores its own
    int pos[MW][4];
#pragma unroll
    for (int mt = 0; mt < MW; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) pos[mt][j] = p.pos[min(mw + 16 * mt + 4 * lq + j, p.M - 1)];
    const bool second = li >= 8;
#pragma unroll
    for (int nt = 0; nt < NS; ++nt) {
      const int col = n0 + 16 * nt + li;
      const QkvColumn<ET> cq(p, min(col, p.N - 1));
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float other = __shfl_xor(acc[mt][nt][j], 8);
          const int r = mw + 16 * mt + 4 * lq + j;
          if (r < p.M && col < p.N) cq.store_one(r, pos[mt][j], acc[mt][nt][j], other, second);
        }
    }
  } else {
    if (p.logits_out)
#pragma unroll
      for (int mt = 0; mt < MW; ++mt)
#pragma unroll
        for (int nt = 0; nt < NS; ++nt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int r = mw + 16 * mt + 4 * lq + j, col = n0 + 16 * nt + li;
            if (r < p.M && col < p.N) p.logits_out[(size_t)r * p.N + col] = acc[mt][nt][j];
          }
    if (!rows_live) return;
    // tree nodes of the pass's sequences (-1 for roots and past the end)
    const int rows_hi = min(p.M, m0 + 16 * MW * WV);
    const int bl = m0 / max(p.T, 1), bh = (rows_hi - 1) / max(p.T, 1);
    const int nchild = (bh - bl + 1) * p.T;
    constexpr int LW = 16 * NS + 4;        // row stride (floats) of the tile
    __shared__ float lt_s[WV][16][LW];
    float(*lt)[LW] = lt_s[wave];
    const int r = lane & 15, part = lane >> 4;
    constexpr int PC = 4 * NS;              // columns a lane scans
    const int G = gridDim.x;
    // the pass's tree nodes (lane's node e0 + lane of each batch of 64): node,
    // token and parent row, loaded once for all the wave's m-tiles
    constexpr int kChildBatches = 8;        // 512 nodes; more are loaded per m-tile
    int cnode[kChildBatches], ctok[kChildBatches], cpr[kChildBatches];
    auto child_load = [&](int e, int& node, int& tok, int& pr) {
      const int cn = e % p.T;
      node = e < nchild && cn >= 1 ? (bl + e / p.T) * p.T + cn : -1;
      const int nd = max(node, 0);
      tok = p.tokens[nd];
      pr = (nd / p.T) * p.T + min(max(p.parent[nd % p.T], 0), p.T - 1);
    };
#pragma unroll
    for (int q = 0; q < kChildBatches; ++q)
      if (64 * q < nchild) child_load(64 * q + lane, cnode[q], ctok[q], cpr[q]);
#pragma unroll
    for (int mt = 0; mt < MW; ++mt) {
      if (mt > 0) wave_lds_sync();         // the previous tile's reads are done
#pragma unroll
      for (int nt = 0; nt < NS; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j) lt[4 * lq + j][16 * nt + li] = acc[mt][nt][j];
      wave_lds_sync();
      const int g0 = mw + 16 * mt;          // first row of the tile
      const int c0 = n0 + part * PC;
      float bv = kNegInf;
      int bi = 0x7fffffff;
#pragma unroll
      for (int c = 0; c < PC; ++c) {
        const float v = lt[r][part * PC + c];
        if (c0 + c < p.N && v > bv) {
          bv = v;
          bi = c0 + c;
        }
      }
      float sv = 0.f, wv = 0.f;
#pragma unroll
      for (int c = 0; c < PC; ++c)
        if (c0 + c < p.N) {
          const float z = (lt[r][part * PC + c] - bv) * p.inv_tau;
          const float e = exp_e(z);
          sv += e;
          wv += e * z;
        }
      // parts (0, 1) and (2, 3), then the two pairs
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float m2 = __shfl_xor(bv, off), s2 = __shfl_xor(sv, off), w2 = __shfl_xor(wv, off);
        const int a2 = __shfl_xor(bi, off);
        rec_merge(bv, sv, wv, bi, m2, s2, w2, a2, p.inv_tau);
      }
      if (part == 0 && g0 + r < p.M)
        *reinterpret_cast<float4*>(p.part + ((size_t)(g0 + r) * G + g) * 4) =
            make_float4(bv, sv, wv, __int_as_float(bi));
      // logit of each tree node's token under its parent's row, where both
      // fall in this tile
      const int g1 = min(p.M, g0 + 16);
      auto child_store = [&](int node, int tok, int pr) {
        if (node >= 0 && tok >= n0 && tok < n0 + 16 * NS && tok < p.N && pr >= g0 && pr < g1)
          p.child_logit[node] = lt[pr - g0][tok - n0];
      };
#pragma unroll
      for (int q = 0; q < kChildBatches; ++q)
        if (64 * q < nchild) child_store(cnode[q], ctok[q], cpr[q]);
      for (int e0 = 64 * kChildBatches; e0 < nchild; e0 += 64) {
        int node, tok, pr;
        child_load(e0 + lane, node, tok, pr);
        child_store(node, tok, pr);
      }
    }
  }
}

// Row statistics from the G records of row r: 256 threads, thread t takes
// records t + 256 u in u order (every load of a round issued before any is
// used), then a lane butterfly and the four waves in order.
constexpr int kRowMergeThreads = 256;
__global__ __launch_bounds__(kRowMergeThreads) void row_stats_merge_kernel(
    const float* __restrict__ part, int G, float inv_tau, float* __restrict__ row_stats,
    int* __restrict__ row_argmax) {
  __shared__ floatx4_t wr[kRowMergeThreads / 64];
  row_records_merge(part, G, inv_tau, blockIdx.x, threadIdx.x, true, wr, row_stats, row_argmax);
}

// Tile configuration: waves per workgroup (= 16-column stripes), m-tiles
// per pass, k-tiles per A chunk, weight loads in flight per wave.
struct Config {
  int wv, mt, ch, d;
};

// The 48-row tile of the QKV and output projections, and its K slices (0:
// as many as gemm_splits gives). With 2 to 4 sixteen-column stripes per
// compute unit one workgroup of 3 or 4 waves per compute unit streams the
// whole K (no hand-off between workgroups: the 7B QKV, 768 stripes); with
// fewer stripes 4-wave workgroups split K (the 7B output projection, 256
// stripes, 4 slices).
struct SmallConfig {
  Config c;
  int ks;
};
SmallConfig small_config(int N) {
  const int stripes = (N + 15) / 16, cus = device_cus();
  if (stripes > 2 * cus && stripes <= 3 * cus) return SmallConfig{{3, 3, 8, 16}, 1};
  if (stripes > 3 * cus && stripes <= 4 * cus) return SmallConfig{{4, 3, 8, 16}, 1};
  return SmallConfig{{4, 3, 4, 8}, 0};
}

Config config_for(int M, int N, int epi) {
  if (M <= 48) {
    // LM head: one 8-wave workgroup per compute unit, 16 weight loads in
    // flight per wave, no K split (split variants measured slower: the
    // 4-wave workgroups they need read the tree rows from L2 twice as often)
    if (epi == EPI_LM) return Config{8, 3, 8, 16};
    return small_config(N).c;
  }
  // The output projection of more than 48 rows: passes of 48 rows, 8-wave
  // workgroups (128 columns) with 16 weight loads in flight per wave; the
  // passes of a column group run on one XCD and share its weight reads in
  // L2 (vicuna13b 136 rows: 25.1 us where one 192-row pass took 39.9, its
  // eight waves each reading twelve A tiles from LDS every k-tile).
  if (epi == EPI_OPROJ) return Config{8, 3, 8, 16};
  // QKV and LM head of more rows where the row-split kernel does not apply
  // (fp32): 8-wave workgroups of 12 m-tiles (A chunks of 48 KB, double
  // buffered) with 4 weight loads in flight per wave (8 spills registers
  // and measured no faster)
  return Config{8, 12, 4, 4};
}

template <class ET, int EPI>
hipError_t launch_main(const GemmParams& p, int KS, hipStream_t st) {
  const Config c = config_for(p.M, p.N, EPI);
  const int groups = (p.N + 16 * c.wv - 1) / (16 * c.wv);
  const int passes = (p.M + 16 * c.mt - 1) / (16 * c.mt);
  dim3 grid(groups, KS, passes), block(64 * c.wv);
  if (c.mt == 3 && c.wv == 3)
    hipLaunchKernelGGL((node_gemm_kernel<ET, 3, 3, 8, 16, EPI>), grid, block, 0, st, p);
  else if (c.mt == 3 && c.wv == 4 && c.d == 16)
    hipLaunchKernelGGL((node_gemm_kernel<ET, 4, 3, 8, 16, EPI>), grid, block, 0, st, p);
  else if (c.mt == 3 && c.wv == 4)
    hipLaunchKernelGGL((node_gemm_kernel<ET, 4, 3, 4, 8, EPI>), grid, block, 0, st, p);
  else if (c.mt == 3)
    hipLaunchKernelGGL((node_gemm_kernel<ET, 8, 3, 8, 16, EPI>), grid, block, 0, st, p);
  else
    hipLaunchKernelGGL((node_gemm_kernel<ET, 8, 12, 4, 4, EPI>), grid, block, 0, st, p);
  return hipGetLastError();
}

// Shape of the row-split kernel (bf16 QKV projection or LM head of more than
// 48 rows): WV waves of 48 rows -- 4 (one pass of 192 rows) up to 192 rows,
// else 8 (passes of 384) -- and NS stripes a workgroup -- the fewest of 3,
// 4, 8 whose column groups fit one workgroup per compute unit, else 8.
struct RowsCfg {
  int wv, ns;
};
bool rows_config(int M, int N, int epi, bool f32, RowsCfg& c) {
  if (f32 || M <= 48 || (epi != EPI_QKV && epi != EPI_LM)) return false;
  const int stripes = (N + 15) / 16, cus = device_cus();
  if (epi == EPI_QKV && M > 192) {
    // several passes of 192 rows (the passes of a column group share its
    // weight reads in L2) when 3, 4 or 6 stripes a workgroup fit one
    // workgroup per compute unit
    const int passes = (M + 191) / 192;
    for (int ns : {3, 4, 6})
      if ((stripes + ns - 1) / ns * passes <= cus) {
        c.wv = 4;
        c.ns = ns;
        return true;
      }
  }
  c.wv = M <= 192 ? 4 : 8;
  c.ns = 8;
  for (int ns : {3, 4, 8})
    if ((stripes + ns - 1) / ns <= cus) {
      c.ns = ns;
      break;
    }
  return true;
}

template <int EPI>
hipError_t launch_rows(const GemmParams& p, const RowsCfg& c, hipStream_t st) {
  const dim3 grid((p.N + 16 * c.ns - 1) / (16 * c.ns), 1, (p.M + 48 * c.wv - 1) / (48 * c.wv));
  const dim3 block(64 * c.wv);
#define ROWS_CASE(WV_, NS_)                                                                    \
  if (c.wv == WV_ && c.ns == NS_) {                                                            \
    hipLaunchKernelGGL((node_gemm_rows_kernel<WV_, NS_, EPI>), grid, block, 0, st, p);         \
    return hipGetLastError();                                                                  \
  }
  ROWS_CASE(4, 3)
  ROWS_CASE(4, 4)
  if constexpr (EPI == EPI_QKV) ROWS_CASE(4, 6)
  ROWS_CASE(4, 8)
  ROWS_CASE(8, 3)
  ROWS_CASE(8, 4)
  ROWS_CASE(8, 8)
#undef ROWS_CASE
  return hipErrorInvalidValue;
}

template <int EPI>
hipError_t launch_split(GemmParams p, hipStream_t st) {
  if constexpr (EPI == EPI_QKV) {
    RowsCfg rc;
    if (rows_config(p.M, p.N, EPI, p.f32, rc)) return launch_rows<EPI>(p, rc, st);
  }
  const int KS = gemm_splits(EPI, p.N, p.K, p.f32, p.M);
  p.group_cols = 16 * config_for(p.M, p.N, EPI).wv;
  return p.f32 ? launch_main<F32, EPI>(p, KS, st) : launch_main<BF16, EPI>(p, KS, st);
}

}  // namespace

// Records per row the LM head writes: one per (row, 16-column stripe), or
// with the row-split kernel one per (row, workgroup).
int lm_head_blocks(int N, int M, bool f32) {
  RowsCfg rc;
  if (rows_config(M, N, EPI_LM, f32, rc)) return (N + 16 * rc.ns - 1) / (16 * rc.ns);
  const Config c = config_for(M, N, EPI_LM);
  return (N + 16 * c.wv - 1) / (16 * c.wv) * c.wv;
}
int lm_record_slots(int N) { return (N + 15) / 16 + 8; }
int gemm_groups_max(int N) { return (N + 15) / 16; }
int gemm_passes_max(int M) { return (M + 47) / 48; }

size_t packed_weight_bytes(int rows, int K, bool f32) {
  return (size_t)((rows + 15) / 16) * 16 * K * (f32 ? 4 : 2);
}

hipError_t launch_pack_weight(bool f32, const void* W, int rows, int K, int pair_dh, void* out,
                              hipStream_t st) {
  const size_t pieces = packed_weight_bytes(rows, K, f32) / 16;
  const int threads = 256;
  const size_t blocks = (pieces + threads - 1) / threads;
  if (f32)
    hipLaunchKernelGGL(pack_weight_kernel<F32>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const float*>(W), rows, K, pair_dh,
                       static_cast<u32x4_t*>(out), pieces);
  else
    hipLaunchKernelGGL(pack_weight_kernel<BF16>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const uint16_t*>(W), rows, K, pair_dh,
                       static_cast<u32x4_t*>(out), pieces);
  return hipGetLastError();
}

// Slices of K: the count the tile configuration fixes, else the smallest
// power of two that gives the grid at least kGemmMinWaves waves (4 per
// compute unit); either way every wave keeps at least 8 k-tiles per slice.
constexpr int kGemmMinWaves = 1024;
int gemm_splits(int epi, int N, int K, bool f32, int M) {
  const int nkt = K / (f32 ? 16 : 32);
  int ks = 1;
  if (M > 48) {
    // split K while the grid still fits one workgroup per compute unit
    const Config c = config_for(M, N, epi);
    const int wgs = (N + 16 * c.wv - 1) / (16 * c.wv) * ((M + 16 * c.mt - 1) / (16 * c.mt));
    // (two a unit measured slower: 13B output projection 35.5 against 25.0 us)
    while (wgs * ks * 2 <= device_cus() && nkt / (ks * 2) >= 8 && ks < kMaxSplits) ks *= 2;
    return ks;
  }
  const int forced = small_config(N).ks;
  const int stripes = (N + 15) / 16;
  if (forced > 0) {
    while (ks * 2 <= forced && nkt / (ks * 2) >= 8 && ks < kMaxSplits) ks *= 2;
    return ks;
  }
  while (stripes * ks < kGemmMinWaves && nkt / (ks * 2) >= 8 && ks < kMaxSplits) ks *= 2;
  return ks;
}

hipError_t launch_qkv(const GemmParams& p, hipStream_t st) { return launch_split<EPI_QKV>(p, st); }

hipError_t launch_oproj(const GemmParams& p, hipStream_t st) {
  return launch_split<EPI_OPROJ>(p, st);
}

hipError_t launch_row_stats_merge(const float* part, int G, int M, float inv_tau,
                                  float* row_stats, int* row_argmax, hipStream_t st) {
  hipLaunchKernelGGL(row_stats_merge_kernel, dim3(M), dim3(kRowMergeThreads), 0, st, part, G,
                     inv_tau, row_stats, row_argmax);
  return hipGetLastError();
}

hipError_t launch_lm_head(GemmParams p, float* row_stats, int* row_argmax, hipStream_t st,
                          bool merge_rows) {
  p.group_cols = 16 * config_for(p.M, p.N, EPI_LM).wv;
  RowsCfg rc;
  hipError_t e;
  if (rows_config(p.M, p.N, EPI_LM, p.f32, rc))
    e = launch_rows<EPI_LM>(p, rc, st);
  else
    e = p.f32 ? launch_main<F32, EPI_LM>(p, 1, st) : launch_main<BF16, EPI_LM>(p, 1, st);
  if (e != hipSuccess || !merge_rows) return e;
  hipLaunchKernelGGL(row_stats_merge_kernel, dim3(p.M), dim3(kRowMergeThreads), 0, st, p.part,
                     lm_head_blocks(p.N, p.M, p.f32), p.inv_tau, row_stats, row_argmax);
  return hipGetLastError();
}

}  // namespace medusa
