// Tree attention on gfx950 ("Medusa: Faster LLM text generation", Tree
// attention; "Medusa 深读", §6.1): every tree node attends to the whole
// prefix KV cache and to its own ancestors (and itself) among the tree nodes.
//
// Split-KV (flash-decoding) layout: workgroup (s, h, b) handles prefix keys
// [s*C, (s+1)*C), C = kAttnChunk, for all T queries of (b, h), and leaves an
// unnormalised partial (m, l, O) per query (m in log2 units of the scaled
// score; O of a split stored [dh tile][query][16], so that a wave's 16x16
// output tile is one contiguous 1 KB store). The merge kernel, one wave per (b, query, h), combines the splits
// in order and then adds the query's tree keys -- the nodes the ancestor
// mask allows, at most the tree depth plus one of them, so a few dot
// products per query -- in increasing node order.
//
// bf16 prefix kernel (8 waves, 32 keys each; as many workgroups as fit the
// device at once, each looping over chunks s, s + G, ... of its (b, h) with
// the next chunk's K and V loads in flight while it computes the current):
//   * S^T = K Q^T on MFMA: the K fragments (A operand, 16 keys x 32 dh) are
//     16-byte pieces of cache rows, loaded straight into registers; each
//     wave scores its own 32 keys against all query tiles.
//   * Exact softmax over the chunk: per-query maxima and sums of the 8 waves
//     meet in LDS (fixed order).
//   * P (bf16) goes to LDS, V rows to LDS (row-major, padded); then the
//     waves split O^T = V^T P^T by output dh tile: the A operand (16 dh x 32
//     keys of V^T) comes from gfx950's transposing LDS read
//     (ds_read_b64_tr_b16), the B operand (32 keys x 16 queries of P^T) is
//     one 16-byte LDS read, P being stored in the key order the transposing
//     read produces. No wave has to reduce another's O.
// fp32 prefix kernel (4 waves, one query tile per wave, online softmax over
// rounds of keys staged in LDS) for fp32 storage.
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

constexpr int kPfxWaves = 8;   // waves of the bf16 prefix kernel, 32 keys each
static_assert(kPfxWaves * 32 == kAttnChunk, "one 32-key MFMA step per wave");

// QG query tiles are processed per pass over a chunk. With QH > QG the Q
// rows of all (at most QH) query tiles are held in LDS for the whole kernel,
// loaded once; with QH == QG a query group's rows are reloaded for every
// chunk when the tree has more than QG tiles.
// ACC: the workgroup folds its chunks into one running partial (for trees of
// several query groups, or workgroups that loop over more than two chunks);
// otherwise every chunk leaves its own partial at its chunk index (one query
// group only).
template <int DH, int QG, int QH, bool ACC>
__global__ __launch_bounds__(64 * kPfxWaves) void prefix_attn_bf16_kernel(AttnArgs a) {
  using S = uint16_t;
  static_assert(64 * kPfxWaves == 512, "Q staging assumes 512 threads");
  constexpr int DS = DH / 32;             // 32-element k-steps of q.k
  constexpr int DT = DH / 16;             // output dh tiles
  constexpr int VP = DH / 8;              // 16-byte pieces per key row
  constexpr int VL = 32 * VP / 64;        // V pieces per lane (32 keys per wave)
  constexpr int VSTR = DH + 16;           // V row stride in LDS: 288 / 160 bytes keep the
                                          // transposing reads conflict-free
  constexpr int PSTR = kAttnChunk + 8;    // P row stride in LDS (528 bytes)
  constexpr int QSTR = DH + 8;            // Q row stride in LDS (272 / 144 bytes)
  constexpr int ITEMS = (QG * DT + kPfxWaves - 1) / kPfxWaves;   // (query tile, dh tile) per wave
  constexpr int QPIECES = 16 * QG * VP;   // 16-byte pieces of a query group's Q rows
  constexpr int QR = (QPIECES + 511) / 512;
  const int h = blockIdx.y, b = blockIdx.z, G = gridDim.x;
  const int T = a.T, H = a.H;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  int s = blockIdx.x;   // chunks s, s + G, ... of (b, h)
  if (s * kAttnChunk >= L) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int MQ = (T + 15) / 16;
  constexpr bool kHold = QH > QG;
  const bool one_group = kHold || MQ <= QG;   // Q stays in LDS for every chunk
  const float sl2 = a.scale * kLog2e;

  __shared__ S qs[16 * QH][QSTR];
  __shared__ S vs[kAttnChunk][VSTR];
  __shared__ S ps[16 * QG][PSTR];
  __shared__ float red_m[kPfxWaves][16 * QG];
  __shared__ float red_l[kPfxWaves][16 * QG];

  const size_t head = ((size_t)b * H + h) * a.Lmax;
  const S* __restrict__ kc = reinterpret_cast<const S*>(a.k_cache) + head * DH;
  const S* __restrict__ vc = reinterpret_cast<const S*>(a.v_cache) + head * DH;
  const S* __restrict__ qb = reinterpret_cast<const S*>(a.q);

  // Q rows of query tiles g0 .. g0 + QG - 1, one 16-byte piece per thread and round
  auto load_q = [&](int g0, u32x4_t(&qv)[QR]) {
#pragma unroll
    for (int r = 0; r < QR; ++r) {
      const int p = min((int)threadIdx.x + 512 * r, QPIECES - 1), qr = p / VP, c = p - qr * VP;
      const int qi = min(16 * g0 + qr, T - 1);
      qv[r] = load16(qb + (((size_t)b * T + qi) * H + h) * DH + 8 * c);
    }
  };
  // this wave's 32 keys of a chunk (rows past L are read clamped and masked later):
  // K fragments (A operand), key 16 kt + li, dh 8 lq + 32 ds .. + 7; V rows, piece
  // p = lane + 64 i at key p / VP, dh 8 (p % VP)
  auto load_kv = [&](int chunk, u32x4_t(&kf)[2][DS], u32x4_t(&vv)[VL]) {
    const int key0 = chunk * kAttnChunk + 32 * wave;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kf[kt][ds] = load16(kc + (size_t)min(key0 + 16 * kt + li, L - 1) * DH + 8 * lq + 32 * ds);
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int p = lane + 64 * i, kk = p / VP, c = p - kk * VP;
      vv[i] = load16(vc + (size_t)min(key0 + kk, L - 1) * DH + 8 * c);
    }
  };

  u32x4_t qv[QR];
  if constexpr (kHold) {
    // every query tile's rows, once (rows past T read clamped, never used)
    constexpr int QPA = 16 * QH * VP, QRA = (QPA + 511) / 512;
#pragma unroll
    for (int r = 0; r < QRA; ++r) {
      const int p = threadIdx.x + 512 * r;
      const int pc = min(p, QPA - 1), qr = pc / VP, c = pc - qr * VP;
      const u32x4_t v = load16(qb + (((size_t)b * T + min(qr, T - 1)) * H + h) * DH + 8 * c);
      if (p < QPA) *reinterpret_cast<u32x4_t*>(&qs[qr][8 * c]) = v;
    }
  } else {
    load_q(0, qv);
  }
  // Running (max, sum, output) of every query over this workgroup's chunks
  // (online softmax: a chunk's own exact softmax is folded in with the
  // rescaling 2^(M_old - M_new)); one partial per workgroup at the end.
  // Output tiles of group gi live in orun[gi] (the group loop is unrolled).
  constexpr int NGR = !ACC ? 1 : kHold ? (QH + QG - 1) / QG : (QG < 4 ? 1 : (MAXT / 16) / QG);
  constexpr int NRQ = 16 * QG * NGR;   // query rows with running statistics
  __shared__ float run_m[NRQ], run_l[NRQ];
  floatx4_t orun[NGR][ITEMS];
#pragma unroll
  for (int gi = 0; gi < NGR; ++gi)
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) orun[gi][it] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if (ACC)
    for (int i = threadIdx.x; i < NRQ; i += 64 * kPfxWaves) {
      run_m[i] = kNegInf;
      run_l[i] = 0.f;
    }
  // (published by the first barrier below)

  u32x4_t kf[2][DS], vv[VL];
  load_kv(s, kf, vv);
  for (bool first = true;; first = false) {
    const int key0 = s * kAttnChunk + 32 * wave;
    const int sn = s + G;
    const bool more = sn * kAttnChunk < L;
#pragma unroll
    for (int i = 0; i < VL; ++i) {
      const int p = lane + 64 * i, kk = p / VP, c = p - kk * VP;
      *reinterpret_cast<u32x4_t*>(&vs[32 * wave + kk][8 * c]) = vv[i];
    }
    u32x4_t kn[2][DS], vn[VL];
    if (more) load_kv(sn, kn, vn);   // next chunk in flight during this one

#pragma unroll
    for (int gi = 0; gi < NGR; ++gi) {
      const int g0 = gi * QG;
      if (g0 >= MQ) continue;   // uniform over the workgroup
      if (kHold) {
        if (first && g0 == 0) __syncthreads();   // the held Q rows are published
      } else if (first || !one_group) {
        if (g0 > 0 || !first) load_q(g0, qv);
#pragma unroll
        for (int r = 0; r < QR; ++r) {
          const int p = threadIdx.x + 512 * r, qr = p / VP, c = p - qr * VP;
          if (p < QPIECES) *reinterpret_cast<u32x4_t*>(&qs[qr][8 * c]) = qv[r];
        }
        __syncthreads();   // Q rows of the group published
      }
      // ---- S^T: lane holds keys key0 + 16 kt + 4 lq + j of query 16 (g0 + u) + li ----
      floatx4_t st[2][QG];
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        // Q fragments of tile u (B operand): query 16 (g0 + u) + li, dh 8 lq + 32 ds .. + 7
        // (held rows: tile g0 + u, clamped into the held tiles; tiles past
        // the tree compute values that are never stored)
        const int qrow = kHold ? 16 * min(g0 + u, QH - 1) + li : 16 * u + li;
        u32x4_t qf[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          qf[ds] = *reinterpret_cast<const u32x4_t*>(&qs[qrow][8 * lq + 32 * ds]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          st[kt][u] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            st[kt][u] = mfma16x16x32_bf16(kf[kt][ds], qf[ds], st[kt][u]);
        }
      }
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = key0 + 16 * kt + 4 * lq + j < L;
            const float v = ok ? st[kt][u][j] * sl2 : kNegInf;
            st[kt][u][j] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (lq == 0) red_m[wave][16 * u + li] = mx;
      }
      __syncthreads();   // maxima (and the chunk's V rows) published
      // ---- P = 2^(s - M) over the chunk; row sums; P to LDS in the transposed-read key order ----
#pragma unroll
      for (int u = 0; u < QG; ++u) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kPfxWaves; ++w) M = fmaxf(M, red_m[w][16 * u + li]);
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pv = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(st[kt][u][j] - M);
            st[kt][u][j] = pv;
            ls += pv;
          }
        ls += __shfl_xor(ls, 16);
        ls += __shfl_xor(ls, 32);
        if (lq == 0) red_l[wave][16 * u + li] = ls;
        // key 32 wave + 16 kt + 4 lq + j sits at column 32 wave + 8 lq + 4 kt + j
        u32x4_t pw;
        pw[0] = pack_bf16x2(st[0][u][0], st[0][u][1]);
        pw[1] = pack_bf16x2(st[0][u][2], st[0][u][3]);
        pw[2] = pack_bf16x2(st[1][u][0], st[1][u][1]);
        pw[3] = pack_bf16x2(st[1][u][2], st[1][u][3]);
        *reinterpret_cast<u32x4_t*>(&ps[16 * u + li][32 * wave + 8 * lq]) = pw;
      }
      __syncthreads();   // P and the row sums are published
      // chunk statistics of query row 16 g0 + rl of the group, and the
      // rescaling factors of the running and the chunk's values
      const auto fold = [&](int rl, float& Mn, float& ca, float& cb, float& lc) {
        float Mc = kNegInf;
        lc = 0.f;
#pragma unroll
        for (int w = 0; w < kPfxWaves; ++w) {
          Mc = fmaxf(Mc, red_m[w][rl]);
          lc += red_l[w][rl];
        }
        const float Mr = run_m[16 * g0 + rl];
        Mn = fmaxf(Mr, Mc);
        ca = Mr == kNegInf ? 0.f : __builtin_amdgcn_exp2f(Mr - Mn);
        cb = Mc == kNegInf ? 0.f : __builtin_amdgcn_exp2f(Mc - Mn);
      };
      // ---- O^T += V^T P^T: item = wave + 8 it is (query tile item / DT, dh tile item % DT) ----
#pragma unroll
      for (int it = 0; it < ITEMS; ++it) {
        const int item = wave + kPfxWaves * it;
        const int u = item / DT, dt = item - u * DT;
        if (item >= QG * DT || g0 + u >= MQ) continue;
        floatx4_t o = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < kAttnChunk / 32; ++t) {
          // A: lane gets dh 16 dt + li of keys 32t + 4 lq + (0..3) and 32t + 16 + 4 lq + (0..3)
          const S* v0 = &vs[32 * t + 4 * lq + (li >> 2)][16 * dt + 4 * (li & 3)];
          const uint2 lo = lds_read_tr16(v0);
          const uint2 hi = lds_read_tr16(v0 + 16 * VSTR);
          u32x4_t vf;
          vf[0] = lo.x;
          vf[1] = lo.y;
          vf[2] = hi.x;
          vf[3] = hi.y;
          const u32x4_t pf = *reinterpret_cast<const u32x4_t*>(&ps[16 * u + li][32 * t + 8 * lq]);
          o = mfma16x16x32_bf16(vf, pf, o);
        }
        // lane holds O^T[dh 16 dt + 4 lq + j][query 16 (g0 + u) + li]
        if constexpr (ACC) {
          float Mn, ca, cb, lc;
          fold(16 * u + li, Mn, ca, cb, lc);
#pragma unroll
          for (int j = 0; j < 4; ++j) orun[gi][it][j] = orun[gi][it][j] * ca + o[j] * cb;
        } else {
          const int query = 16 * (g0 + u) + li;
          const size_t base = ((size_t)b * H + h) * a.NS * T + (size_t)s * T;
          if (query < T)
            *reinterpret_cast<float4*>(a.part_o + base * DH + ((size_t)dt * T + query) * 16 +
                                       4 * lq) = make_float4(o[0], o[1], o[2], o[3]);
        }
      }
      if constexpr (!ACC) {
        // this chunk's statistics (one group: the next writes of red_m and
        // red_l come after the barrier that ends the chunk)
        if (wave == 0 && lane < 16 * QG) {
          const int query = 16 * g0 + lane;
          if (query < T) {
            float M = kNegInf, l = 0.f;
#pragma unroll
            for (int w = 0; w < kPfxWaves; ++w) M = fmaxf(M, red_m[w][lane]);
#pragma unroll
            for (int w = 0; w < kPfxWaves; ++w) l += red_l[w][lane];
            const size_t base = ((size_t)b * H + h) * a.NS * T + (size_t)s * T;
            a.part_ml[(base + query) * 2 + 0] = M;
            a.part_ml[(base + query) * 2 + 1] = l;
          }
        }
        continue;
      }
      // the group's running statistics: every read above happens before the
      // barrier, wave 0 writes after it (so the next group's writes of red_m
      // and these reads do not overlap)
      float nm = kNegInf, nl = 0.f;
      if (wave == 0 && lane < 16 * QG) {
        float Mn, ca, cb, lc;
        fold(lane, Mn, ca, cb, lc);
        nm = Mn;
        nl = run_l[16 * g0 + lane] * ca + lc * cb;
      }
      __syncthreads();
      if (wave == 0 && lane < 16 * QG) {
        run_m[16 * g0 + lane] = nm;
        run_l[16 * g0 + lane] = nl;
      }
    }
    if (!more) break;
    s = sn;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kf[kt][ds] = kn[kt][ds];
#pragma unroll
    for (int i = 0; i < VL; ++i) vv[i] = vn[i];
    __syncthreads();   // every wave is done with this chunk's V, P and row statistics
  }
  if constexpr (!ACC) return;
  // this workgroup's partial: slot blockIdx.x of (b, h)
  __syncthreads();   // the last running statistics are published
  const size_t base = ((size_t)b * H + h) * a.NS * T + (size_t)blockIdx.x * T;
#pragma unroll
  for (int gi = 0; gi < NGR; ++gi) {
    const int g0 = gi * QG;
    if (g0 >= MQ) continue;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = wave + kPfxWaves * it;
      const int u = item / DT, dt = item - u * DT;
      const int query = 16 * (g0 + u) + li;
      if (item >= QG * DT || g0 + u >= MQ || query >= T) continue;
      *reinterpret_cast<float4*>(a.part_o + base * DH + ((size_t)dt * T + query) * 16 + 4 * lq) =
          make_float4(orun[gi][it][0], orun[gi][it][1], orun[gi][it][2], orun[gi][it][3]);
    }
  }
  for (int query = threadIdx.x; query < min(T, NRQ); query += 64 * kPfxWaves) {
    a.part_ml[(base + query) * 2 + 0] = run_m[query];
    a.part_ml[(base + query) * 2 + 1] = run_l[query];
  }
}

// Prefix chunks of sequence `lane` (0 past B; B <= 64, one per lane) and
// their sum over the wave, for the balanced split of the per-wave kernel.
// (the load is clamped rather than branched around, so that it issues
// beside the caller's other loads)
__device__ __forceinline__ int lane_chunks(const AttnArgs& a, int lane) {
  const int n = attn_chunks(a.kv_len[min(lane, a.B - 1)], a.Lmax);
  return lane < a.B ? n : 0;
}
// Weight of one (b, h) segment's start (its Q loads, the first chunk's
// exposed load latency, the closing exchange and partial store) in the
// balanced split, in half chunks: a chunk weighs 2. Measured on the batch of
// 8 (7B): a segment costs about one and a half chunks.
constexpr int kSegWeight = 3;
// Weight of sequence b's H segments of nch chunks (none without chunks).
__device__ __forceinline__ int seq_weight(int H, int nch) {
  return nch > 0 ? H * (kSegWeight + 2 * nch) : 0;
}
// Sum over the wave of non-negative integers whose total is below 2^24
// (the launcher bounds the balanced weights far below that): every partial
// sum is then exact in fp32, and the DPP row sums need no LDS round trips.
__device__ __forceinline__ int wave_sum_int(int v) {
  return (int)wave_sum((float)v);
}

// Per-wave split-KV kernel for 128-wide heads, one group of at most three
// query tiles a workgroup (trees of more tiles run a workgroup set per
// group): wave w of a workgroup takes keys 32 w .. 32 w + 31 of each of its
// chunks and keeps its own running softmax (max, sum, output) for every
// query of the group, so that a chunk needs no exchange between the waves
// and no barrier: S^T = K Q^T (K fragments from memory, Q fragments
// from LDS); P = 2^(s - m) stays in registers, packed in the key order of
// the transposing read, as the B operand of O^T += V^T P^T (V^T read from
// the wave's own V rows in LDS); the next chunk's K and V loads go out into
// the registers the current one has finished with. The eight states are
// combined once, at the end of each segment (a run of chunks of one (b, h)),
// into that segment's partial: maxima and sums
// through LDS (each wave then scales its outputs), and the outputs summed
// over the waves in wave order, wave w owning dh tile w.
template <int QT, bool BAL>
__global__ __launch_bounds__(64 * kPfxWaves) void prefix_attn_wave_kernel(AttnArgs a) {
  using S = uint16_t;
  constexpr int DH = 128, DS = DH / 32, DT = DH / 16, VP = DH / 8, VL = 32 * VP / 64;
  constexpr int VSTR = DH + 16, QSTR = DH + 8;
  static_assert(DT == kPfxWaves, "wave w owns dh tile w of the partial");
  constexpr int kQBytes = 16 * QT * QSTR * 2, kVBytes = kPfxWaves * 32 * VSTR * 2;
  constexpr int kXBytes = kPfxWaves * (DT / 2) * QT * 64 * 16;   // half the dh tiles of every wave
  constexpr int kLdsBytes = kQBytes + kVBytes > kXBytes ? kQBytes + kVBytes : kXBytes;
  // One-dimensional grid over units and query groups qg (tiles 3 qg ..
  // 3 qg + QT - 1): linear id 8 nqg j + 8 qg + i is unit 8 j + i, so that a
  // unit's query groups have ids 8 apart (one XCD, at about the same time:
  // its chunks are read from HBM once and from the L2 by the others). With
  // one group, unit = linear id.
  // Strided units (b, h, s), s < G = chunk_sets: chunks s, s + G, ... of
  // (b, h), one partial at slot s. Balanced units (several sequences of
  // ragged prefixes): the C chunks of all (b, h), in (b, h, chunk) order,
  // are cut into min(G, C) contiguous ranges of floor(C / G) or one more;
  // unit w takes range w and leaves one partial per (b, h) it meets, at the
  // slot of its first chunk there (attn_merge_kernel finds the same slots).
  const int nqg = a.qgroups, G = a.chunk_sets;
  const int lin = blockIdx.x, blk = lin / (8 * nqg), within = lin - blk * 8 * nqg;
  const int qg = within >> 3, unit = 8 * blk + (within & 7);
  const int q0 = 48 * qg;
  const int T = a.T, H = a.H;
  const float sl2 = a.scale * kLog2e;
  // the Q rows and each wave's V rows during the chunks; the outputs' exchange after them
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
  __shared__ float st_m[kPfxWaves][16 * QT], st_l[kPfxWaves][16 * QT];
  S* qs = reinterpret_cast<S*>(lds);                                   // [16 QT][QSTR]
  const S* __restrict__ qb = reinterpret_cast<const S*>(a.q);

  // Chunks first, first + stride, ... (at most through `last`) of (b, h)
  // into the partial at `slot`. Every thread of the workgroup runs the same
  // segments; the LDS is free on entry.
  auto segment = [&](int b, int h, int first, int stride, int last,
                     int slot) __attribute__((always_inline)) {
    // lane indices taken afresh in each segment, so that the addressing
    // built from them is not held in registers across segments
    const int tid = opaque((int)threadIdx.x);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int li = lane & 15, lq = lane >> 4;
    const int L = min(max(a.kv_len[b], 0), a.Lmax);
    const size_t head = ((size_t)b * H + h) * a.Lmax;
    const S* __restrict__ kc = reinterpret_cast<const S*>(a.k_cache) + head * DH;
    const S* __restrict__ vc = reinterpret_cast<const S*>(a.v_cache) + head * DH;
    S* vw = reinterpret_cast<S*>(lds + kQBytes) + wave * 32 * VSTR;   // this wave's [32][VSTR]
    // this wave's 32 keys of a chunk (rows past L are read clamped and masked
    // later): K fragments (A operand), key 16 kt + li, dh 8 lq + 32 ds .. + 7;
    // V rows, piece p = lane + 64 i at key p / VP, dh 8 (p % VP)
    auto load_kv = [&](int chunk, u32x4_t(&kf)[2][DS], u32x4_t(&vv)[VL]) {
      const int key0 = chunk * kAttnChunk + 32 * wave;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          kf[kt][ds] = load16(kc + (size_t)min(key0 + 16 * kt + li, L - 1) * DH + 8 * lq + 32 * ds);
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int p = lane + 64 * i, kk = p / VP, c = p - kk * VP;
        vv[i] = load16(vc + (size_t)min(key0 + kk, L - 1) * DH + 8 * c);
      }
    };
    int s = first;
    u32x4_t kf[2][DS], vv[VL];
    load_kv(s, kf, vv);
    {
      // every query tile's rows, once (rows past T read clamped, never used)
      constexpr int QP = 16 * QT * VP, QRN = (QP + 64 * kPfxWaves - 1) / (64 * kPfxWaves);
#pragma unroll
      for (int r = 0; r < QRN; ++r) {
        const int p = threadIdx.x + 64 * kPfxWaves * r;
        const int pc = min(p, QP - 1), qr = pc / VP, c = pc - qr * VP;
        const u32x4_t v =
            load16(qb + (((size_t)b * T + min(q0 + qr, T - 1)) * H + h) * DH + 8 * c);
        if (p < QP) *reinterpret_cast<u32x4_t*>(qs + qr * QSTR + 8 * c) = v;
      }
    }
    floatx4_t o[QT][DT];
    float m_run[QT], l_run[QT];   // of query 16 u + li
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      m_run[u] = kNegInf;
      l_run[u] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[u][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();   // the Q rows are published
    for (;;) {
      const int key0 = s * kAttnChunk + 32 * wave;
      const int sn = s + stride;
      const bool more = sn <= last && sn * kAttnChunk < L;
      // the V rows into this wave's rows (its reads of the previous chunk's
      // came first: one wave's LDS operations run in order)
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int p = lane + 64 * i, kk = p / VP, c = p - kk * VP;
        *reinterpret_cast<u32x4_t*>(vw + kk * VSTR + 8 * c) = vv[i];
      }
      // ---- S^T: lane holds keys key0 + 16 kt + 4 lq + j of query 16 u + li ----
      floatx4_t st[2][QT];
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        u32x4_t qf[DS];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
          qf[ds] = *reinterpret_cast<const u32x4_t*>(qs + (16 * u + li) * QSTR + 8 * lq + 32 * ds);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          st[kt][u] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            st[kt][u] = mfma16x16x32_bf16(kf[kt][ds], qf[ds], st[kt][u]);
        }
      }
      // the next chunk's loads, into the registers this one is done with
      if (more) load_kv(sn, kf, vv);
      // ---- running softmax of each query over the wave's keys; P^T in registers ----
      u32x4_t pw[QT];
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        float mc = kNegInf;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool ok = key0 + 16 * kt + 4 * lq + j < L;
            const float v = ok ? st[kt][u][j] * sl2 : kNegInf;
            st[kt][u][j] = v;
            mc = fmaxf(mc, v);
          }
        mc = fmaxf(mc, __shfl_xor(mc, 16));
        mc = fmaxf(mc, __shfl_xor(mc, 32));
        const float mn = fmaxf(m_run[u], mc);
        const float alpha = m_run[u] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[u] - mn);
        float rs = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pv = mn == kNegInf ? 0.f : __builtin_amdgcn_exp2f(st[kt][u][j] - mn);
            st[kt][u][j] = pv;
            rs += pv;
          }
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
        l_run[u] = l_run[u] * alpha + rs;
        m_run[u] = mn;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[u][dt][j] *= alpha;
        // key 16 kt + 4 lq + j of the wave's 32 at B-operand position 8 lq + 4 kt + j
        pw[u][0] = pack_bf16x2(st[0][u][0], st[0][u][1]);
        pw[u][1] = pack_bf16x2(st[0][u][2], st[0][u][3]);
        pw[u][2] = pack_bf16x2(st[1][u][0], st[1][u][1]);
        pw[u][3] = pack_bf16x2(st[1][u][2], st[1][u][3]);
      }
      // ---- O^T += V^T P^T over the wave's 32 keys ----
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // A: lane gets dh 16 dt + li of keys 4 lq + (0..3) and 16 + 4 lq + (0..3)
        const S* v0 = vw + (4 * lq + (li >> 2)) * VSTR + 16 * dt + 4 * (li & 3);
        const uint2 lo = lds_read_tr16(v0);
        const uint2 hi = lds_read_tr16(v0 + 16 * VSTR);
        u32x4_t vf;
        vf[0] = lo.x;
        vf[1] = lo.y;
        vf[2] = hi.x;
        vf[3] = hi.y;
#pragma unroll
        for (int u = 0; u < QT; ++u) o[u][dt] = mfma16x16x32_bf16(vf, pw[u], o[u][dt]);
      }
      if (!more) break;
      s = sn;
    }
    // ---- the eight states into the partial at `slot` ----
    if (lq == 0)
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        st_m[wave][16 * u + li] = m_run[u];
        st_l[wave][16 * u + li] = l_run[u];
      }
    __syncthreads();   // every wave is past its chunks (Q and V rows free) and its state is in
    float Mq[QT], Lq[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int q = 16 * u + li;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kPfxWaves; ++w) M = fmaxf(M, st_m[w][q]);
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kPfxWaves; ++w) {
        const float mw = st_m[w][q];
        l += mw == kNegInf ? 0.f : st_l[w][q] * __builtin_amdgcn_exp2f(mw - M);
      }
      Mq[u] = M;
      Lq[u] = l;
      const float c = m_run[u] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[u] - M);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[u][dt][j] *= c;
    }
    const size_t base = ((size_t)b * H + h) * a.NS * T + (size_t)slot * T;
    floatx4_t* xb = reinterpret_cast<floatx4_t*>(lds);   // [wave][DT / 2][QT][64]
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();   // the first half's sums are read
#pragma unroll
      for (int d4 = 0; d4 < DT / 2; ++d4)
#pragma unroll
        for (int u = 0; u < QT; ++u)
          xb[((wave * (DT / 2) + d4) * QT + u) * 64 + lane] = o[u][(DT / 2) * half + d4];
      __syncthreads();
      if (wave / (DT / 2) == half) {
        const int d4 = wave % (DT / 2), dt = wave;
#pragma unroll
        for (int u = 0; u < QT; ++u) {
          floatx4_t acc = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = 0; w < kPfxWaves; ++w) {
            const floatx4_t x = xb[((w * (DT / 2) + d4) * QT + u) * 64 + lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += x[j];
          }
          const int query = q0 + 16 * u + li;
          if (query < T)
            *reinterpret_cast<float4*>(a.part_o + base * DH + ((size_t)dt * T + query) * 16 +
                                       4 * lq) = make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
      }
    }
    if (wave == 0 && lq == 0)
#pragma unroll
      for (int u = 0; u < QT; ++u) {
        const int query = q0 + 16 * u + li;
        if (query < T) {
          a.part_ml[(base + query) * 2 + 0] = Mq[u];
          a.part_ml[(base + query) * 2 + 1] = Lq[u];
        }
      }
  };

  if constexpr (!BAL) {
    // strided: one segment
    if (unit >= G * a.H * a.B) return;
    const int s = unit % G, h = (unit / G) % a.H, b = unit / (G * a.H);
    if (s * kAttnChunk >= min(max(a.kv_len[b], 0), a.Lmax)) return;
    segment(b, h, s, G, 0x7fffffff, s);
  } else {
    // balanced: the (b, h) with chunks lie in order, each weighing
    // kSegWeight + 2 nch, T in all; unit u takes the weights
    // [u T / NWe, (u + 1) T / NWe) and each chunk whose last weight falls in
    // them (chunk j of a (b, h) at P: weight P + kSegWeight + 2 j + 1), so
    // that every unit carries about the same chunks plus segment starts.
    // Every sequence's chunk count at once, one a lane (the walk below
    // reads them back with readlane).
    const int nl = lane_chunks(a, (int)threadIdx.x & 63);
    const int C = H * __builtin_amdgcn_readfirstlane(wave_sum_int(nl));
    const int Tw = __builtin_amdgcn_readfirstlane(wave_sum_int(seq_weight(H, nl)));
    const int NWe = min(G, C);
    if (unit >= NWe) return;
    // (divisions run on the vector ALUs: their uniform results are moved
    // back to scalar registers)
    int x = __builtin_amdgcn_readfirstlane((int)((long long)unit * Tw / NWe));
    const int hi = __builtin_amdgcn_readfirstlane((int)((long long)(unit + 1) * Tw / NWe));
    int b = 0, pb = 0, nch = __builtin_amdgcn_readlane(nl, 0);
    while (x < hi) {
      while (x >= pb + seq_weight(H, nch)) {   // the sequence of weight x (x < Tw)
        pb += seq_weight(H, nch);
        ++b;
        nch = __builtin_amdgcn_readlane(nl, b);
      }
      const int wh = kSegWeight + 2 * nch;
      const int h = __builtin_amdgcn_readfirstlane((x - pb) / wh);
      const int P = pb + h * wh;
      const int off = x - P, e = min(hi - P, wh);
      const int first = off > kSegWeight ? (off - kSegWeight) / 2 : 0;
      const int last = e >= kSegWeight + 2 ? (e - kSegWeight - 2) / 2 : -1;
      x = P + e;
      if (last < first) continue;   // the range ends before this (b, h)'s first chunk
      segment(__builtin_amdgcn_readfirstlane(b), h, first, 1, last, first);
      __syncthreads();   // the segment's exchange is read before the LDS is reused
    }
  }
}

// fp32 prefix kernel: SC keys per round are staged in LDS (K row-major, V
// transposed); the next round's global loads are in flight while the waves
// compute the current one. Waves split the query tiles (16 queries each);
// S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x4_f32, online softmax.
template <int DH, int QT, int SC>
__global__ __launch_bounds__(256) void prefix_attn_f32_kernel(AttnArgs a) {
  constexpr int DS = DH / 16;          // 16-byte steps along Dh per lane group
  constexpr int DT = DH / 16;          // dh tiles of the output
  constexpr int KT = SC / 16;          // key tiles per round
  constexpr int PAD = 4;               // 16 bytes of padding per LDS row
  constexpr int VEC_PER_KEY = DH / 4;
  constexpr int LOADS = SC * VEC_PER_KEY / 256;   // 16-byte loads per thread per tensor
  static_assert(LOADS * 256 == SC * VEC_PER_KEY, "round must divide over the threads");
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, H = a.H;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  const int kbeg = s * kAttnChunk, kend = min(L, kbeg + kAttnChunk);
  if (kbeg >= kend) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int MQ = (T + 15) / 16;
  const float sl2 = a.scale * kLog2e;

  const float* __restrict__ q = reinterpret_cast<const float*>(a.q);
  const float* __restrict__ k_src =
      reinterpret_cast<const float*>(a.k_cache) + ((size_t)b * H + h) * a.Lmax * DH;
  const float* __restrict__ v_src =
      reinterpret_cast<const float*>(a.v_cache) + ((size_t)b * H + h) * a.Lmax * DH;

  __shared__ float ks[SC][DH + PAD];
  __shared__ float vt[DH][SC + PAD];

  u32x4_t qf[QT][DS];
  floatx4_t o[QT][DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qi = min(16 * (wave + 4 * u) + li, T - 1);
    const float* qp = q + (((size_t)b * T + qi) * H + h) * DH + 4 * lq;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[u][ds] = load16(qp + 16 * ds);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[u][dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m_run[u] = kNegInf;
    l_run[u] = 0.f;
  }

  // global loads of one round (keys past the range read a valid row; masked later)
  u32x4_t kv[LOADS], vv[LOADS];
  auto load_round = [&](int kb) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int kk = c / VEC_PER_KEY, part = c - kk * VEC_PER_KEY;
      const size_t off = (size_t)min(kb + kk, kend - 1) * DH + 4 * part;
      kv[i] = load16(k_src + off);
      vv[i] = load16(v_src + off);
    }
  };
  load_round(kbeg);

  for (int kb = kbeg; kb < kend; kb += SC) {
    if (kb > kbeg) __syncthreads();   // previous round's readers are done
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int kk = c / VEC_PER_KEY, part = c - kk * VEC_PER_KEY;
      *reinterpret_cast<u32x4_t*>(&ks[kk][4 * part]) = kv[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[4 * part + e][kk] = __uint_as_float(vv[i][e]);
    }
    __syncthreads();
    if (kb + SC < kend) load_round(kb + SC);   // next round in flight during compute

#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int qt = wave + 4 * u;
      if (qt >= MQ) break;
      floatx4_t st[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        st[kt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const float* kp = &ks[16 * kt + li][4 * lq];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kp + 16 * ds);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            st[kt] = mfma16x16x4_f32(__uint_as_float(kf[j]), __uint_as_float(qf[u][ds][j]),
                                     st[kt]);
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = kb + 16 * kt + 4 * lq + r < kend;
          const float v = ok ? st[kt][r] * sl2 : kNegInf;
          st[kt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[u], mx);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run[u] - m_new);
      float ls = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = m_new == kNegInf ? 0.f : __builtin_amdgcn_exp2f(st[kt][r] - m_new);
          st[kt][r] = pv;
          ls += pv;
        }
      ls += __shfl_xor(ls, 16);
      ls += __shfl_xor(ls, 32);
      l_run[u] = l_run[u] * alpha + ls;
      m_run[u] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[u][dt][j] *= alpha;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float4 vr = *reinterpret_cast<const float4*>(&vt[16 * dt + li][16 * kt + 4 * lq]);
          o[u][dt] = mfma16x16x4_f32(vr.x, st[kt][0], o[u][dt]);
          o[u][dt] = mfma16x16x4_f32(vr.y, st[kt][1], o[u][dt]);
          o[u][dt] = mfma16x16x4_f32(vr.z, st[kt][2], o[u][dt]);
          o[u][dt] = mfma16x16x4_f32(vr.w, st[kt][3], o[u][dt]);
        }
    }
  }

  const size_t base = (((size_t)b * H + h) * a.NS + s) * T;
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qt = wave + 4 * u;
    if (qt >= MQ) break;
    const int query = 16 * qt + li;
    if (query >= T) continue;
    if (lq == 0) {
      a.part_ml[(base + query) * 2 + 0] = m_run[u];
      a.part_ml[(base + query) * 2 + 1] = l_run[u];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(a.part_o + base * DH + ((size_t)dt * T + query) * 16 + 4 * lq) =
          make_float4(o[u][dt][0], o[u][dt][1], o[u][dt][2], o[u][dt][3]);
  }
}

// Merge, one wave per (b, query i, h), each lane holding DH / 64 consecutive
// dh: the prefix splits in order, then the tree keys j the mask allows for
// i, in increasing j, all folded into one running (max, sum, weighted
// value). Loads go out in two waves of requests: the query row, the first
// kMergeBatch splits and the first 64 mask bytes together, then the key and
// value rows of the first kTreeBatch tree keys; further batches (long
// prefixes, wide trees) follow the same pattern. Split indices past the last
// are clamped and given zero weight.
constexpr int kMergeBatch = 8;

constexpr int kTreeBatch = 8;
template <class ET, int DH, bool BAL, int MW>
__global__ __launch_bounds__(64 * MW) void attn_merge_kernel(AttnArgs a) {
  using S = typename ET::storage;
  constexpr int E = DH / 64;
  // (the wave index through readfirstlane, so that the compiler knows i,
  // and the early exit below, to be uniform)
  const int i = blockIdx.x * MW + (MW > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0);
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, H = a.H;
  if (i >= T) return;   // wave-uniform; the kernel has no barriers
  // the query row and the first mask window, loaded ahead of the split
  // bookkeeping below (all three loads in flight together)
  const S* __restrict__ qp = reinterpret_cast<const S*>(a.q) + (((size_t)b * T + i) * H + h) * DH;
  const uint8_t* __restrict__ mrow = a.mask + (size_t)i * T;
  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = ET::load1(qp + E * lane + e);
  const bool allow0 = mrow[min(lane, T - 1)] != 0 && lane < T;
  // every sequence's prefix length, one a lane (B <= 64), by a vector load
  // that issues beside the query and mask loads above (a scalar load of
  // kv_len[b] would be waited for before any of them)
  const int kvl = a.kv_len[min(lane, a.B - 1)];
  const int L = min(max(__builtin_amdgcn_readlane(kvl, b), 0), a.Lmax);
  // partials: one per prefix workgroup that had a chunk (strided units:
  // slots 0 .. ns - 1). Balanced units: this (b, h) weighs kSegWeight + 2 nch
  // from P of the Tw in order, its chunk j's last weight at
  // P + kSegWeight + 2 j + 1; the unit whose range [u Tw / NWe,
  // (u + 1) Tw / NWe) holds weight p is ceil((p + 1) NWe / Tw) - 1. The ns
  // units from wa hold its chunks (each at least one, as a range spans at
  // least two weights) and left their partials at the slot of their first
  // chunk here. ((NWe + 64) Tw < 2^32, which the launcher checks, so 32-bit
  // unsigned products.)
  const int nch = attn_chunks(L, a.Lmax);
  int ns = min(a.NP, nch);
  unsigned wa = 0, NWe = 1, Tw = 1, P = 0;
  if constexpr (BAL) {
    // every sequence's chunks at once, one a lane
    const int nl = lane < a.B ? attn_chunks(kvl, a.Lmax) : 0;
    const unsigned C = H * (unsigned)__builtin_amdgcn_readfirstlane(wave_sum_int(nl));
    Tw = (unsigned)__builtin_amdgcn_readfirstlane(wave_sum_int(seq_weight(H, nl)));
    P = (unsigned)__builtin_amdgcn_readfirstlane(wave_sum_int(lane < b ? seq_weight(H, nl) : 0)) +
        h * (unsigned)(kSegWeight + 2 * nch);
    NWe = min((unsigned)a.chunk_sets, C);
    ns = 0;
    if (nch > 0) {
      wa = ((P + kSegWeight + 2) * NWe + Tw - 1) / Tw - 1;
      ns = (int)(((P + kSegWeight + 2 * nch) * NWe + Tw - 1) / Tw - wa);
    }
  }
  // (balanced: lane j computes partial j's slot once: the first chunk whose
  // last weight is at or past the unit's range start)
  auto slot_of = [&](unsigned j) -> int {
    const unsigned lo = (wa + j) * Tw / NWe;
    return lo <= P + kSegWeight ? 0 : (int)((lo - P - kSegWeight) / 2);
  };
  const int slot_l = BAL ? slot_of(lane) : 0;
  auto slot = [&](int j) -> int {
    if constexpr (BAL)
      return j < 64 ? __builtin_amdgcn_readlane(slot_l, j) : slot_of(j);
    else
      return j;
  };
  const float sl2 = a.scale * kLog2e;
  const size_t hs = ((size_t)b * H + h) * a.NS;   // split 0 of (b, h)
  // dh E lane + e of query i inside a split's [DT][T][16] block
  const size_t oin = ((size_t)(E * lane / 16) * T + i) * 16 + (E * lane) % 16;
  const S* __restrict__ ktr = reinterpret_cast<const S*>(a.k_tree) + ((size_t)b * T * H + h) * DH;
  const S* __restrict__ vtr = reinterpret_cast<const S*>(a.v_tree) + ((size_t)b * T * H + h) * DH;
  const size_t krow = (size_t)H * DH;

  float ms[kMergeBatch], lsv[kMergeBatch], os[kMergeBatch][E];
  auto load_splits = [&](int s0) {
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const size_t sp = hs + slot(min(s0 + j, max(ns - 1, 0)));
      ms[j] = a.part_ml[(sp * T + i) * 2];
      lsv[j] = a.part_ml[(sp * T + i) * 2 + 1];
#pragma unroll
      for (int e = 0; e < E; ++e) os[j][e] = a.part_o[sp * T * DH + oin + e];
    }
  };
  int js[kTreeBatch];
  float kx[kTreeBatch][E], vx[kTreeBatch][E];
  // the next (up to) kTreeBatch keys of window j0 out of `bits`, rows loaded
  auto take_tree = [&](int j0, uint64_t& bits) {
    int nb = 0;
#pragma unroll
    for (int u = 0; u < kTreeBatch; ++u) {
      js[u] = bits ? j0 + __ffsll((unsigned long long)bits) - 1 : js[0];
      if (bits) {
        bits &= bits - 1;
        nb = u + 1;
      }
    }
#pragma unroll
    for (int u = 0; u < kTreeBatch; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        kx[u][e] = ET::load1(ktr + js[u] * krow + E * lane + e);
        vx[u][e] = ET::load1(vtr + js[u] * krow + E * lane + e);
      }
    return nb;
  };

  if (ns > 0) load_splits(0);
  uint64_t bits = __ballot(allow0);
  int nb = bits ? take_tree(0, bits) : 0;

  float M = kNegInf, l = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    if (s0 > 0) load_splits(s0);
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (s0 + j < ns) Mn = fmaxf(Mn, ms[j]);
    const float c = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    l *= c;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= c;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool live = s0 + j < ns && ms[j] != kNegInf;
      const float w = live ? __builtin_amdgcn_exp2f(ms[j] - Mn) : 0.f;
      l += w * lsv[j];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += w * os[j][e];
    }
    M = Mn;
  }

  // the tree keys of query i
  for (int j0 = 0;;) {
    for (int u = 0; u < nb; ++u) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d += qv[e] * kx[u][e];
      const float sc = wave_sum(d) * sl2;
      const float Mn = fmaxf(M, sc);
      const float c = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
      const float w = __builtin_amdgcn_exp2f(sc - Mn);
      l = l * c + w;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = acc[e] * c + w * vx[u][e];
      M = Mn;
    }
    while (!bits) {
      j0 += 64;
      if (j0 >= T) break;
      bits = __ballot(j0 + lane < T && mrow[j0 + lane] != 0);
    }
    if (!bits) break;
    nb = take_tree(j0, bits);
  }

  const float inv = 1.f / l;
  const size_t out = (((size_t)b * T + i) * H + h) * DH + E * lane;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float ov = acc[e] * inv;
    if (a.out) a.out[out + e] = ov;
    if (a.out_elem) reinterpret_cast<S*>(a.out_elem)[out + e] = ET::from_float(ov);
  }
}

// The merge, MW queries (one a wave) a workgroup: four when it has under
// eight waves a compute unit (7B tree, 1440 waves: 6.3 -> 5.5 us), else one
// (13B tree and batch of 8, 5440 and 11520 waves: four measured 0.2-0.4 us
// slower).
template <class ET, int DH, bool BAL>
void launch_merge(const AttnArgs& m, hipStream_t st) {
  if ((long long)m.T * m.H * m.B < 8ll * device_cus())
    hipLaunchKernelGGL((attn_merge_kernel<ET, DH, BAL, 4>), dim3((m.T + 3) / 4, m.H, m.B), dim3(256),
                       0, st, m);
  else
    hipLaunchKernelGGL((attn_merge_kernel<ET, DH, BAL, 1>), dim3(m.T, m.H, m.B), dim3(64), 0, st, m);
}

constexpr int kHeldTiles = 9;   // query tiles whose Q rows the bf16 kernel can hold

// Trees of 5-9 query tiles hold every query row in LDS when the device gives
// a workgroup the kernel's LDS (151 KB for 128-wide heads); else each query
// group's rows are reloaded per chunk.
template <int DH>
bool attn_hold_q_for() {
  static const bool v = [] {
    int dev = 0, lim = 0;
    hipFuncAttributes fa{};
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(
                                      prefix_attn_bf16_kernel<DH, 4, kHeldTiles, true>)) != hipSuccess)
      return false;
    return fa.sharedSizeBytes <= (size_t)lim;
  }();
  return v;
}

template <int DH>
hipError_t launch_bf16(const AttnArgs& a, hipStream_t st) {
  const auto attn_hold_q = [] { return attn_hold_q_for<DH>(); };
  const int MQ = (a.T + 15) / 16;
  // one workgroup per compute unit (its LDS use allows no second): chunks
  // per (b, h) in flight = CUs / (B H), each workgroup looping over the rest.
  // With several sequences and at most one workgroup per (sequence, head),
  // one workgroup would loop over every chunk of its sequence and ragged
  // prefixes would leave compute units idle while the longest finish: then
  // 4x as many workgroups are launched, so that those of short prefixes
  // finish early and free their units (a second round of workgroups
  // measured 2-4x slower for one sequence).
  const int cus = device_cus();
  const int over = a.B > 1 && cus <= a.B * a.H ? 4 : 1;
  int G = over * cus / (a.B * a.H);
  G = G < 1 ? 1 : (G > a.NS ? a.NS : G);
  dim3 grid(G, a.H, a.B), block(64 * kPfxWaves);
  AttnArgs m = a;
  // A workgroup that loops over more than two chunks, or a tree of more
  // than one query group, folds its chunks into one partial; otherwise each
  // chunk leaves its own.
  const bool acc = MQ > 4 || a.NS > 2 * G;
  m.NP = acc ? G : a.NS;
  if constexpr (DH == 128) {
    // workgroups that loop over chunks, trees of at most three query tiles:
    // the per-wave kernel (one partial per workgroup). With one chunk a
    // workgroup its closing exchange costs more than the barriers it saves
    // (7B: 15.2 against 12.1 us).
    if (acc && MQ <= 3) {
      m.NP = G;
      AttnArgs w = a;
      w.qgroups = 1;
      w.chunk_sets = G;
      w.balanced = 0;
      if (a.B > 1 && (long long)(cus + 64) * a.B * a.H * (2 * a.NS + kSegWeight) < (1ll << 32)) {
        // several sequences: one balanced range of the chunks of every
        // (b, h) per compute unit, so that ragged prefixes leave no unit idle
        // (batch of 8, 7B: 79.8 -> 70.6 us; with segment starts weighed in,
        // 67.7 -> 57.1 us)
        w.balanced = 1;
        w.chunk_sets = cus;
      }
      m.balanced = w.balanced;
      m.chunk_sets = w.chunk_sets;
      const dim3 wgrid(w.balanced ? (cus + 7) / 8 * 8 : (G * a.H * a.B + 7) / 8 * 8);
#define WAVE_CASES(BAL)                                                                      \
  switch (MQ) {                                                                              \
    case 1: hipLaunchKernelGGL((prefix_attn_wave_kernel<1, BAL>), wgrid, block, 0, st, w); break; \
    case 2: hipLaunchKernelGGL((prefix_attn_wave_kernel<2, BAL>), wgrid, block, 0, st, w); break; \
    default: hipLaunchKernelGGL((prefix_attn_wave_kernel<3, BAL>), wgrid, block, 0, st, w); break; \
  }
      if (w.balanced)
        WAVE_CASES(true)
      else
        WAVE_CASES(false)
#undef WAVE_CASES
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (w.balanced)
        launch_merge<BF16, DH, true>(m, st);
      else
        launch_merge<BF16, DH, false>(m, st);
      return hipGetLastError();
    }
    if (MQ > 3) {
      // larger trees: a set of workgroups per group of three query tiles,
      // each set reading the same chunks (from L2 or the Infinity Cache for
      // all but one), as many chunk sets as fill the compute units once
      const int nqg = (MQ + 2) / 3;
      int G2 = cus / (nqg * a.B * a.H);
      G2 = G2 < 1 ? 1 : (G2 > a.NS ? a.NS : G2);
      AttnArgs w = a;
      w.qgroups = nqg;
      w.chunk_sets = G2;
      w.balanced = 0;
      m.NP = G2;
      const dim3 wgrid((G2 * a.H * a.B + 7) / 8 * 8 * nqg);
      hipLaunchKernelGGL((prefix_attn_wave_kernel<3, false>), wgrid, block, 0, st, w);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      launch_merge<BF16, DH, false>(m, st);
      return hipGetLastError();
    }
  }
  // 5 to 9 query tiles: all Q rows held in LDS (151 KB with the V and P
  // buffers for 128-wide heads), so no query group is reloaded per chunk
  if (MQ > 4 && MQ <= kHeldTiles && attn_hold_q())
    hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 4, kHeldTiles, true>), grid, block, 0, st, a);
  else if (MQ > 4)
    hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 4, 4, true>), grid, block, 0, st, a);
  else if (acc)
    switch (MQ) {
      case 1: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 1, 1, true>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 2, 2, true>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 3, 3, true>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 4, 4, true>), grid, block, 0, st, a); break;
    }
  else
    switch (MQ) {
      case 1: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 1, 1, false>), grid, block, 0, st, a); break;
      case 2: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 2, 2, false>), grid, block, 0, st, a); break;
      case 3: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 3, 3, false>), grid, block, 0, st, a); break;
      default: hipLaunchKernelGGL((prefix_attn_bf16_kernel<DH, 4, 4, false>), grid, block, 0, st, a); break;
    }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_merge<BF16, DH, false>(m, st);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_f32(const AttnArgs& a, hipStream_t st) {
  // 128-wide heads stage 64 keys per round to keep LDS below 68 KB
  constexpr int SC = DH == 128 ? 64 : 128;
  const int MQ = (a.T + 15) / 16;
  const int QT = (MQ + 3) / 4;
  dim3 grid(a.NS, a.H, a.B), block(256);
  switch (QT) {
    case 1: hipLaunchKernelGGL((prefix_attn_f32_kernel<DH, 1, SC>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefix_attn_f32_kernel<DH, 2, SC>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((prefix_attn_f32_kernel<DH, 3, SC>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((prefix_attn_f32_kernel<DH, 4, SC>), grid, block, 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnArgs m = a;
  m.NP = a.NS;   // one partial per chunk
  launch_merge<F32, DH, false>(m, st);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

int attn_splits(int Lmax) { return Lmax > 0 ? (Lmax + kAttnChunk - 1) / kAttnChunk : 1; }

hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.f32) return a.Dh == 64 ? launch_f32<64>(a, st) : launch_f32<128>(a, st);
  return a.Dh == 64 ? launch_bf16<64>(a, st) : launch_bf16<128>(a, st);
}

}  // namespace medusa
