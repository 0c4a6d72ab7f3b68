// Tree attention on gfx950 ("Medusa: Faster LLM text generation", Tree
// attention; "Medusa 深读", §6.1): every tree node attends to the whole
// prefix KV cache and to its own ancestors (and itself) among the tree nodes.
//
// Split-KV (flash-decoding) layout: workgroup (s, h, b) handles one key
// range -- split 0 is the tree block (T keys under the ancestor mask), split
// s >= 1 covers prefix keys [(s-1)*C, s*C) -- for all T queries of (b, h),
// and leaves an unnormalised partial (m, l, O) per query. A merge kernel
// combines the splits in a fixed order.
//
// Inside a workgroup everything is computed transposed, so that no lane
// shuffles are needed between the two products:
//   S^T = K Q^T     (A = K rows from LDS; B = Q rows, in registers),
//   P^T = 2^(S^T * scale*log2e - m),
//   O^T += V^T P^T  (A = V^T: V rows sit row-major in LDS and gfx950's
//                    transposing LDS read (ds_read_b64_tr_b16) returns each
//                    lane 4 keys of one dh; B = P^T straight from the S^T
//                    accumulators, since the MFMA result layout puts the 4
//                    keys of a lane exactly where the next MFMA's B operand
//                    expects its k slots, up to a permutation shared with A).
// In every accumulator a lane's column is one query, so the online-softmax
// statistics (m, l, rescale factor) of a query live in that lane alone.
// Waves split the query tiles (16 queries each).
#include "common.h"
#include "kernels.h"

namespace medusa {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// SC keys are staged per round: K and V rows go to LDS (row-major, padded)
// with 16-byte stores; the global loads of the next round are in flight
// while the waves compute the current one from LDS.
template <class ET, int DH, int QT, int SC>
__global__ __launch_bounds__(256) void tree_attn_kernel(AttnArgs a) {
  using S = typename ET::storage;
  constexpr int PV = ET::kPerVec;
  constexpr bool BF = PV == 8;
  constexpr int DS = DH / (4 * PV);   // 16-byte steps along Dh per lane group
  constexpr int DT = DH / 16;         // dh tiles of the output
  constexpr int KT = SC / 16;         // key tiles per round
  constexpr int PAD = 16 / sizeof(S); // 16 bytes of padding per LDS row
  constexpr int VEC_PER_KEY = DH / PV;
  constexpr int LOADS = SC * VEC_PER_KEY / 256;   // 16-byte loads per thread per tensor
  static_assert(LOADS * 256 == SC * VEC_PER_KEY, "round must divide over the threads");
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int T = a.T, H = a.H;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  const bool tree = s == 0;
  int kbeg, kend;
  if (tree) {
    kbeg = 0;
    kend = T;
  } else {
    kbeg = (s - 1) * kAttnChunk;
    kend = min(L, s * kAttnChunk);
    if (kbeg >= kend) return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, lq = lane >> 4;
  const int MQ = (T + 15) / 16;
  const float sl2 = a.scale * 1.4426950408889634f;

  const S* __restrict__ q = reinterpret_cast<const S*>(a.q);
  const S* __restrict__ k_src;
  const S* __restrict__ v_src;
  size_t krow;   // elements between consecutive keys
  if (tree) {
    k_src = reinterpret_cast<const S*>(a.k_tree) + ((size_t)b * T * H + h) * DH;
    v_src = reinterpret_cast<const S*>(a.v_tree) + ((size_t)b * T * H + h) * DH;
    krow = (size_t)H * DH;
  } else {
    k_src = reinterpret_cast<const S*>(a.k_cache) + ((size_t)b * H + h) * a.Lmax * DH;
    v_src = reinterpret_cast<const S*>(a.v_cache) + ((size_t)b * H + h) * a.Lmax * DH;
    krow = DH;
  }

  // bf16: V row-major like K (row stride 288 / 160 bytes keeps the
  // transposed reads conflict-free); fp32: V transposed.
  constexpr int PADV = 32 / sizeof(S);
  __shared__ S ks[SC][DH + PAD];
  __shared__ S vt[BF ? SC : DH][BF ? DH + PADV : SC + PAD];

  // Q fragments of my query tiles (B operand: lane = query, 16 B along Dh)
  u32x4_t qf[QT][DS];
  floatx4_t o[QT][DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    const int qt = wave + 4 * u;
    const int qi = min(16 * qt + li, T - 1);
    const S* qp = q + (((size_t)b * T + qi) * H + h) * DH + PV * lq;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) qf[u][ds] = load16(qp + 4 * PV * ds);
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
      const size_t off = (size_t)min(kb + kk, kend - 1) * krow + PV * part;
      kv[i] = load16(k_src + off);
      vv[i] = load16(v_src + off);
    }
  };
  load_round(kbeg);

  for (int kb = kbeg; kb < kend; kb += SC) {
    if (kb > kbeg) __syncthreads();   // previous round's readers are done
    // ---- stage K and V^T ----
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int c = threadIdx.x + 256 * i;
      const int kk = c / VEC_PER_KEY, part = c - kk * VEC_PER_KEY;
      *reinterpret_cast<u32x4_t*>(&ks[kk][PV * part]) = kv[i];
      if constexpr (BF) {
        *reinterpret_cast<u32x4_t*>(&vt[kk][PV * part]) = vv[i];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) vt[PV * part + e][kk] = __uint_as_float(vv[i][e]);
      }
    }
    __syncthreads();
    if (kb + SC < kend) load_round(kb + SC);   // next round in flight during compute

#pragma unroll
    for (int u = 0; u < QT; ++u) {
      const int qt = wave + 4 * u;
      if (qt >= MQ) break;
      const int query = 16 * qt + li;
      // ---- S^T = K Q^T over the round's key tiles ----
      floatx4_t st[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        st[kt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        const S* kp = &ks[16 * kt + li][PV * lq];
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kp + 4 * PV * ds);
          if constexpr (BF) {
            st[kt] = mfma16x16x32_bf16(kf, qf[u][ds], st[kt]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              st[kt] = mfma16x16x4_f32(__uint_as_float(kf[j]), __uint_as_float(qf[u][ds][j]),
                                       st[kt]);
          }
        }
      }
      // ---- scale, mask, online softmax (lane = query) ----
      const uint8_t* mrow = a.mask + (size_t)min(query, T - 1) * T;
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 16 * kt + 4 * lq + r;
          bool ok = key < kend;
          if (tree && ok && query < T) ok = mrow[key] != 0;
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
      // ---- O^T += V^T P^T ----
      if constexpr (BF) {
#pragma unroll
        for (int t = 0; t < KT / 2; ++t) {
          u32x4_t pf;
          pf[0] = pack_bf16x2(st[2 * t][0], st[2 * t][1]);
          pf[1] = pack_bf16x2(st[2 * t][2], st[2 * t][3]);
          pf[2] = pack_bf16x2(st[2 * t + 1][0], st[2 * t + 1][1]);
          pf[3] = pack_bf16x2(st[2 * t + 1][2], st[2 * t + 1][3]);
          // k slot j of this lane group is key 32t + 4lq + j (j < 4) or
          // 32t + 16 + 4lq + j - 4: the S^T accumulator order
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const S* v0 = &vt[32 * t + 4 * lq + (li >> 2)][16 * dt + 4 * (li & 3)];
            u32x4_t vf;
            const uint2 lo = lds_read_tr16(v0);
            const uint2 hi = lds_read_tr16(v0 + 16 * (DH + PADV));
            vf[0] = lo.x;
            vf[1] = lo.y;
            vf[2] = hi.x;
            vf[3] = hi.y;
            o[u][dt] = mfma16x16x32_bf16(vf, pf, o[u][dt]);
          }
        }
      } else {
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
  }

  // ---- partial (m, l, O) per query ----
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
    float* op = a.part_o + (base + query) * DH;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(op + 16 * dt + 4 * lq) =
          make_float4(o[u][dt][0], o[u][dt][1], o[u][dt][2], o[u][dt][3]);
  }
}

// Combine the splits of every (b, query, h): fixed order, tree split first.
// Splits are read in batches of kMergeBatch with every load of a batch
// issued before any is used (indices past the last split are clamped to it
// and given zero weight), so a thread waits once per batch.
constexpr int kMergeBatch = 16;
template <class ET>
__global__ void attn_merge_kernel(AttnArgs a) {
  using S = typename ET::storage;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int x = threadIdx.x;   // one dh element per thread
  const int T = a.T, H = a.H, DH = a.Dh;
  const int L = min(max(a.kv_len[b], 0), a.Lmax);
  const int ns = 1 + (L + kAttnChunk - 1) / kAttnChunk;
  const size_t base = ((size_t)b * H + h) * a.NS * T + i;
  float M = kNegInf, l = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float ms[kMergeBatch], lsv[kMergeBatch], os[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const size_t r = base + (size_t)min(s0 + j, ns - 1) * T;
      ms[j] = a.part_ml[r * 2];
      lsv[j] = a.part_ml[r * 2 + 1];
      os[j] = a.part_o[r * DH + x];
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mn = fmaxf(Mn, ms[j]);
    const float c = M == kNegInf ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
    l *= c;
    acc *= c;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool live = s0 + j < ns && ms[j] != kNegInf;
      const float w = live ? __builtin_amdgcn_exp2f(ms[j] - Mn) : 0.f;
      l += w * lsv[j];
      acc += w * os[j];
    }
    M = Mn;
  }
  const float ov = acc / l;
  const size_t out = (((size_t)b * T + i) * H + h) * DH + x;
  if (a.out) a.out[out] = ov;
  if (a.out_elem) reinterpret_cast<S*>(a.out_elem)[out] = ET::from_float(ov);
}

template <class ET, int DH>
hipError_t launch_dh(const AttnArgs& a, hipStream_t st) {
  // fp32 with 128-wide heads stages 64 keys per round to keep LDS below 68 KB
  constexpr int SC = (sizeof(typename ET::storage) == 4 && DH == 128) ? 64 : 128;
  const int MQ = (a.T + 15) / 16;
  const int QT = (MQ + 3) / 4;
  dim3 grid(a.NS, a.H, a.B), block(256);
  switch (QT) {
    case 1: hipLaunchKernelGGL((tree_attn_kernel<ET, DH, 1, SC>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((tree_attn_kernel<ET, DH, 2, SC>), grid, block, 0, st, a); break;
    case 3: hipLaunchKernelGGL((tree_attn_kernel<ET, DH, 3, SC>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((tree_attn_kernel<ET, DH, 4, SC>), grid, block, 0, st, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel<ET>, dim3(a.T, a.H, a.B), dim3(DH), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int attn_splits(int Lmax) { return 1 + (Lmax + kAttnChunk - 1) / kAttnChunk; }

hipError_t launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.f32) return a.Dh == 64 ? launch_dh<F32, 64>(a, st) : launch_dh<F32, 128>(a, st);
  return a.Dh == 64 ? launch_dh<BF16, 64>(a, st) : launch_dh<BF16, 128>(a, st);
}

}  // namespace medusa
