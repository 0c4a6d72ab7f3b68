// Device helpers shared by the gfx950 kernels of the Medusa verify step.
//
// Wavefronts are 64 lanes. Cross-lane reductions use DPP inside 16-lane rows
// (quad permutes and row rotations) and DPP row broadcasts across rows, the
// GFX9-family forms that gfx950 keeps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace medusa {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---- bf16 <-> fp32 ----------------------------------------------------------

// Low / high bf16 of a packed pair, widened exactly to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float round_to_bf16(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

// ---- element type traits ----------------------------------------------------
// Weights, embeddings and the KV cache are stored as bf16 (uint16 bits) or
// fp32. A 16-byte vector load carries 8 bf16 or 4 fp32 elements.

struct BF16 {
  typedef uint16_t storage;
  static constexpr int kPerVec = 8;
  __device__ __forceinline__ static void widen(const u32x4_t& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16lo(v[i]);
      out[2 * i + 1] = bf16hi(v[i]);
    }
  }
  __device__ __forceinline__ static float load1(const storage* p) {
    return __uint_as_float(((uint32_t)*p) << 16);
  }
  // the bits of one element, widened to 32 (converted later by from_raw)
  __device__ __forceinline__ static uint32_t load_raw(const storage* p) { return *p; }
  __device__ __forceinline__ static float from_raw(uint32_t r) { return __uint_as_float(r << 16); }
  __device__ __forceinline__ static storage from_float(float f) {
    return (storage)f32_to_bf16_bits(f);
  }
  __device__ __forceinline__ static float round(float f) { return round_to_bf16(f); }
};

struct F32 {
  typedef float storage;
  static constexpr int kPerVec = 4;
  __device__ __forceinline__ static void widen(const u32x4_t& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static float load1(const storage* p) { return *p; }
  __device__ __forceinline__ static uint32_t load_raw(const storage* p) { return __float_as_uint(*p); }
  __device__ __forceinline__ static float from_raw(uint32_t r) { return __uint_as_float(r); }
  __device__ __forceinline__ static storage from_float(float f) { return f; }
  __device__ __forceinline__ static float round(float f) { return f; }
};

// An empty asm that claims to change v: arithmetic on a prefetched value
// placed after it cannot be hoisted up to the load (where it would wait for
// the data before later loads are issued); the wait for the load lands here.
template <class T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// 16-byte global load that bypasses nothing special (plain vector load).
__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// Streaming (read-once) 16-byte load: non-temporal hint so the stream does
// not evict reused data from the caches.
__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// ---- direct global -> LDS loads (gfx950) ---------------------------------------
// Each lane names one 16-byte piece in global memory; the wave's 64 pieces
// land in LDS contiguously at `lds` (lane-major), without passing through
// VGPRs. Completion is tracked by the vector-memory counter, so a reader of
// that LDS must first wait with vmcnt() below.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(const_cast<void*>(g), (lds_void_t*)lds, 16, 0, 0);
}
// Wait until at most N vector-memory operations of this wave are in flight
// (GFX9 s_waitcnt encoding: vmcnt low bits [3:0] and high bits [15:14];
// expcnt and lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// vmcnt() with a run-time count (0..63), for pipelines whose tail issues
// fewer loads than their steady state.
__device__ __forceinline__ void vmcnt_rt(int n) {
  switch (n) {
#define MEDUSA_VMCNT_CASE(N) \
  case N:                    \
    vmcnt<N>();              \
    break;
    MEDUSA_VMCNT_CASE(0) MEDUSA_VMCNT_CASE(1) MEDUSA_VMCNT_CASE(2) MEDUSA_VMCNT_CASE(3)
    MEDUSA_VMCNT_CASE(4) MEDUSA_VMCNT_CASE(5) MEDUSA_VMCNT_CASE(6) MEDUSA_VMCNT_CASE(7)
    MEDUSA_VMCNT_CASE(8) MEDUSA_VMCNT_CASE(9) MEDUSA_VMCNT_CASE(10) MEDUSA_VMCNT_CASE(11)
    MEDUSA_VMCNT_CASE(12) MEDUSA_VMCNT_CASE(13) MEDUSA_VMCNT_CASE(14) MEDUSA_VMCNT_CASE(15)
    MEDUSA_VMCNT_CASE(16) MEDUSA_VMCNT_CASE(17) MEDUSA_VMCNT_CASE(18) MEDUSA_VMCNT_CASE(19)
    MEDUSA_VMCNT_CASE(20) MEDUSA_VMCNT_CASE(21) MEDUSA_VMCNT_CASE(22) MEDUSA_VMCNT_CASE(23)
    MEDUSA_VMCNT_CASE(24) MEDUSA_VMCNT_CASE(25) MEDUSA_VMCNT_CASE(26) MEDUSA_VMCNT_CASE(27)
    MEDUSA_VMCNT_CASE(28) MEDUSA_VMCNT_CASE(29) MEDUSA_VMCNT_CASE(30) MEDUSA_VMCNT_CASE(31)
#undef MEDUSA_VMCNT_CASE
    default:
      vmcnt<0>();   // conservative: wait for everything
      break;
  }
}

// Workgroup barrier for LDS-DMA pipelines: s_barrier without the release /
// acquire fence of __syncthreads(), which would drain every outstanding
// direct-to-LDS load (vmcnt 0). The caller waits for its own loads first
// (vmcnt); the compiler-only fences keep LDS accesses on their side.
__device__ __forceinline__ void stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier that publishes this wave's LDS writes (lgkmcnt 0) but
// leaves its global loads in flight (no vmcnt wait, unlike __syncthreads).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Makes this wave's LDS writes visible to its own other lanes: the LDS
// queue of one wave completes in order, so waiting for its writes and
// keeping the compiler from moving accesses across is enough.
__device__ __forceinline__ void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt 0
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---- hand-off between the workgroups of one launch -----------------------------
// The L2 caches of the XCDs are not coherent with each other. Relaxed atomic
// loads and stores at agent scope are: they compile to ordinary vector
// loads and stores with the sc1 cache-policy bit (stores written through to
// the coherent level, loads served from it), with no L2 write-back or
// invalidate. Data that one workgroup hands to another in the same launch
// goes through these, so the hand-off needs no device-wide fence (whose L2
// write-back and invalidate would also evict the weight and activation lines
// the other workgroups are still using).
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int coherent_load(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A-fragment order of a [rows][K] operand of v_mfma_f32_16x16x32_bf16 (PV =
// 8 elements per 16-byte piece) or of four v_mfma_f32_16x16x4_f32 (PV = 4):
// tile (k-tile kt, m-tile mt) is 64 lane pieces of 16 bytes, lane 16 lq + li
// holding row 16 mt + li, elements 4 PV kt + PV lq .. + PV - 1; the tiles of
// a k-tile are adjacent (mtiles of them), so a wave loads one fragment as
// one contiguous 1 KB. Element index of (row r, column c):
__device__ __forceinline__ size_t frag_index(int r, int c, int mtiles, int PV) {
  const int kt = c / (4 * PV), rem = c - kt * 4 * PV, lq = rem / PV;
  return (((size_t)kt * mtiles + (r >> 4)) * 64 + 16 * lq + (r & 15)) * PV + (rem - lq * PV);
}

// Counts the calling workgroup in on `counter` and returns, in every thread,
// whether it is the last of `n` workgroups to arrive; the last one resets the
// counter to zero for the next launch. Every coherent_store of the workgroup
// issued before the call is complete (each wave waits for its vector memory
// operations, vmcnt 0) before the count moves, so the last workgroup's
// coherent_loads afterwards see them all.
__device__ __forceinline__ bool last_to_arrive(int* counter, int n) {
  __shared__ int s_last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  vmcnt<0>();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int before =
        __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == n - 1;
    if (before == n - 1) coherent_store(counter, 0);
  }
  __syncthreads();
  return s_last != 0;
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16). Within each group of 16
// lanes, let lane 4k + q pass the address of 4 consecutive 16-bit elements
// of row R_k (elements c + 4q .. c + 4q + 3): lane i then receives element
// c + i of rows R_0 .. R_3, in that order (as 2 dwords, row R_0 in the low
// half of the first).
typedef short short4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4_t*)(p));
  uint2 r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

// ---- DPP wave reductions ----------------------------------------------------
// DPP control codes (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;   // row_ror:4
constexpr int kDppRowRor8 = 0x128;   // row_ror:8
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Sum over each 16-lane row; every lane of the row gets the row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kDppQuadXor1>(v);
  v += dpp<kDppQuadXor2>(v);
  v += dpp<kDppRowRor4>(v);
  v += dpp<kDppRowRor8>(v);
  return v;
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppQuadXor1>(v));
  v = fmaxf(v, dpp<kDppQuadXor2>(v));
  v = fmaxf(v, dpp<kDppRowRor4>(v));
  v = fmaxf(v, dpp<kDppRowRor8>(v));
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the whole wave, returned to every lane (uniform). Rows are
// combined in a fixed order, so the result does not depend on timing.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// ---- ordering of (logit, token id) candidates --------------------------------
// Higher logit first; equal logits: lower id first.
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// ---- row statistics of a logit row at temperature tau -----------------------
// Record (m, S, W, a): max m, argmax a (lowest id on ties), S = sum
// e^{(l-m)/tau}, W = sum e^{(l-m)/tau} (l-m)/tau over a set of columns.
// Merge of two records (m = -inf marks an empty record).
__device__ __forceinline__ void rec_merge(float& m, float& s, float& w, int& a, float m2,
                                          float s2, float w2, int a2, float inv_tau) {
  if (m2 == -__builtin_huge_valf()) return;
  if (m == -__builtin_huge_valf()) {
    m = m2; s = s2; w = w2; a = a2;
    return;
  }
  const float mn = fmaxf(m, m2);
  const float d1 = (m - mn) * inv_tau, d2 = (m2 - mn) * inv_tau;
  const float c1 = __builtin_amdgcn_exp2f(d1 * 1.4426950408889634f);
  const float c2 = __builtin_amdgcn_exp2f(d2 * 1.4426950408889634f);
  const int an = (m > m2 || (m == m2 && a < a2)) ? a : a2;
  w = c1 * (w + s * d1) + c2 * (w2 + s2 * d2);
  s = c1 * s + c2 * s2;
  m = mn;
  a = an;
}

// Merge of row r's G records part[r][g][4] (m, S, W, argmax bits) by a group
// of 256 threads (t = 0..255 within the group, `wr` 4 LDS slots of its own),
// in a fixed order: thread t its records t, t + 256, ... in turn, a butterfly
// over each wave, then thread 0 the group's 4 waves in order; it writes
// row_stats[r] (m, S, W) and row_argmax[r] when `live`. Every thread of the
// calling workgroup calls it once (one barrier).
__device__ __forceinline__ void row_records_merge(const float* __restrict__ part, int G,
                                                  float inv_tau, int r, int t, bool live,
                                                  floatx4_t* wr, float* __restrict__ row_stats,
                                                  int* __restrict__ row_argmax) {
  constexpr int RB = 8;
  const int lane = t & 63, wave = t >> 6;
  float m = -__builtin_huge_valf(), s = 0.f, w = 0.f;
  int a = 0x7fffffff;
  for (int g0 = 0; g0 < G; g0 += 256 * RB) {
    floatx4_t rec[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int g = min(g0 + t + 256 * u, G - 1);
      rec[u] = *reinterpret_cast<const floatx4_t*>(part + ((size_t)r * G + g) * 4);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (g0 + t + 256 * u < G)
        rec_merge(m, s, w, a, rec[u][0], rec[u][1], rec[u][2], __float_as_int(rec[u][3]),
                  inv_tau);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off), w2 = __shfl_xor(w, off);
    const int a2 = __shfl_xor(a, off);
    rec_merge(m, s, w, a, m2, s2, w2, a2, inv_tau);
  }
  if (lane == 0) wr[wave] = floatx4_t{m, s, w, __int_as_float(a)};
  __syncthreads();
  if (t != 0 || !live) return;
  m = -__builtin_huge_valf();
  s = w = 0.f;
  a = 0x7fffffff;
  for (int i = 0; i < 4; ++i)
    rec_merge(m, s, w, a, wr[i][0], wr[i][1], wr[i][2], __float_as_int(wr[i][3]), inv_tau);
  row_stats[(size_t)r * 3 + 0] = m;
  row_stats[(size_t)r * 3 + 1] = s;
  row_stats[(size_t)r * 3 + 2] = w;
  row_argmax[r] = a;
}

// ---- MFMA ---------------------------------------------------------------------
// v_mfma_f32_16x16x32_bf16: A 16x32, B 32x16, C 16x16 fp32.
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// C[4*(l/16) + j][l%16] for j = 0..3.
__device__ __forceinline__ floatx4_t mfma16x16x32_bf16(const u32x4_t& a, const u32x4_t& b,
                                                       floatx4_t c) {
  bf16x8_t av, bv;
  __builtin_memcpy(&av, &a, 16);
  __builtin_memcpy(&bv, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c, 0, 0, 0);
}
// v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16], B[l/16][l%16].
__device__ __forceinline__ floatx4_t mfma16x16x4_f32(float a, float b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// e^x through the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

}  // namespace medusa
