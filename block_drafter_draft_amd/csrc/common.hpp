// Device helpers shared by the DFlash2 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dflash2.h"

namespace df2 {

constexpr int kTopK = 16;  // candidates per block position

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Results that nothing in the same launch reads again are stored nontemporally: written
// through rather than left dirty in L2, where the end-of-kernel release would have to
// write them back before the next kernel may start.
__device__ __forceinline__ void store_nt(u32x4_t* p, u32x4_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(u32x2_t* p, u32x2_t v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// binary32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------------------
// Order keys for the top-16 order: a larger key comes first. NaN (any sign or payload)
// gets the largest key; -0 gets the key of +0; otherwise the usual sign-magnitude flip.
// Packed candidates are (key << 32) | ~index, so the larger packed value comes first and
// equal keys go to the smaller index. Packed 0 is "no candidate" (no real key is 0).
// ---------------------------------------------------------------------------------------

struct KeyBF16 {
  using elem_t = uint16_t;
  static constexpr uint32_t kNaN = 0xffffu;
  static constexpr uint32_t kPosZero = 0x8000u;
  static constexpr uint32_t kNegZeroRaw = 0x7fffu;
  static constexpr uint32_t kNegInf = 0x007fu;  // lowest non-NaN key
  static constexpr uint32_t kPosInf = 0xff80u;  // highest non-NaN key
  // sign-magnitude flip without NaN/-0 canonicalisation
  __device__ __forceinline__ static uint32_t raw(uint32_t h) {
    return h ^ (0x8000u | ((0u - (h >> 15)) & 0x7fffu));
  }
  __device__ __forceinline__ static uint32_t canon(uint32_t h) {
    if ((h & 0x7fffu) > 0x7f80u) return kNaN;
    if (h == 0x8000u) h = 0;
    return raw(h);
  }
  __device__ __forceinline__ static float widen(uint32_t h) { return bf16_to_f32(h); }
};

struct KeyF32 {
  using elem_t = float;
  static constexpr uint32_t kNaN = 0xffffffffu;
  static constexpr uint32_t kPosZero = 0x80000000u;
  static constexpr uint32_t kNegZeroRaw = 0x7fffffffu;
  static constexpr uint32_t kNegInf = 0x007fffffu;
  static constexpr uint32_t kPosInf = 0xff800000u;
  __device__ __forceinline__ static uint32_t raw(uint32_t u) {
    return u ^ (0x80000000u | (0u - (u >> 31)));
  }
  __device__ __forceinline__ static uint32_t canon(uint32_t u) {
    if ((u & 0x7fffffffu) > 0x7f800000u) return kNaN;
    if (u == 0x80000000u) u = 0;
    return raw(u);
  }
  __device__ __forceinline__ static float widen(uint32_t u) { return __uint_as_float(u); }
};

__device__ __forceinline__ uint64_t pack_cand(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ uint32_t cand_idx(uint64_t p) { return ~(uint32_t)p; }
__device__ __forceinline__ uint32_t cand_key(uint64_t p) { return (uint32_t)(p >> 32); }

// ---------------------------------------------------------------------------------------
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): key (seed, 0), counter
// (step, b, j, 0). Word 0: walk uniform of slot j; word 1: accept uniform of proposal j;
// word 2: residual/bonus draw for the token emitted at position j.
// ---------------------------------------------------------------------------------------

struct Draw {
  uint64_t w[4];
};

__device__ inline Draw philox_draw(uint64_t seed, uint64_t step, uint32_t b, uint32_t j) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = step, x1 = b, x2 = j, x3 = 0;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    uint64_t hi_a = __umul64hi(M0, x0), lo_a = M0 * x0;
    uint64_t hi_b = __umul64hi(M1, x2), lo_b = M1 * x2;
    uint64_t y0 = hi_b ^ x1 ^ k0;
    uint64_t y2 = hi_a ^ x3 ^ k1;
    x0 = y0;
    x1 = lo_b;
    x2 = y2;
    x3 = lo_a;
    k0 += W0;
    k1 += W1;
  }
  Draw d;
  d.w[0] = x0;
  d.w[1] = x1;
  d.w[2] = x2;
  d.w[3] = x3;
  return d;
}

// top 24 bits over 2^24: exact in binary32, in [0, 1 - 2^-24]
__device__ __forceinline__ float uniform24(uint64_t w) {
  return (float)(uint32_t)(w >> 40) * 0x1p-24f;
}

// floor(w * Z / 2^64)
__device__ __forceinline__ uint64_t scale_draw(uint64_t w, uint64_t Z) { return __umul64hi(w, Z); }

// ---------------------------------------------------------------------------------------
// exp_c(y), y <= 0: 2^k * P7(r) with k = rint(y * log2 e), r = y - k ln 2 by a two-constant
// reduction, P7 the degree-7 Taylor polynomial of exp in Horner form; results under e^-87
// are flushed to 0. Every step is one correctly rounded binary32 operation, so the value
// is identical on any IEEE implementation that evaluates the same steps.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float exp_c(float y) {
  if (!(y >= -87.0f)) return 0.0f;
  const float kLog2e = 1.44269502f;
  const float kLn2Hi = 0.693145751953125f;
  const float kLn2Lo = 1.42860677e-06f;
  float k = rintf(__fmul_rn(y, kLog2e));
  float r = __fmaf_rn(-k, kLn2Hi, y);
  r = __fmaf_rn(-k, kLn2Lo, r);
  float p = 1.98412698e-04f;
  p = __fmaf_rn(p, r, 1.38888889e-03f);
  p = __fmaf_rn(p, r, 8.33333377e-03f);
  p = __fmaf_rn(p, r, 4.16666679e-02f);
  p = __fmaf_rn(p, r, 1.66666672e-01f);
  p = __fmaf_rn(p, r, 0.5f);
  p = __fmaf_rn(p, r, 1.0f);
  p = __fmaf_rn(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

// ---------------------------------------------------------------------------------------
// log_c(x), x > 0 finite: x = 2^e m with m in [sqrt(1/2), sqrt(2)); log x = e ln 2 +
// 2 atanh(u), u = (m - 1) / (m + 1), with 2 atanh(u) = 2u (1 + u^2/3 + u^4/5 + u^6/7 +
// u^8/9) in Horner form and e ln 2 split in two constants. Each step is one correctly
// rounded binary32 operation, so every IEEE implementation of these steps agrees.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ float log_c(float x) {
  const float kLn2Hi = 0.693145751953125f;
  const float kLn2Lo = 1.42860677e-06f;
  int e = 0;
  float m = frexpf(x, &e);  // [0.5, 1), exact
  if (m < 0.707106769f) {
    m = __fmul_rn(m, 2.0f);
    e -= 1;
  }
  const float u = __fdiv_rn(__fsub_rn(m, 1.0f), __fadd_rn(m, 1.0f));
  const float u2 = __fmul_rn(u, u);
  float p = 0.111111112f;
  p = __fmaf_rn(p, u2, 0.142857149f);
  p = __fmaf_rn(p, u2, 0.2f);
  p = __fmaf_rn(p, u2, 0.333333343f);
  p = __fmaf_rn(p, u2, 1.0f);
  const float t = __fmul_rn(__fmul_rn(2.0f, u), p);
  const float ef = (float)e;
  return __fmaf_rn(ef, kLn2Hi, __fmaf_rn(ef, kLn2Lo, t));
}

// ---------------------------------------------------------------------------------------
// Temperature classes: 0 greedy, 1 sampled; sets DFLASH2_ST_BADTEMP for invalid values.
// ---------------------------------------------------------------------------------------

__device__ __forceinline__ int temp_mode(float T, float* invT, int* st) {
  if (T == 0.0f) return 0;
  if (T > 0.0f && T <= 3.40282347e38f) {
    float inv = __fdiv_rn(1.0f, T);
    if (inv <= 3.40282347e38f) {
      *invT = inv;
      return 1;
    }
  }
  *st |= DFLASH2_ST_BADTEMP;
  return 0;
}

// probability sanitiser: values outside [0, 1] (and NaN) count as 0 and flag BADPROB
__device__ __forceinline__ float prob_ok(float p, int* st) {
  if (p >= 0.0f && p <= 1.0f) return p;
  *st |= DFLASH2_ST_BADPROB;
  return 0.0f;
}

// floor(p * 2^40) for p in [0, 1]: the scaling is exact; split so that each part converts
// exactly through a 32-bit conversion.
__device__ __forceinline__ uint64_t quant40(float p) {
  float s = p * 256.0f;                    // exact
  float hi = floorf(s);                    // <= 256
  float lo = (s - hi) * 4294967296.0f;     // exact, < 2^32
  return ((uint64_t)(uint32_t)hi << 32) + (uint64_t)(uint32_t)lo;
}

// ---------------------------------------------------------------------------------------
// Wave helpers (wave64)
// ---------------------------------------------------------------------------------------

// The value held by lane l ^ 16 (or l ^ 32) of the wave, through the CDNA4 row swaps: with
// both operands x, v_permlane16_swap leaves each odd row of the first result holding the
// even row before it and each even row of the second result holding the odd row after it
// (rows of 16 lanes); v_permlane32_swap does the same for the two halves of the wave.
// VALU operations, so the exchange takes no LDS round trip. Only for code where all 64
// lanes are active (the helpers below serve divergent code too and keep the permutes).
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (lane & 16) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x, int lane) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (lane & 32) ? r[0] : r[1];
}

// DPP partners within a row of 16 lanes (CDNA DPP controls): the lane 8 and 4 places on
// (rotating within the row), then the lane two and one away within its group of four. For a
// reduction whose combining rule is associative and commutative (a maximum; a maximum with
// ties to the smaller index), combining with these four partners in turn gives every lane
// of the row the row's result, like the xor butterfly. All lanes of the row must be active.
constexpr int kDppRowRor8 = 0x128, kDppRowRor4 = 0x124;
constexpr int kDppQuadXor2 = 0x4E, kDppQuadXor1 = 0xB1;  // quad_perm [2,3,0,1], [1,0,3,2]
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, __uint_as_float(dpp_row<kDppRowRor8>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_row<kDppRowRor4>(__float_as_uint(x))));
  x = fmaxf(x, __uint_as_float(dpp_row<kDppQuadXor2>(__float_as_uint(x))));
  return fmaxf(x, __uint_as_float(dpp_row<kDppQuadXor1>(__float_as_uint(x))));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Wave maxima for code where all 64 lanes are active: halves and rows are combined through
// the row swaps, then each row through DPP. A maximum does not depend on the order in which
// values are combined, so the result equals the butterfly's, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32_all(uint32_t v, int lane) {
  uint32_t o = lane_xor32(v, lane);
  v = o > v ? o : v;
  o = lane_xor16(v, lane);
  v = o > v ? o : v;
  o = dpp_row<kDppRowRor8>(v);
  v = o > v ? o : v;
  o = dpp_row<kDppRowRor4>(v);
  v = o > v ? o : v;
  o = dpp_row<kDppQuadXor2>(v);
  v = o > v ? o : v;
  o = dpp_row<kDppQuadXor1>(v);
  return o > v ? o : v;
}

// Wave sum for code where all 64 lanes are active; integer addition is exact, so the
// combining order does not matter.
__device__ __forceinline__ uint64_t wave_sum_u64_all(uint64_t v, int lane) {
  auto add = [&v](uint32_t lo, uint32_t hi) { v += ((uint64_t)hi << 32) | lo; };
  add(lane_xor32((uint32_t)v, lane), lane_xor32((uint32_t)(v >> 32), lane));
  add(lane_xor16((uint32_t)v, lane), lane_xor16((uint32_t)(v >> 32), lane));
  add(dpp_row<kDppRowRor8>((uint32_t)v), dpp_row<kDppRowRor8>((uint32_t)(v >> 32)));
  add(dpp_row<kDppRowRor4>((uint32_t)v), dpp_row<kDppRowRor4>((uint32_t)(v >> 32)));
  add(dpp_row<kDppQuadXor2>((uint32_t)v), dpp_row<kDppQuadXor2>((uint32_t)(v >> 32)));
  add(dpp_row<kDppQuadXor1>((uint32_t)v), dpp_row<kDppQuadXor1>((uint32_t)(v >> 32)));
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64_all(uint64_t v, int lane) {
  auto take = [&v](uint32_t lo, uint32_t hi) {
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  };
  take(lane_xor32((uint32_t)v, lane), lane_xor32((uint32_t)(v >> 32), lane));
  take(lane_xor16((uint32_t)v, lane), lane_xor16((uint32_t)(v >> 32), lane));
  take(dpp_row<kDppRowRor8>((uint32_t)v), dpp_row<kDppRowRor8>((uint32_t)(v >> 32)));
  take(dpp_row<kDppRowRor4>((uint32_t)v), dpp_row<kDppRowRor4>((uint32_t)(v >> 32)));
  take(dpp_row<kDppQuadXor2>((uint32_t)v), dpp_row<kDppQuadXor2>((uint32_t)(v >> 32)));
  take(dpp_row<kDppQuadXor1>((uint32_t)v), dpp_row<kDppQuadXor1>((uint32_t)(v >> 32)));
  return v;
}

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, 64);
  return v;
}

// Sort 64 values (one per lane) descending; lane 0 ends with the largest.
__device__ __forceinline__ uint32_t wave_sort_desc_u32(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint32_t o = __shfl_xor(v, j, 64);
      bool desc = (lane & k) == 0;   // direction of this bitonic block
      bool low = (lane & j) == 0;    // lower partner
      bool take_max = (desc == low);
      uint32_t mx = o > v ? o : v, mn = o > v ? v : o;
      v = take_max ? mx : mn;
    }
  }
  return v;
}

// ---------------------------------------------------------------------------------------
// Row chunks read by a 256-thread workgroup. With 16-byte loads (VEC), element e of thread
// t sits at chunk offset (e / EPV) * 256 * EPV + t * EPV + e % EPV (each load instruction of
// a wave covers 1 KiB contiguous); otherwise at e * 256 + t. Either way a thread visits its
// elements in increasing index order. Elements at or past V read as 0.
// ---------------------------------------------------------------------------------------

constexpr int kChunkThreads = 256;

template <class KT, int EPT>
struct ChunkLoad {
  using E = typename KT::elem_t;
  static constexpr int kEPV = 16 / (int)sizeof(E);  // elements per 16-byte vector
  static constexpr int kNV = EPT / kEPV;              // vectors per thread
};

// element e of thread t lives at chunk offset (e / EPV) * 256 * EPV + t * EPV + e % EPV
template <int EPV>
__device__ __forceinline__ int elem_offset(int t, int e) {
  return (e / EPV) * (kChunkThreads * EPV) + t * EPV + (e % EPV);
}

template <class KT, int EPT, bool VEC>
__device__ __forceinline__ void load_chunk(const typename KT::elem_t* __restrict__ row, int base,
                                           int V, uint32_t (&bits)[EPT]) {
  using E = typename KT::elem_t;
  const int t = threadIdx.x;
  if constexpr (VEC) {
    constexpr int EPV = ChunkLoad<KT, EPT>::kEPV;
#pragma unroll
    for (int v = 0; v < EPT / EPV; ++v) {
      int off = base + v * (kChunkThreads * EPV) + t * EPV;
      if (off + EPV <= V) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + off);
        const uint32_t ws[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          if constexpr (sizeof(E) == 2)
            bits[v * EPV + e] = (ws[e / 2] >> (16 * (e & 1))) & 0xffffu;
          else
            bits[v * EPV + e] = ws[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          int x = off + e;
          uint32_t u = 0;
          if (x < V) {
            if constexpr (sizeof(E) == 2)
              u = reinterpret_cast<const uint16_t*>(row)[x];
            else
              u = __float_as_uint(reinterpret_cast<const float*>(row)[x]);
          }
          bits[v * EPV + e] = u;
        }
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      int x = base + e * kChunkThreads + t;
      uint32_t u = 0;
      if (x < V) {
        if constexpr (sizeof(E) == 2)
          u = reinterpret_cast<const uint16_t*>(row)[x];
        else
          u = __float_as_uint(reinterpret_cast<const float*>(row)[x]);
      }
      bits[e] = u;
    }
  }
}

// A chunk that lies wholly inside the row with 16-byte aligned rows: every load is issued
// unconditionally before any is used, so a thread's loads are in flight together.
template <class KT, int EPT>
__device__ __forceinline__ void load_chunk_full(const typename KT::elem_t* __restrict__ row,
                                                int base, uint32_t (&bits)[EPT]) {
  using E = typename KT::elem_t;
  constexpr int EPV = 16 / (int)sizeof(E);
  constexpr int NV = EPT / EPV;
  const int t = threadIdx.x;
  u32x4_t w[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v)
    w[v] = *reinterpret_cast<const u32x4_t*>(row + base + v * (kChunkThreads * EPV) + t * EPV);
#pragma unroll
  for (int v = 0; v < NV; ++v)
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      if constexpr (sizeof(E) == 2)
        bits[v * EPV + e] = (w[v][e / 2] >> (16 * (e & 1))) & 0xffffu;
      else
        bits[v * EPV + e] = w[v][e];
    }
}

template <int EPT, bool VEC, class KT>
__device__ __forceinline__ int index_of(int base, int e) {
  if constexpr (VEC)
    return base + elem_offset<ChunkLoad<KT, EPT>::kEPV>(threadIdx.x, e);
  else
    return base + e * kChunkThreads + threadIdx.x;
}


// ---------------------------------------------------------------------------------------
// Host-side launch helper
// ---------------------------------------------------------------------------------------

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DFLASH2_OK : DFLASH2_EHIP;
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kWsAlign = 256;
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace df2
