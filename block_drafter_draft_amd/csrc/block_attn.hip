// dflash2_block_attn: attention of the P block positions over their sliding context
// window and the whole block ("Geramy/LSE docs/DFLASH2.md", drafter geometry paragraph:
// 32 query heads, 8 KV heads, head dim 128; attention noncausal within the draft block,
// including future mask positions; context keys obey the 2048-position sliding window).
//
// bf16 path (MFMA). The P block positions times the G = Hq/Hkv query heads of one KV head
// form one 32-row query tile (8 x 4 = 32 at the drafter geometry), so the context ring of
// each (sequence, KV head) is streamed once for all of them. One wave owns one split of
// that ring: for each tile of 32 keys it computes S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16 (keys as rows, queries as columns), so each lane holds the
// scores of a single query and the online softmax (max, rescale, sum) stays in-lane apart
// from one exchange with the partner half-wave. The probabilities are then used directly
// as the B operand of O^T = V^T P^T: the key order inside the contraction is permuted
// to match the accumulator layout, and V is read through LDS in that same order. Splits
// write unnormalised partial outputs with their (max, sum); a second kernel combines them.
// Context position j of sequence b is in ring row j mod S; slot i sees positions j with
// L_b + i - j < W, plus all P block keys.
//
// f32 path: a plain VALU kernel (one wave per query row), used for small f32 problems.
#include "common.hpp"

namespace df2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;       // query rows per tile
constexpr int kKeys = 32;       // keys per tile
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <int D>
struct AttnSmem {
  static constexpr int kVRS = D + 32;  // padded LDS row stride (elements)
  uint16_t v[kKeys * kVRS];
};

// Split of the keys of one (sequence, KV head): context tiles [t0, t1), plus the block
// keys in split 0.
template <int D>
__global__ __launch_bounds__(64) void attn_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vr, const int32_t* __restrict__ ctx_len, int P, int Hq, int Hkv,
    int S, int W, float scale_log2, int nsplit, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml) {
  constexpr int KS = D / 16;  // k-steps of QK^T
  constexpr int DT = D / 32;  // 32-wide d tiles of PV
  constexpr int VRS = AttnSmem<D>::kVRS;
  __shared__ AttnSmem<D> sm;

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, n = lane & 31, hh = lane >> 5;
  const int G = Hq / Hkv, rows = P * G;
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  const int lo = L - W + 1 > 0 ? L - W + 1 : 0;  // oldest position any slot can see
  const int nt = (L - lo + kKeys - 1) / kKeys;
  const int tps = (nt + nsplit - 1) / nsplit;
  const int t0 = split * tps;
  const int t1 = nt < t0 + tps ? nt : t0 + tps;

  // Q^T as the B operand: lane (n, hh) holds q[n][16 ks + 8 hh .. +7]
  const bool qvalid = n < rows;
  const int slot_n = qvalid ? n / G : 0;
  const int head_n = g * G + (qvalid ? n % G : 0);
  const uint16_t* qrow = q + (((int64_t)b * P + slot_n) * Hq + head_n) * D;
  bf16x8_t qop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4_t w = qvalid ? ld16(qrow + 16 * ks + 8 * hh) : u32x4_t{0, 0, 0, 0};
    qop[ks] = __builtin_bit_cast(bf16x8_t, w);
  }
  const int jmin = L + slot_n - W + 1;  // this query's oldest visible position

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};

  const int ntiles = (t1 > t0 ? t1 - t0 : 0) + (split == 0 ? 1 : 0);
  for (int it = 0; it < ntiles; ++it) {
    const bool blk = it == ntiles - 1 && split == 0;
    const int jbase = lo + (t0 + it) * kKeys;  // context tiles only
    // key row addressing: the row held by lane (as A operand of QK) and V staging rows
    auto key_ptr = [&](const uint16_t* ring, const uint16_t* block, int key, bool& valid) {
      if (blk) {
        valid = key < P;
        return block + (((int64_t)b * P + (valid ? key : 0)) * Hkv + g) * D;
      }
      const int j = jbase + key;
      valid = j < L;
      return ring + (((int64_t)b * S + (valid ? j % S : 0)) * Hkv + g) * D;
    };
    // K as the A operand: lane (key n, hh) holds k[key][16 ks + 8 hh .. +7]
    bool kvalid;
    const uint16_t* krow = key_ptr(kr, kb, n, kvalid);
    u32x4_t ka[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) ka[ks] = kvalid ? ld16(krow + 16 * ks + 8 * hh) : u32x4_t{0, 0, 0, 0};
    // V tile, coalesced: vector vi = v * 64 + lane covers key vi / (D/8), d (vi % (D/8)) * 8
    constexpr int VPL = D / 16;  // vectors per lane
    u32x4_t vv[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * 64 + lane;
      const int key = vi / (D / 8), d0 = (vi % (D / 8)) * 8;
      bool ok;
      const uint16_t* vrow = key_ptr(vr, vb, key, ok);
      vv[v] = ok ? ld16(vrow + d0) : u32x4_t{0, 0, 0, 0};
    }

    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, ka[ks]), qop[ks], s, 0, 0, 0);

    // scores: accumulator i of lane (n, hh) is key 8(i/4) + 4hh + i%4 of this tile
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
      bool vis;
      if (blk) {
        vis = key < P;
      } else {
        const int j = jbase + key;
        vis = j < L && j >= jmin;
      }
      s[i] = vis ? s[i] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    const float base = mnew == -INFINITY ? 0.0f : mnew;
    const float alpha = exp2f(m - base);
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = exp2f(s[i] - base);
      psum += s[i];
    }
    psum += __shfl_xor(psum, 32, 64);
    l = l * alpha + psum;
    m = mnew;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    // stage V (row = key) in LDS
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int vi = v * 64 + lane;
      const int key = vi / (D / 8), d0 = (vi % (D / 8)) * 8;
      *reinterpret_cast<u32x4_t*>(&sm.v[key * VRS + d0]) = vv[v];
    }
    __syncthreads();

    // P^T as the B operand, k-step t: lane's own accumulators 8t .. 8t+7, i.e. keys
    // 16t + 8(e/4) + 4hh + e%4 for element e
    bf16x8_t pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[t][e] = (__bf16)s[8 * t + e];
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + n;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8_t va;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = 16 * t + 8 * (e >> 2) + 4 * hh + (e & 3);
          va[e] = __builtin_bit_cast(__bf16, sm.v[key * VRS + d]);
        }
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[t], o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // partial result: O^T accumulator i of d tile dt is d = 32dt + 8(i/4) + 4hh + i%4
  const int64_t part = ((int64_t)b * Hkv + g) * nsplit + split;
  float* po = ws_o + (part * kRows + n) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = 32 * dt + 8 * a + 4 * hh;
      *reinterpret_cast<float4*>(po + d) =
          make_float4(o[dt][4 * a + 0], o[dt][4 * a + 1], o[dt][4 * a + 2], o[dt][4 * a + 3]);
    }
  if (hh == 0) ws_ml[part * kRows + n] = make_float2(m, l);
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ ws_o,
                                                           const float2* __restrict__ ws_ml, int P,
                                                           int Hq, int Hkv, int nsplit,
                                                           uint16_t* __restrict__ out) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int n = threadIdx.x >> 3, part = threadIdx.x & 7;
  const int G = Hq / Hkv;
  if (n >= P * G) return;
  constexpr int DPT = D / 8;
  const int64_t p0 = ((int64_t)b * Hkv + g) * nsplit;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ws_ml[(p0 + s) * kRows + n].x);
  float acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) acc[e] = 0.0f;
  float den = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float2 ml = ws_ml[(p0 + s) * kRows + n];
    if (ml.x == -INFINITY) continue;
    const float w = exp2f(ml.x - M);
    den += w * ml.y;
    const float* po = ws_o + ((p0 + s) * kRows + n) * D + part * DPT;
#pragma unroll
    for (int e = 0; e < DPT; e += 4) {
      const float4 v = *reinterpret_cast<const float4*>(po + e);
      acc[e] += w * v.x;
      acc[e + 1] += w * v.y;
      acc[e + 2] += w * v.z;
      acc[e + 3] += w * v.w;
    }
  }
  const float inv = 1.0f / den;
  const int slot = n / G, head = g * G + n % G;
  uint16_t* dst = out + (((int64_t)b * P + slot) * Hq + head) * D + part * DPT;
#pragma unroll
  for (int e = 0; e < DPT; e += 8) {
    uint32_t w4[4];
#pragma unroll
    for (int h = 0; h < 4; ++h)
      w4[h] = (uint32_t)f32_to_bf16(acc[e + 2 * h] * inv) |
              ((uint32_t)f32_to_bf16(acc[e + 2 * h + 1] * inv) << 16);
    *reinterpret_cast<uint4*>(dst + e) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// f32: one wave per query row; lanes hold d and d + 64.
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kb, const float* __restrict__ vb,
    const float* __restrict__ kr, const float* __restrict__ vr, const int32_t* __restrict__ ctx_len,
    int P, int Hq, int Hkv, int D, int S, int W, float scale, float* __restrict__ out) {
  const int g = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int G = Hq / Hkv, rows = P * G;
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  for (int n = w; n < rows; n += 4) {
    const int slot = n / G, head = g * G + n % G;
    const float* qr = q + (((int64_t)b * P + slot) * Hq + head) * D;
    const float q0 = lane < D ? qr[lane] : 0.0f, q1 = lane + 64 < D ? qr[lane + 64] : 0.0f;
    float m = -INFINITY, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
    int j0 = L + slot - W + 1;
    j0 = j0 < 0 ? 0 : j0;
    const int nkeys = (L - j0) + P;
    for (int e = 0; e < nkeys; ++e) {
      const float *kp, *vp;
      if (e < L - j0) {
        const int64_t r = (((int64_t)b * S + (j0 + e) % S) * Hkv + g) * D;
        kp = kr + r;
        vp = vr + r;
      } else {
        const int64_t r = (((int64_t)b * P + (e - (L - j0))) * Hkv + g) * D;
        kp = kb + r;
        vp = vb + r;
      }
      float part = (lane < D ? q0 * kp[lane] : 0.0f) + (lane + 64 < D ? q1 * kp[lane + 64] : 0.0f);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      const float sc = part * scale;
      const float mn = fmaxf(m, sc);
      const float a = expf(m - mn), p = expf(sc - mn);
      l = l * a + p;
      o0 = o0 * a + p * (lane < D ? vp[lane] : 0.0f);
      o1 = o1 * a + p * (lane + 64 < D ? vp[lane + 64] : 0.0f);
      m = mn;
    }
    float* dst = out + (((int64_t)b * P + slot) * Hq + head) * D;
    if (lane < D) dst[lane] = o0 / l;
    if (lane + 64 < D) dst[lane + 64] = o1 / l;
  }
}

int plan_splits(int B, int Hkv, int W) {
  const int max_tiles = (W - 1 + kKeys - 1) / kKeys;
  int by_size = (max_tiles + 1) / 2;  // at least ~2 tiles per split
  int by_grid = (2048 + B * Hkv - 1) / (B * Hkv);
  int s = by_size < by_grid ? by_size : by_grid;
  return s < 1 ? 1 : s;
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_block_attn_workspace_bytes(int B, int P, int Hq, int Hkv, int D, int S,
                                                     int W, int dtype) {
  (void)P;
  (void)Hq;
  (void)S;
  if (B < 1 || Hkv < 1 || W < 1 || (D != 64 && D != 128)) return 0;
  if (dtype != DFLASH2_BF16) return 0;
  const int ns = plan_splits(B, Hkv, W);
  const size_t parts = (size_t)B * Hkv * ns;
  return round_up(parts * kRows * D * sizeof(float), kWsAlign) +
         round_up(parts * kRows * sizeof(float2), kWsAlign);
}

extern "C" int dflash2_block_attn(const void* q, const void* k_blk, const void* v_blk,
                                  const void* k_ring, const void* v_ring, const int32_t* ctx_len,
                                  void* out, int B, int P, int Hq, int Hkv, int D, int S, int W,
                                  float scale, int dtype, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!q || !k_blk || !v_blk || !k_ring || !v_ring || !ctx_len || !out) return DFLASH2_EINVAL;
  if (B < 1 || P < 2 || P > 16 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || W < 1 || S < 1)
    return DFLASH2_EINVAL;
  if (S < W - 1) return DFLASH2_EINVAL;
  if (D != 64 && D != 128) return DFLASH2_EUNSUPPORTED;
  if (B > 65535 || Hkv > 65535) return DFLASH2_EUNSUPPORTED;
  const int rows = P * (Hq / Hkv);
  if (dtype == DFLASH2_F32) {
    if (rows > 64) return DFLASH2_EUNSUPPORTED;
    attn_f32_kernel<<<dim3(Hkv, B), 256, 0, stream>>>(
        (const float*)q, (const float*)k_blk, (const float*)v_blk, (const float*)k_ring,
        (const float*)v_ring, ctx_len, P, Hq, Hkv, D, S, W, scale, (float*)out);
    return launch_status();
  }
  if (dtype != DFLASH2_BF16) return DFLASH2_EUNSUPPORTED;
  if (rows > kRows) return DFLASH2_EUNSUPPORTED;
  for (const void* p : {q, k_blk, v_blk, k_ring, v_ring, (const void*)out})
    if (!aligned(p, 16)) return DFLASH2_EUNSUPPORTED;
  const size_t need = dflash2_block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, dtype);
  if (!ws || !aligned(ws, kWsAlign) || ws_bytes < need) return DFLASH2_EWORKSPACE;
  const int ns = plan_splits(B, Hkv, W);
  const size_t parts = (size_t)B * Hkv * ns;
  float* ws_o = (float*)ws;
  float2* ws_ml = (float2*)((char*)ws + round_up(parts * kRows * D * sizeof(float), kWsAlign));
  const float sl2 = scale * kLog2e;
  dim3 grid(ns, Hkv, B);
  if (D == 128) {
    attn_split_kernel<128><<<grid, 64, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k_blk, (const uint16_t*)v_blk,
        (const uint16_t*)k_ring, (const uint16_t*)v_ring, ctx_len, P, Hq, Hkv, S, W, sl2, ns, ws_o,
        ws_ml);
    attn_combine_kernel<128><<<dim3(Hkv, B), 256, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, ns,
                                                               (uint16_t*)out);
  } else {
    attn_split_kernel<64><<<grid, 64, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k_blk, (const uint16_t*)v_blk,
        (const uint16_t*)k_ring, (const uint16_t*)v_ring, ctx_len, P, Hq, Hkv, S, W, sl2, ns, ws_o,
        ws_ml);
    attn_combine_kernel<64><<<dim3(Hkv, B), 256, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, ns,
                                                              (uint16_t*)out);
  }
  return launch_status();
}
