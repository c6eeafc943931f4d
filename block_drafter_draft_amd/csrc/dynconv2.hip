// dflash2_dynconv2: grouped dynamic two-tap convolution over the draft block ("[Spec
// Decode] DFlash2: local convolution + candidate selector - #52816", PR description, first
// item; "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625", DFlash 2
// commit: two taps over the block, per-element base plus per-group dynamic coefficient):
//
//   out[b,i,c] = (base[0,c] + delta[b,i,0,c/16]) x[b,i,c] + (base[1,c] + delta[b,i,1,c/16]) x[b,i-1,c]
//
// with x[b,-1,c] = 0. One thread owns 8 consecutive channels of one (sequence, position):
// it loads x at that position and the one before (16-byte loads for bf16), the two base
// rows and the two coefficients of its group, all independent of each other and issued
// together, so a call is one memory round trip. The neighbour row is re-read from L2, not HBM. The op moves
// B*P*C*(2+2) bytes plus the base and coefficients and is bound by memory (or by launch
// latency at small B). The output is stored nontemporally: left dirty in L2, its
// write-back at the end of the kernel cost about 2 us per call at batch 64.
#include "common.hpp"

namespace df2 {
namespace {

constexpr int kCPT = 8;  // channels per thread (one 16-byte bf16 vector)

template <bool BF16>
__device__ __forceinline__ void load8(const void* x, int64_t off, float (&v)[kCPT]) {
  if constexpr (BF16) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int e = 0; e < kCPT; ++e) v[e] = bf16_to_f32((w[e / 2] >> (16 * (e & 1))) & 0xffffu);
  } else {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    const float4 u0 = p[0], u1 = p[1];
    v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
    v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
  }
}

// Grid: (channel blocks of 128 threads x 8 channels, sequence-position rows). Every load of
// a thread is issued before any is used: the neighbour row is always read (row 0 reads its
// own row) and replaced by zeros afterwards, so there is no branch between the loads.
constexpr int kConvThreads = 128;

template <bool BF16>
__global__ __launch_bounds__(kConvThreads) void dynconv2_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ base,
                                                                const float* __restrict__ delta,
                                                                void* __restrict__ out, int P,
                                                                int C, int G) {
  const int row = blockIdx.y;  // b * P + i
  const int i = row % P;
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * kCPT;
  if (c0 >= C) return;
  const int grp = c0 / 16;
  const int64_t prow = i > 0 ? row - 1 : row;
  float cur[kCPT], prev[kCPT], b0[kCPT], b1[kCPT];
  load8<BF16>(x, (int64_t)row * C + c0, cur);
  load8<BF16>(x, prow * C + c0, prev);
  const float4* bp0 = reinterpret_cast<const float4*>(base + c0);
  const float4* bp1 = reinterpret_cast<const float4*>(base + C + c0);
  const float4 a0 = bp0[0], a1 = bp0[1], e0 = bp1[0], e1 = bp1[1];
  const float d0 = delta[((int64_t)row * 2 + 0) * G + grp];
  const float d1 = delta[((int64_t)row * 2 + 1) * G + grp];
  b0[0] = a0.x; b0[1] = a0.y; b0[2] = a0.z; b0[3] = a0.w;
  b0[4] = a1.x; b0[5] = a1.y; b0[6] = a1.z; b0[7] = a1.w;
  b1[0] = e0.x; b1[1] = e0.y; b1[2] = e0.z; b1[3] = e0.w;
  b1[4] = e1.x; b1[5] = e1.y; b1[6] = e1.z; b1[7] = e1.w;
  if (i == 0) {
#pragma unroll
    for (int e = 0; e < kCPT; ++e) prev[e] = 0.0f;
  }
  float y[kCPT];
#pragma unroll
  for (int e = 0; e < kCPT; ++e) {
    const float w0 = __fadd_rn(b0[e], d0);
    const float w1 = __fadd_rn(b1[e], d1);
    y[e] = __fadd_rn(__fmul_rn(w0, cur[e]), __fmul_rn(w1, prev[e]));
  }
  if constexpr (BF16) {
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = (uint32_t)f32_to_bf16(y[2 * h]) | ((uint32_t)f32_to_bf16(y[2 * h + 1]) << 16);
    store_nt(reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + (int64_t)row * C + c0), o);
  } else {
    u32x4_t* p = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(out) + (int64_t)row * C + c0);
    store_nt(p, u32x4_t{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                        __float_as_uint(y[3])});
    store_nt(p + 1, u32x4_t{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                            __float_as_uint(y[7])});
  }
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" int dflash2_dynconv2(const void* x, const float* base, const float* delta, void* out,
                                int B, int P, int C, int group, int dtype, hipStream_t stream) {
  if (!x || !base || !delta || !out) return DFLASH2_EINVAL;
  if (B < 1 || P < 1 || C < 16) return DFLASH2_EINVAL;
  if (group != 16 || C % 16 != 0 || P > 16) return DFLASH2_EUNSUPPORTED;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_F32) return DFLASH2_EUNSUPPORTED;
  if (!aligned(x, 16) || !aligned(out, 16)) return DFLASH2_EUNSUPPORTED;
  if (x == out) return DFLASH2_EINVAL;
  if (!aligned(base, 16)) return DFLASH2_EUNSUPPORTED;
  if ((int64_t)B * P > 65535) return DFLASH2_EUNSUPPORTED;
  const dim3 grid((C / kCPT + kConvThreads - 1) / kConvThreads, B * P);
  if (dtype == DFLASH2_BF16)
    dynconv2_kernel<true><<<grid, kConvThreads, 0, stream>>>(x, base, delta, out, P, C, C / 16);
  else
    dynconv2_kernel<false><<<grid, kConvThreads, 0, stream>>>(x, base, delta, out, P, C, C / 16);
  return launch_status();
}
