// dflash2_dynconv2: grouped dynamic two-tap convolution over the draft block ("[Spec
// Decode] DFlash2: local convolution + candidate selector - #52816", PR description, first
// item; "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625", DFlash 2
// commit: two taps over the block, per-element base plus per-group dynamic coefficient):
//
//   out[b,i,c] = (base[0,c] + delta[b,i,0,c/16]) x[b,i,c] + (base[1,c] + delta[b,i,1,c/16]) x[b,i-1,c]
//
// with x[b,-1,c] = 0. One thread owns 8 consecutive channels of one or two consecutive
// positions of a sequence: it loads x at those positions and the one before (16-byte
// loads for bf16), the two base rows and the two coefficients of its group per position,
// all independent of each other and issued together, so a call is one memory round trip.
// A neighbour row that another thread also loads mostly comes from cache. The op moves
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

template <bool BF16>
__device__ __forceinline__ void store8(void* out, int64_t off, const float (&y)[kCPT]) {
  if constexpr (BF16) {
    u32x4_t o;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      o[h] = (uint32_t)f32_to_bf16(y[2 * h]) | ((uint32_t)f32_to_bf16(y[2 * h + 1]) << 16);
    store_nt(reinterpret_cast<u32x4_t*>(reinterpret_cast<uint16_t*>(out) + off), o);
  } else {
    u32x4_t* p = reinterpret_cast<u32x4_t*>(reinterpret_cast<float*>(out) + off);
    store_nt(p, u32x4_t{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                        __float_as_uint(y[3])});
    store_nt(p + 1, u32x4_t{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                            __float_as_uint(y[7])});
  }
}

// Grid: (channel blocks of kConvThreads threads x 8 channels, sequences x position groups).
// A thread owns 8 channels of RPT consecutive positions i0 .. i0 + RPT - 1 of one sequence:
// it loads x at those positions and the one before (RPT + 1 rows, so each neighbour row is
// loaded once per thread instead of twice), the two base rows once, and two coefficients
// per position, every load issued before any is used. Rows past the sequence's end re-read
// its last row and are not stored; position 0's neighbour reads its own row and is
// replaced by zeros; so there is no branch between the loads.
#ifndef DF2_CONV_THREADS
#define DF2_CONV_THREADS 64
#endif
constexpr int kConvThreads = DF2_CONV_THREADS;

template <bool BF16, int RPT>
__global__ __launch_bounds__(kConvThreads) void dynconv2_kernel(const void* __restrict__ x,
                                                                const float* __restrict__ base,
                                                                const float* __restrict__ delta,
                                                                void* __restrict__ out, int P,
                                                                int C, int G) {
  const int PG = (P + RPT - 1) / RPT;  // position groups per sequence
  const int b = blockIdx.y / PG, i0 = RPT * (blockIdx.y % PG);
  const int c0 = (blockIdx.x * kConvThreads + threadIdx.x) * kCPT;
  if (c0 >= C) return;
  const int grp = c0 / 16;
  const int64_t r0 = (int64_t)b * P + i0;
  const int64_t last = (int64_t)b * P + P - 1;
  float xr[RPT + 1][kCPT];  // xr[0]: position i0 - 1, xr[1 + k]: position i0 + k
  load8<BF16>(x, (i0 > 0 ? r0 - 1 : r0) * C + c0, xr[0]);
#pragma unroll
  for (int k = 0; k < RPT; ++k) load8<BF16>(x, (r0 + k <= last ? r0 + k : last) * C + c0, xr[1 + k]);
  const float4* bp0 = reinterpret_cast<const float4*>(base + c0);
  const float4* bp1 = reinterpret_cast<const float4*>(base + C + c0);
  const float4 a0 = bp0[0], a1 = bp0[1], e0 = bp1[0], e1 = bp1[1];
  float d[RPT][2];
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    const int64_t r = r0 + k <= last ? r0 + k : last;
    d[k][0] = delta[(r * 2 + 0) * G + grp];
    d[k][1] = delta[(r * 2 + 1) * G + grp];
  }
  const float b0[kCPT] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const float b1[kCPT] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
  if (i0 == 0) {
#pragma unroll
    for (int e = 0; e < kCPT; ++e) xr[0][e] = 0.0f;
  }
#pragma unroll
  for (int k = 0; k < RPT; ++k) {
    float y[kCPT];
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
      const float w0 = __fadd_rn(b0[e], d[k][0]);
      const float w1 = __fadd_rn(b1[e], d[k][1]);
      y[e] = __fadd_rn(__fmul_rn(w0, xr[1 + k][e]), __fmul_rn(w1, xr[k][e]));
    }
    if (k == 0 || i0 + k < P) store8<BF16>(out, (r0 + k) * C + c0, y);
  }
}

// Positions per thread: 2 from 256 sequence-position rows (at batch 64, 8 positions, it
// takes a call from 5.9 to 5.3 us), else 1 (at 128 rows and fewer, two per thread halve
// the threads of an already small grid and were slower).
#ifndef DF2_CONV_RPT
#define DF2_CONV_RPT 0  // 0: by the number of rows
#endif

template <bool BF16>
void launch_conv(const void* x, const float* base, const float* delta, void* out, int B, int P,
                 int C, hipStream_t stream) {
  const int64_t rows = (int64_t)B * P;
  const int rpt = DF2_CONV_RPT ? DF2_CONV_RPT : (rows >= 256 ? 2 : 1);
  const int bx = (C / kCPT + kConvThreads - 1) / kConvThreads;
  if (rpt == 4)
    dynconv2_kernel<BF16, 4><<<dim3(bx, B * ((P + 3) / 4)), kConvThreads, 0, stream>>>(
        x, base, delta, out, P, C, C / 16);
  else if (rpt == 2)
    dynconv2_kernel<BF16, 2><<<dim3(bx, B * ((P + 1) / 2)), kConvThreads, 0, stream>>>(
        x, base, delta, out, P, C, C / 16);
  else
    dynconv2_kernel<BF16, 1><<<dim3(bx, B * P), kConvThreads, 0, stream>>>(x, base, delta, out, P,
                                                                          C, C / 16);
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
  if (dtype == DFLASH2_BF16)
    launch_conv<true>(x, base, delta, out, B, P, C, stream);
  else
    launch_conv<false>(x, base, delta, out, B, P, C, stream);
  return launch_status();
}
