// dflash2_dynconv2: grouped dynamic two-tap convolution over the draft block ("[Spec
// Decode] DFlash2: local convolution + candidate selector - #52816", PR description, first
// item; "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625", DFlash 2
// commit: two taps over the block, per-element base plus per-group dynamic coefficient):
//
//   out[b,i,c] = (base[0,c] + delta[b,i,0,c/16]) x[b,i,c] + (base[1,c] + delta[b,i,1,c/16]) x[b,i-1,c]
//
// with x[b,-1,c] = 0. One thread owns 8 consecutive channels of one sequence and walks the
// P positions, so each activation is read once (16-byte loads for bf16 rows) and the
// previous position stays in registers. The op moves B*P*C*(2+2) bytes plus the base and
// coefficients and is bound by memory (or launch latency at small B).
#include "common.hpp"

namespace df2 {
namespace {

constexpr int kCPT = 8;  // channels per thread (one 16-byte bf16 vector)

template <bool BF16>
__global__ __launch_bounds__(256) void dynconv2_kernel(const void* __restrict__ x,
                                                       const float* __restrict__ base,
                                                       const float* __restrict__ delta,
                                                       void* __restrict__ out, int B, int P, int C,
                                                       int G) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_seq = C / kCPT;
  if (tid >= (int64_t)B * per_seq) return;
  const int b = (int)(tid / per_seq);
  const int c0 = (int)(tid % per_seq) * kCPT;
  const int grp = c0 / 16;
  float b0[kCPT], b1[kCPT], prev[kCPT];
#pragma unroll
  for (int e = 0; e < kCPT; ++e) {
    b0[e] = base[c0 + e];
    b1[e] = base[C + c0 + e];
    prev[e] = 0.0f;
  }
  for (int i = 0; i < P; ++i) {
    const int64_t row = ((int64_t)b * P + i) * C + c0;
    float cur[kCPT];
    if constexpr (BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(x) + row);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < kCPT; ++e) cur[e] = bf16_to_f32((ws[e / 2] >> (16 * (e & 1))) & 0xffffu);
    } else {
      const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + row);
      const float4 u0 = p[0], u1 = p[1];
      cur[0] = u0.x; cur[1] = u0.y; cur[2] = u0.z; cur[3] = u0.w;
      cur[4] = u1.x; cur[5] = u1.y; cur[6] = u1.z; cur[7] = u1.w;
    }
    const float d0 = delta[(((int64_t)b * P + i) * 2 + 0) * G + grp];
    const float d1 = delta[(((int64_t)b * P + i) * 2 + 1) * G + grp];
    float y[kCPT];
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
      const float w0 = __fadd_rn(b0[e], d0);
      const float w1 = __fadd_rn(b1[e], d1);
      y[e] = __fadd_rn(__fmul_rn(w0, cur[e]), __fmul_rn(w1, prev[e]));
      prev[e] = cur[e];
    }
    if constexpr (BF16) {
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[h] = (uint32_t)f32_to_bf16(y[2 * h]) | ((uint32_t)f32_to_bf16(y[2 * h + 1]) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + row) = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + row);
      p[0] = make_float4(y[0], y[1], y[2], y[3]);
      p[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
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
  const int64_t threads = (int64_t)B * (C / kCPT);
  const int blocks = (int)((threads + 255) / 256);
  if (dtype == DFLASH2_BF16)
    dynconv2_kernel<true><<<blocks, 256, 0, stream>>>(x, base, delta, out, B, P, C, C / 16);
  else
    dynconv2_kernel<false><<<blocks, 256, 0, stream>>>(x, base, delta, out, B, P, C, C / 16);
  return launch_status();
}
