// dflash2_proj: the drafter's linear projections on either side of the path. The dynamic
// conv's per-group coefficients come from one projection of the sublayer's input, and the
// selector's edge multiplies A[p] elementwise by a projection of the hidden state
// ("[Spec Decode] DFlash2: local convolution + candidate selector - #52816", PR
// description, both items; "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) -
// #625", DFlash 2 commit: kernel projections and hproj):
//
//   out[m, o] = sum_c hidden[m, c] * weight[o, c]   (binary32 accumulation of exact
//                                                    bf16 x bf16 products)
//
// for the rows m of B sequences (N rows each from row0, addressed by element strides) and
// a weight [O, C] in a linear layer's usual layout.
//
// The weight is read once and each of its bytes feeds exactly one wave, so operands go
// straight from memory into MFMA registers; LDS only carries the reduction. A workgroup
// owns 16 output features (the M side of v_mfma_f32_16x16x32_bf16) and up to 16 * MT
// hidden rows (the N side, MT tiles of 16), and its 8 waves split the contraction: wave w
// takes a contiguous range of 32-column steps. For each step, lane (r = lane % 16,
// g = lane / 16) loads columns 32 s + 8 g .. + 8 of weight row o0 + r and of hidden row
// m0 + r: the four lanes of a row read 64 contiguous bytes, and the pair of steps s, s + 1
// completes a 128-byte line. All NS steps' loads of a pass are issued before the first
// product. The waves' 16 x 16 partial tiles are then added in wave order through LDS, so
// the result does not depend on timing. At batch 1 the call is a latency-bound read of
// the weight (6.5 MB for a conv site's 640 coefficients at width 5120).
#include "common.hpp"

namespace df2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPjWaves = 8;   // contraction split
constexpr int kPjRows = 16;   // output features per workgroup
constexpr int kPjStep = 32;   // columns per MFMA
constexpr int kPjPad = 17;    // LDS row pitch of a partial tile (floats)

template <int MT, int NS>
__global__ __launch_bounds__(64 * kPjWaves) void proj_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int O, float* __restrict__ out, int64_t oss,
    int64_t ors) {
  __shared__ float part[kPjWaves * 16 * MT * kPjPad];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int o0 = blockIdx.x * kPjRows;
  const int m0 = blockIdx.y * (16 * MT);
  const int steps = (C + kPjStep - 1) / kPjStep;
  const int sb = (int)((int64_t)steps * w / kPjWaves);
  const int se = (int)((int64_t)steps * (w + 1) / kPjWaves);

  // rows past O or M are clamped to the last one (their results are never written)
  const uint16_t* wrow = wt + (int64_t)min(o0 + r, O - 1) * C;
  const uint16_t* hrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(m0 + 16 * mt + r, M - 1);
    const int b = m / N, rr = m - b * N;
    hrow[mt] = hid + (int64_t)b * hss + (int64_t)(row0 + rr) * hrs;
  }

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int s0 = sb; s0 < se; s0 += NS) {
    u32x4_t a[NS];
    u32x4_t bv[MT][NS];
    bool ok[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = (s0 + s) * kPjStep + 8 * g;
      // C % 8 == 0, so a piece that starts inside the row ends inside it
      ok[s] = (s0 + s < se) && (c < C);
      const int cl = ok[s] ? c : 0;
      a[s] = *reinterpret_cast<const u32x4_t*>(wrow + cl);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) bv[mt][s] = *reinterpret_cast<const u32x4_t*>(hrow[mt] + cl);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4_t av = ok[s] ? a[s] : zero;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t hv = ok[s] ? bv[mt][s] : zero;
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                          __builtin_bit_cast(bf16x8_t, hv),
                                                          acc[mt], 0, 0, 0);
      }
    }
  }

  // lane (r, g) holds output feature 4 g + i of hidden row 16 mt + r
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      part[(w * 16 * MT + 16 * mt + r) * kPjPad + 4 * g + i] = acc[mt][i];
  __syncthreads();

  for (int e = threadIdx.x; e < 16 * 16 * MT; e += 64 * kPjWaves) {
    const int ml = e >> 4, ol = e & 15;
    float s = part[ml * kPjPad + ol];
#pragma unroll
    for (int v = 1; v < kPjWaves; ++v) s = __fadd_rn(s, part[(v * 16 * MT + ml) * kPjPad + ol]);
    const int m = m0 + ml, o = o0 + ol;
    if (m < M && o < O) {
      const int b = m / N, rr = m - b * N;
      out[(int64_t)b * oss + (int64_t)rr * ors + o] = s;
    }
  }
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" int dflash2_proj(const void* hidden, int64_t hid_seq_stride, int64_t hid_row_stride,
                            int row0, const void* weight, int C, int O, int B, int N, float* out,
                            int64_t out_seq_stride, int64_t out_row_stride, hipStream_t stream) {
  if (!hidden || !weight || !out) return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || row0 < 0 || C < 1 || O < 1 || hid_seq_stride < 0 || hid_row_stride < 0)
    return DFLASH2_EINVAL;
  if (out_seq_stride < 0 || out_row_stride < 0) return DFLASH2_EINVAL;
  // distinct output rows must not overlap: sequence-major or row-major placement
  {
    const int64_t ors = N > 1 ? out_row_stride : (int64_t)O;
    const int64_t oss = B > 1 ? out_seq_stride : (int64_t)O;
    const bool seq_major = ors >= O && (B == 1 || oss >= (int64_t)(N - 1) * ors + O);
    const bool row_major = oss >= O && (N == 1 || ors >= (int64_t)(B - 1) * oss + O);
    if (!seq_major && !row_major) return DFLASH2_EINVAL;
  }
  if (C % 8 != 0) return DFLASH2_EUNSUPPORTED;
  if ((int64_t)B * N > (1 << 20) || O > (1 << 26)) return DFLASH2_EUNSUPPORTED;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || hid_seq_stride % 8 != 0 ||
      hid_row_stride % 8 != 0)
    return DFLASH2_EUNSUPPORTED;
  const int M = B * N;
  const int gx = (O + kPjRows - 1) / kPjRows;
  const hipStream_t st = stream;
  if (M <= 16) {
    proj_kernel<1, 20><<<dim3(gx, 1), 64 * kPjWaves, 0, st>>>(
        (const uint16_t*)hidden, hid_seq_stride, hid_row_stride, row0, N, M,
        (const uint16_t*)weight, C, O, out, out_seq_stride, out_row_stride);
  } else if (M <= 32) {
    proj_kernel<2, 12><<<dim3(gx, 1), 64 * kPjWaves, 0, st>>>(
        (const uint16_t*)hidden, hid_seq_stride, hid_row_stride, row0, N, M,
        (const uint16_t*)weight, C, O, out, out_seq_stride, out_row_stride);
  } else {
    proj_kernel<4, 8><<<dim3(gx, (M + 63) / 64), 64 * kPjWaves, 0, st>>>(
        (const uint16_t*)hidden, hid_seq_stride, hid_row_stride, row0, N, M,
        (const uint16_t*)weight, C, O, out, out_seq_stride, out_row_stride);
  }
  return launch_status();
}
