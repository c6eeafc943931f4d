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
// the result does not depend on timing.
//
// A compute unit keeps only so many lines in flight, so a small call is paced by how many
// units pull the weight, not by HBM: at batch 1 a conv site's 640 coefficients (6.5 MB of
// weight at width 5120) make only 40 workgroups of 16 features. When the output tiles
// number fewer than the compute units, the contraction is also split over KS workgroups
// (grid z) that write binary32 partials to the workspace, and a second kernel adds the KS
// partials of each output in split order. Either way the sum's order is fixed.
#include "common.hpp"

namespace df2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPjWaves = 8;   // contraction split
constexpr int kPjRows = 16;   // output features per workgroup
constexpr int kPjStep = 32;   // columns per MFMA
constexpr int kPjPad = 17;    // LDS row pitch of a partial tile (floats)

constexpr int kPjMaxSplit = 32;   // most contraction splits over workgroups
constexpr int kPjTargetWGs = 256;  // one workgroup per compute unit

template <int MT, int NS>
__global__ __launch_bounds__(64 * kPjWaves) void proj_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int O, float* __restrict__ out, int64_t oss,
    int64_t ors, float* __restrict__ part_out) {
  __shared__ float part[kPjWaves * 16 * MT * kPjPad];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int o0 = blockIdx.x * kPjRows;
  const int m0 = blockIdx.y * (16 * MT);
  // this workgroup's share of the 32-column steps (split blockIdx.z of gridDim.z), then
  // wave w's contiguous part of it
  const int steps = (C + kPjStep - 1) / kPjStep;
  const int gb = (int)((int64_t)steps * blockIdx.z / gridDim.z);
  const int ge = (int)((int64_t)steps * (blockIdx.z + 1) / gridDim.z);
  const int sb = gb + (int)((int64_t)(ge - gb) * w / kPjWaves);
  const int se = gb + (int)((int64_t)(ge - gb) * (w + 1) / kPjWaves);

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
      // lanes past the range issue no load (their operands are zero)
      ok[s] = (s0 + s < se) && (c < C);
      a[s] = zero;
      if (ok[s]) a[s] = *reinterpret_cast<const u32x4_t*>(wrow + c);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bv[mt][s] = zero;
        if (ok[s]) bv[mt][s] = *reinterpret_cast<const u32x4_t*>(hrow[mt] + c);
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                          __builtin_bit_cast(bf16x8_t, bv[mt][s]),
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
      if (part_out) {
        part_out[((int64_t)blockIdx.z * M + m) * O + o] = s;
      } else {
        const int b = m / N, rr = m - b * N;
        out[(int64_t)b * oss + (int64_t)rr * ors + o] = s;
      }
    }
  }
}

// More than 32 hidden rows: a workgroup of 4 waves owns a 64 x 64 tile (64 features x 64
// rows) and each wave computes all 16 MFMA tiles of it over its quarter of the
// contraction, so every operand fragment it loads feeds four products. Per step a lane
// loads four weight pieces and four hidden pieces (columns 32 s + 8 g .. + 8 of rows
// 16 t + r). This reads the hidden rows once per 64 features instead of once per 16:
// about 105 MB instead of 262 MB of L2 traffic at batch 64 (512 rows, 640 features).
constexpr int kTlWaves = 4;
constexpr int kTlPad = 65;  // LDS row pitch (floats) of a 64 x 64 partial tile

template <int NS>
__global__ __launch_bounds__(64 * kTlWaves) void proj_tile_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int O, float* __restrict__ out, int64_t oss,
    int64_t ors, float* __restrict__ part_out) {
  __shared__ float part[kTlWaves * 64 * kTlPad];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int o0 = blockIdx.x * 64;
  const int m0 = blockIdx.y * 64;
  const int steps = (C + kPjStep - 1) / kPjStep;
  const int gb = (int)((int64_t)steps * blockIdx.z / gridDim.z);
  const int ge = (int)((int64_t)steps * (blockIdx.z + 1) / gridDim.z);
  const int sb = gb + (int)((int64_t)(ge - gb) * w / kTlWaves);
  const int se = gb + (int)((int64_t)(ge - gb) * (w + 1) / kTlWaves);

  // rows past O or M are clamped to the last one (their results are never written)
  const uint16_t* wrow[4];
  const uint16_t* hrow[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    wrow[u] = wt + (int64_t)min(o0 + 16 * u + r, O - 1) * C;
    const int m = min(m0 + 16 * u + r, M - 1);
    const int b = m / N, rr = m - b * N;
    hrow[u] = hid + (int64_t)b * hss + (int64_t)(row0 + rr) * hrs;
  }
  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  for (int s0 = sb; s0 < se; s0 += NS) {
    u32x4_t a[NS][4], bv[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = (s0 + s) * kPjStep + 8 * g;
      const bool ok = (s0 + s < se) && (c < C);  // C % 8 == 0: a piece is wholly inside
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[s][u] = zero;
        bv[s][u] = zero;
        if (ok) {
          a[s][u] = *reinterpret_cast<const u32x4_t*>(wrow[u] + c);
          bv[s][u] = *reinterpret_cast<const u32x4_t*>(hrow[u] + c);
        }
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a[s][i]), __builtin_bit_cast(bf16x8_t, bv[s][j]),
              acc[i][j], 0, 0, 0);
  }

  // lane (r, g) of tile (i, j) holds feature 16 i + 4 g + e of row 16 j + r; LDS [o][m]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[(w * 64 + 16 * i + 4 * g + e) * kTlPad + 16 * j + r] = acc[i][j][e];
  __syncthreads();

  for (int e = threadIdx.x; e < 64 * 64; e += 64 * kTlWaves) {
    const int ml = e >> 6, ol = e & 63;
    float sum = part[ol * kTlPad + ml];
#pragma unroll
    for (int v = 1; v < kTlWaves; ++v) sum = __fadd_rn(sum, part[(v * 64 + ol) * kTlPad + ml]);
    const int m = m0 + ml, o = o0 + ol;
    if (m < M && o < O) {
      if (part_out) {
        part_out[((int64_t)blockIdx.z * M + m) * O + o] = sum;
      } else {
        const int b = m / N, rr = m - b * N;
        out[(int64_t)b * oss + (int64_t)rr * ors + o] = sum;
      }
    }
  }
}

// out[m, o] = sum over splits k in order of part[k, m, o], KS <= KMAX. Every load is issued
// first, unconditionally (splits past KS re-read the last one and are not added).
template <int KMAX>
__global__ __launch_bounds__(256) void proj_reduce_kernel(const float* __restrict__ part, int KS,
                                                          int M, int O, int N,
                                                          float* __restrict__ out, int64_t oss,
                                                          int64_t ors) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t MO = (int64_t)M * O;
  if (e >= MO) return;
  float v[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) v[k] = part[(k < KS ? k : KS - 1) * MO + e];
  float s = v[0];
#pragma unroll
  for (int k = 1; k < KMAX; ++k)
    if (k < KS) s = __fadd_rn(s, v[k]);
  const int m = (int)(e / O), o = (int)(e - (int64_t)m * O);
  const int b = m / N, rr = m - b * N;
  out[(int64_t)b * oss + (int64_t)rr * ors + o] = s;
}

struct ProjPlan {
  int mt;     // row tiles of 16 per workgroup (16-feature kernel)
  bool tile;  // the 64 x 64 tile kernel instead
  int ks;     // contraction splits over workgroups
};

// The tile kernel pays off once the hidden rows are re-read enough: measured from 256 rows,
// or from 33 rows with at least 512 features (at 112 rows x 256 features the 16-feature
// kernel is faster).
ProjPlan plan_proj(int M, int O, int C) {
  ProjPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.tile = M >= 256 || (M > 32 && O >= 512);
  const int orows = p.tile ? 64 : kPjRows;
  const int waves = p.tile ? kTlWaves : kPjWaves;
  const int mrows = p.tile ? 64 : 16 * p.mt;
  const int64_t tiles = (int64_t)((O + orows - 1) / orows) * ((M + mrows - 1) / mrows);
  const int steps = (C + kPjStep - 1) / kPjStep;
  int ks = (int)((kPjTargetWGs + tiles - 1) / tiles);
  const int by_steps = steps / waves;  // at least one step per wave
  ks = ks < by_steps ? ks : by_steps;
  ks = ks < kPjMaxSplit ? ks : kPjMaxSplit;
  p.ks = ks < 1 ? 1 : ks;
  return p;
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_proj_workspace_bytes(int B, int N, int O, int C) {
  if (B < 1 || N < 1 || O < 1 || C < 1 || (int64_t)B * N > (1 << 20) || O > (1 << 26)) return 0;
  const int M = B * N;
  const ProjPlan p = plan_proj(M, O, C);
  if (p.ks == 1) return 0;
  return round_up((size_t)p.ks * M * O * sizeof(float), kWsAlign);
}

extern "C" int dflash2_proj(const void* hidden, int64_t hid_seq_stride, int64_t hid_row_stride,
                            int row0, const void* weight, int C, int O, int B, int N, float* out,
                            int64_t out_seq_stride, int64_t out_row_stride, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
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
  const size_t need = dflash2_proj_workspace_bytes(B, N, O, C);
  if (need && (!ws || !aligned(ws, kWsAlign) || ws_bytes < need)) return DFLASH2_EWORKSPACE;
  const int M = B * N;
  const ProjPlan p = plan_proj(M, O, C);
  float* part = p.ks > 1 ? (float*)ws : nullptr;
  const int orows = p.tile ? 64 : kPjRows;
  const int mrows = p.tile ? 64 : 16 * p.mt;
  const int gx = (O + orows - 1) / orows;
  const int gy = (M + mrows - 1) / mrows;
  const dim3 grid(gx, gy, p.ks);
  // steps per wave: at most ceil(ceil(C / 32) / ks / waves)
  const int waves = p.tile ? kTlWaves : kPjWaves;
  const int per_wave = (((C + kPjStep - 1) / kPjStep + p.ks - 1) / p.ks + waves - 1) / waves;
  const uint16_t* h = (const uint16_t*)hidden;
  const uint16_t* wt = (const uint16_t*)weight;
  const hipStream_t st = stream;
  if (p.tile) {
    if (per_wave <= 2)
      proj_tile_kernel<2><<<grid, 64 * kTlWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride,
                                                           row0, N, M, wt, C, O, out,
                                                           out_seq_stride, out_row_stride, part);
    else
      proj_tile_kernel<4><<<grid, 64 * kTlWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride,
                                                           row0, N, M, wt, C, O, out,
                                                           out_seq_stride, out_row_stride, part);
  } else if (p.mt == 1) {
    if (per_wave <= 4)
      proj_kernel<1, 4><<<grid, 64 * kPjWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0,
                                                         N, M, wt, C, O, out, out_seq_stride,
                                                         out_row_stride, part);
    else
      proj_kernel<1, 20><<<grid, 64 * kPjWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0,
                                                          N, M, wt, C, O, out, out_seq_stride,
                                                          out_row_stride, part);
  } else if (p.mt == 2) {
    if (per_wave <= 4)
      proj_kernel<2, 4><<<grid, 64 * kPjWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0,
                                                         N, M, wt, C, O, out, out_seq_stride,
                                                         out_row_stride, part);
    else
      proj_kernel<2, 12><<<grid, 64 * kPjWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0,
                                                          N, M, wt, C, O, out, out_seq_stride,
                                                          out_row_stride, part);
  } else {
    proj_kernel<4, 8><<<grid, 64 * kPjWaves, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0, N,
                                                       M, wt, C, O, out, out_seq_stride,
                                                       out_row_stride, part);
  }
  if (p.ks > 1) {
    const int64_t MO = (int64_t)M * O;
    const unsigned nb = (unsigned)((MO + 255) / 256);
    if (p.ks <= 4)
      proj_reduce_kernel<4><<<nb, 256, 0, st>>>(part, p.ks, M, O, N, out, out_seq_stride,
                                                out_row_stride);
    else if (p.ks <= 8)
      proj_reduce_kernel<8><<<nb, 256, 0, st>>>(part, p.ks, M, O, N, out, out_seq_stride,
                                                out_row_stride);
    else if (p.ks <= 16)
      proj_reduce_kernel<16><<<nb, 256, 0, st>>>(part, p.ks, M, O, N, out, out_seq_stride,
                                                 out_row_stride);
    else
      proj_reduce_kernel<kPjMaxSplit><<<nb, 256, 0, st>>>(part, p.ks, M, O, N, out,
                                                          out_seq_stride, out_row_stride);
  }
  return launch_status();
}
