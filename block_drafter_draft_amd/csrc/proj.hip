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

// Many rows, staged through LDS: a workgroup of 4 waves owns a 64 x 64 tile (64 features x
// 64 hidden rows) and walks its share of the contraction in stages of 128 columns. Per
// stage the workgroup copies the tile's 64 weight rows and 64 hidden rows (256 bytes of
// each row, 32 KiB in all) into LDS with global_load_lds, each copy instruction covering
// 4 rows x 256 contiguous bytes; two stages are in flight. Loading MFMA operands straight
// into registers makes every load instruction touch 16 rows (the operand layout puts one
// row in each of 16 lanes), and at batch 64 the L1 could not keep up (the address unit
// stalled for most of the call). Each wave computes one 32 x 32 quadrant from LDS: per
// 32-column step two weight and two hidden fragments (16-byte reads; the 16-byte chunks of
// a row are XOR-swizzled by the row index, so the 16 rows of a read hit distinct banks)
// and four v_mfma_f32_16x16x32_bf16. Columns past the workgroup's share are zeroed in the
// fragments, so they add exactly nothing. At batch 64 (512 rows, 640 features, width 5120)
// a call went from 29.5 to 25.0 us; with two 32 KiB stages in flight per workgroup and ten
// stages each, the call is now bound by that latency chain.
constexpr int kLsCols = 128;              // columns per stage
constexpr int kLsChunks = kLsCols / 8;    // 16-byte chunks per row and stage
constexpr int kLsTile = 64 * kLsChunks;   // 16-byte chunks per operand tile (16 KiB)

__global__ __launch_bounds__(256) void proj_lds_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int O, float* __restrict__ out, int64_t oss,
    int64_t ors, float* __restrict__ part_out) {
  __shared__ u32x4_t buf[2][2][kLsTile];  // [stage slot][weight, hidden][row * 16 + chunk]
  const int tz = blockIdx.z, ks = gridDim.z;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform
  const int r = lane & 15, g = lane >> 4;
  const int o0 = blockIdx.x * 64, m0 = blockIdx.y * 64;
  const int nst = (C + kLsCols - 1) / kLsCols;
  const int sb = (int)((int64_t)nst * tz / ks);
  const int se = (int)((int64_t)nst * (tz + 1) / ks);
  const int ce = se * kLsCols < C ? se * kLsCols : C;  // end of the column share

  // copy piece i of thread t: p = t + 256 i; operand p / 1024, slot q = p % 1024 (row q / 16,
  // physical chunk q % 16), fetching the row's logical chunk (q % 16) ^ (row % 16). Rows past
  // O or M are clamped to the last one (their results are never written); chunks past C are
  // clamped to the row's last whole chunk (their columns are zeroed in the fragments).
  const uint16_t* src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int p = t + 256 * i, q = p & 1023, row = q >> 4, ch = (q & 15) ^ (row & 15);
    if (p < 1024) {
      src[i] = wt + (int64_t)min(o0 + row, O - 1) * C + 8 * ch;
    } else {
      const int m = min(m0 + row, M - 1);
      const int b = m / N, rr = m - b * N;
      src[i] = hid + (int64_t)b * hss + (int64_t)(row0 + rr) * hrs + 8 * ch;
    }
  }
  auto issue = [&](int stage, int slot) {
    const int c0 = stage * kLsCols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = t + 256 * i, q = p & 1023, row = q >> 4, ch = (q & 15) ^ (row & 15);
      int off = c0;
      if (c0 + 8 * ch + 8 > C) off = C - 8 - 8 * ch;  // stays inside the row
      // the wave's 64 pieces land at consecutive slots from 64 w + 256 (i % 4) of operand i / 4
      __builtin_amdgcn_global_load_lds(
          (const void*)(src[i] + off),
          (__attribute__((address_space(3))) void*)&buf[slot][i >> 2][64 * w + 256 * (i & 3)], 16,
          0, 0);
    }
  };

  const int wo = w & 1, wm = w >> 1;  // this wave's quadrant
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  const int ns = se - sb;
  if (ns > 0) issue(sb, 0);
  if (ns > 1) issue(sb + 1, 1);
  for (int s = 0; s < ns; ++s) {
    if (s + 1 < ns)
      __asm__ volatile("s_waitcnt vmcnt(8)" ::: "memory");  // stage s's 8 copies have landed
    else
      __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // ... everyone's
    const u32x4_t* A = buf[s & 1][0];
    const u32x4_t* Bh = buf[s & 1][1];
    const int c0 = (sb + s) * kLsCols;
#pragma unroll
    for (int k = 0; k < kLsCols / 32; ++k) {
      const int ch = 4 * k + g;                 // logical chunk of this lane
      const bool live = c0 + 8 * ch < ce;       // inside the workgroup's column share
      u32x4_t a[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = 32 * wo + 16 * i + r, rb = 32 * wm + 16 * i + r;
        a[i] = A[ra * kLsChunks + (ch ^ (ra & 15))];
        bv[i] = Bh[rb * kLsChunks + (ch ^ (rb & 15))];
        if (!live) {
          a[i] = zero;
          bv[i] = zero;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a[i]), __builtin_bit_cast(bf16x8_t, bv[j]), acc[i][j],
              0, 0, 0);
    }
    __syncthreads();  // every wave is done with this slot before it is refilled
    if (s + 2 < ns) issue(sb + s + 2, s & 1);
  }

  // lane (r, g) of tile (i, j) holds features 16 i + 4 g .. + 3 of hidden row 16 j + r of the
  // quadrant
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int o = o0 + 32 * wo + 16 * i + 4 * g;
      const int m = m0 + 32 * wm + 16 * j + r;
      if (m >= M) continue;
      float* dst;
      if (part_out) {
        dst = part_out + ((int64_t)tz * M + m) * O + o;
      } else {
        const int b = m / N, rr = m - b * N;
        dst = out + (int64_t)b * oss + (int64_t)rr * ors + o;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (o + e < O) dst[e] = acc[i][j][e];
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
  bool tile;  // the staged 64 x 64 tile kernel instead
  int ks;     // contraction splits over workgroups
};

// The tile kernel pays off once the hidden rows are re-read enough: measured from 256 rows,
// or from 33 rows with at least 512 features (at 112 rows x 256 features the 16-feature
// kernel is faster; at 8 rows it takes 8.7 us per conv-coefficient call against 7.5).
ProjPlan plan_proj(int M, int O, int C) {
  ProjPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.tile = M >= 256 || (M > 32 && O >= 512);
  const int orows = p.tile ? 64 : kPjRows;
  const int mrows = p.tile ? 64 : 16 * p.mt;
  const int64_t tiles = (int64_t)((O + orows - 1) / orows) * ((M + mrows - 1) / mrows);
  int ks = (int)((kPjTargetWGs + tiles - 1) / tiles);
  // at least one 32-column step per wave of the 16-feature kernel, one 128-column stage per
  // workgroup of the tile kernel
  const int by_steps = p.tile ? (C + kLsCols - 1) / kLsCols
                              : (C + kPjStep - 1) / kPjStep / kPjWaves;
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
  // steps per wave of the 16-feature kernel: at most ceil(ceil(C / 32) / ks / waves)
  const int per_wave =
      (((C + kPjStep - 1) / kPjStep + p.ks - 1) / p.ks + kPjWaves - 1) / kPjWaves;
  const uint16_t* h = (const uint16_t*)hidden;
  const uint16_t* wt = (const uint16_t*)weight;
  const hipStream_t st = stream;
  if (p.tile) {
    proj_lds_kernel<<<grid, 256, 0, st>>>(h, hid_seq_stride, hid_row_stride, row0, N, M, wt, C,
                                           O, out, out_seq_stride, out_row_stride, part);
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
