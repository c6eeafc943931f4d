// dflash2_select: the candidate selector ("[Spec Decode] DFlash2: local convolution +
// candidate selector - #52816", PR description, second item; "Geramy/LSE docs/DFLASH2.md",
// drafter geometry paragraph: each choice conditioned on its predecessor, top-16
// candidates, rank-256 codebooks; top-k paragraph: nonfinite scores are rejected).
//
// Kernel 1 (grid: slots x sequences, 256 threads): gathers the slot's predecessor rows of
// the pred codebook (the anchor's for slot 1, else the 16 candidates of the previous slot)
// and its 16 successor rows of the succ codebook into LDS, then thread (kp, k) evaluates
// the edge score s(kp -> k) = val[k] + sum_r fl(fl(A[p,r] g[r]) B[c,r]), summed left to
// right over r in binary32 with no contraction. Scores go to the workspace lattice.
// Kernel 2 (one wave per sequence): the nonfinite/index checks, then the max-sum path
// (Viterbi, ties to the lower slot) when greedy, or the inverse-CDF walk with exp_c and
// Philox uniforms when sampled.
#include <mutex>

#include "common.hpp"

namespace df2 {
namespace {

constexpr int kMaxN = 15;
constexpr int kMaxR = 512;

// Edge sums unrolled this many steps, so that the LDS reads of several steps are in
// flight before their terms are added (still one at a time, in order).
#ifndef DF2_SEL_UNROLL
#define DF2_SEL_UNROLL 2
#endif
#define DF2_DO_PRAGMA(x) _Pragma(#x)
#define DF2_UNROLL(n) DF2_DO_PRAGMA(unroll n)

// LDS row stride in elements: 8 extra bf16 keep rows 16-byte aligned and shift the banks
__host__ __device__ inline int lat_row_stride(int R) { return ((R + 7) / 8) * 8 + 8; }

// PER: 16-byte gathers per thread (2 * 16 rows * R / 8 / 256 for R <= 64 * PER)
template <bool VEC, int PER>
__global__ __launch_bounds__(256) void select_lattice_kernel(
    const int32_t* __restrict__ cidx, const float* __restrict__ cval,
    const float* __restrict__ gate, const uint16_t* __restrict__ pred_cb,
    const uint16_t* __restrict__ succ_cb, int V, int R, const int32_t* __restrict__ anchor, int N,
    float* __restrict__ lattice) {
  extern __shared__ uint8_t smem[];
  const int i = blockIdx.x + 1;  // slot 1..N
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int kp = t >> 4, k = t & 15;
  const int RS = lat_row_stride(R);
  uint16_t* A = reinterpret_cast<uint16_t*>(smem);  // [16][RS] predecessor rows
  uint16_t* Bm = A + 16 * RS;                       // [16][RS] successor rows
  float* g = reinterpret_cast<float*>(Bm + 16 * RS);  // [RS] gate (zero padded)
  __shared__ int32_t prow[kTopK], srow[kTopK];

  const int npred = i == 1 ? 1 : kTopK;
  // the candidate's value, loaded now so that its latency hides behind the gathers
  const float cv = cval[((int64_t)b * N + (i - 1)) * kTopK + k];
  if (t < kTopK) {
    int32_t p = i == 1 ? anchor[b] : cidx[((int64_t)b * N + (i - 2)) * kTopK + t];
    int32_t c = cidx[((int64_t)b * N + (i - 1)) * kTopK + t];
    prow[t] = (p >= 0 && p < V) ? p : -1;  // invalid indices are never gathered
    srow[t] = (c >= 0 && c < V) ? c : -1;
  }
  __syncthreads();
  const float* gi = gate + ((int64_t)b * N + (i - 1)) * R;
  if constexpr (VEC) {
    // R % 8 == 0: 16-byte row pieces. Every load of the thread is issued before any is
    // used, with no conditions: pieces past the end re-read the last one and invalid rows
    // read row 0, and both are dropped or zeroed afterwards.
    const int vpr = R / 8;
    const int nvec = (npred + kTopK) * vpr;
    u32x4_t buf[PER];
    bool valid[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = min(t + 256 * u, nvec - 1);
      const int row = e / vpr, c8 = (e % vpr) * 8;
      const int32_t r = row < npred ? prow[row] : srow[row - npred];
      const uint16_t* src = row < npred ? pred_cb : succ_cb;
      valid[u] = r >= 0;
      buf[u] = *reinterpret_cast<const u32x4_t*>(src + (int64_t)(r >= 0 ? r : 0) * R + c8);
    }
    const float4 gv = reinterpret_cast<const float4*>(gi)[t < R / 4 ? t : 0];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = t + 256 * u;
      if (e < nvec) {
        const int row = e / vpr, c8 = (e % vpr) * 8;
        uint16_t* dst = row < npred ? A + row * RS : Bm + (row - npred) * RS;
        *reinterpret_cast<u32x4_t*>(dst + c8) = valid[u] ? buf[u] : u32x4_t{0, 0, 0, 0};
      }
    }
    if (t < R / 4) reinterpret_cast<float4*>(g)[t] = gv;
  } else {
    for (int r = t; r < R; r += 256) g[r] = gi[r];
    for (int e = t; e < npred * R; e += 256) {
      const int row = e / R, r = e % R;
      const int32_t p = prow[row];
      A[row * RS + r] = p >= 0 ? pred_cb[(int64_t)p * R + r] : (uint16_t)0;
    }
    for (int e = t; e < kTopK * R; e += 256) {
      const int row = e / R, r = e % R;
      const int32_t c = srow[row];
      Bm[row * RS + r] = c >= 0 ? succ_cb[(int64_t)c * R + r] : (uint16_t)0;
    }
  }
  __syncthreads();
  const uint16_t* bb = Bm + k * RS;
  float acc = 0.0f;
  int r = 0;
  if constexpr (VEC) {
    // fl(A[p,r] g[r]) once per predecessor row, in LDS (it is shared by the 16 successors)
    float* AG = g + RS;  // [16][RS]
    for (int e = t; e < npred * (R / 4); e += 256) {
      const int row = e / (R / 4), c4 = (e % (R / 4)) * 4;
      const uint2 a4 = *reinterpret_cast<const uint2*>(A + row * RS + c4);
      const float4 g4 = *reinterpret_cast<const float4*>(g + c4);
      float4 o;
      o.x = __fmul_rn(bf16_to_f32(a4.x & 0xffffu), g4.x);
      o.y = __fmul_rn(bf16_to_f32(a4.x >> 16), g4.y);
      o.z = __fmul_rn(bf16_to_f32(a4.y & 0xffffu), g4.z);
      o.w = __fmul_rn(bf16_to_f32(a4.y >> 16), g4.w);
      *reinterpret_cast<float4*>(AG + row * RS + c4) = o;
    }
    __syncthreads();
    if (kp >= npred) return;
    const float* ag = AG + kp * RS;
    // eight terms per LDS access, still added one at a time in order
    DF2_UNROLL(DF2_SEL_UNROLL)
    for (; r < R; r += 8) {
      const u32x4_t b8 = *reinterpret_cast<const u32x4_t*>(bb + r);
      const float4 a0 = *reinterpret_cast<const float4*>(ag + r);
      const float4 a1 = *reinterpret_cast<const float4*>(ag + r + 4);
      const float aa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bv = bf16_to_f32((b8[e / 2] >> (16 * (e & 1))) & 0xffffu);
        acc = __fadd_rn(acc, __fmul_rn(aa[e], bv));
      }
    }
  } else {
    if (kp >= npred) return;
    const uint16_t* a = A + kp * RS;
    for (; r < R; ++r) {
      const float ag = __fmul_rn(bf16_to_f32(a[r]), g[r]);
      const float pr = __fmul_rn(ag, bf16_to_f32(bb[r]));
      acc = __fadd_rn(acc, pr);
    }
  }
  lattice[(((int64_t)b * N + (i - 1)) * kTopK + kp) * kTopK + k] = __fadd_rn(cv, acc);
}

// Affine-Q8 codebooks ("Geramy/LSE docs/DFLASH2.md", conversion notes: selector codebooks
// in affine Q8 with groups of 64, BF16 scale and bias, FP32 activations and accumulation):
// element r of a row is fl(fl(scale * q) + bias), q its unsigned 8-bit code and scale, bias
// those of its group of 64, widened from bf16. Same lattice as above: each thread gathers
// 16-byte code pieces with their group's scale and bias (and, for predecessor rows, the
// gate), every load issued before any is used; predecessor rows are dequantised straight
// into fl(A g) and successor rows into binary32, both in LDS; then thread (kp, k) sums
// fl(fl(A g) B) left to right over r. PER: code pieces per thread (R / 16 * 32 / 256).
template <int PER>
__global__ __launch_bounds__(256) void select_lattice_q8_kernel(
    const int32_t* __restrict__ cidx, const float* __restrict__ cval,
    const float* __restrict__ gate, const uint8_t* __restrict__ pcodes,
    const uint16_t* __restrict__ pscale, const uint16_t* __restrict__ pbias,
    const uint8_t* __restrict__ scodes, const uint16_t* __restrict__ sscale,
    const uint16_t* __restrict__ sbias, int V, int R, const int32_t* __restrict__ anchor, int N,
    float* __restrict__ lattice) {
  extern __shared__ uint8_t smem[];
  const int i = blockIdx.x + 1;  // slot 1..N
  const int b = blockIdx.y;
  const int t = threadIdx.x;
  const int kp = t >> 4, k = t & 15;
  const int RS = R + 4;                               // floats per LDS row (16-byte aligned)
  float* AG = reinterpret_cast<float*>(smem);         // [16][RS] fl(A g)
  float* Bf = AG + 16 * RS;                           // [16][RS] successor rows
  __shared__ int32_t prow[kTopK], srow[kTopK];

  const int npred = i == 1 ? 1 : kTopK;
  const float cv = cval[((int64_t)b * N + (i - 1)) * kTopK + k];
  if (t < kTopK) {
    int32_t p = i == 1 ? anchor[b] : cidx[((int64_t)b * N + (i - 2)) * kTopK + t];
    int32_t c = cidx[((int64_t)b * N + (i - 1)) * kTopK + t];
    prow[t] = (p >= 0 && p < V) ? p : -1;  // invalid indices are never gathered
    srow[t] = (c >= 0 && c < V) ? c : -1;
  }
  __syncthreads();
  const float* gi = gate + ((int64_t)b * N + (i - 1)) * R;
  const int ppr = R / 16, G = R / 64;
  const int npieces = (npred + kTopK) * ppr;
  u32x4_t code[PER];
  float sc[PER], bi[PER];
  float4 gq[PER][4];
  bool valid[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = min(t + 256 * u, npieces - 1);
    const int row = e / ppr, c16 = (e % ppr) * 16;
    const bool isp = row < npred;
    const int32_t r = isp ? prow[row] : srow[row - npred];
    valid[u] = r >= 0;
    const int64_t rr = r >= 0 ? r : 0;
    code[u] = *reinterpret_cast<const u32x4_t*>((isp ? pcodes : scodes) + rr * R + c16);
    sc[u] = bf16_to_f32((isp ? pscale : sscale)[rr * G + c16 / 64]);
    bi[u] = bf16_to_f32((isp ? pbias : sbias)[rr * G + c16 / 64]);
    const float4* g4 = reinterpret_cast<const float4*>(gi + c16);
#pragma unroll
    for (int h = 0; h < 4; ++h) gq[u][h] = g4[h];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = t + 256 * u;
    if (e < npieces) {
      const int row = e / ppr, c16 = (e % ppr) * 16;
      const bool isp = row < npred;
      float* dst = isp ? AG + row * RS + c16 : Bf + (row - npred) * RS + c16;
      const float gv[16] = {gq[u][0].x, gq[u][0].y, gq[u][0].z, gq[u][0].w,
                            gq[u][1].x, gq[u][1].y, gq[u][1].z, gq[u][1].w,
                            gq[u][2].x, gq[u][2].y, gq[u][2].z, gq[u][2].w,
                            gq[u][3].x, gq[u][3].y, gq[u][3].z, gq[u][3].w};
      float v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float code_q = (float)((code[u][q / 4] >> (8 * (q & 3))) & 0xffu);
        float a = valid[u] ? __fadd_rn(__fmul_rn(sc[u], code_q), bi[u]) : 0.0f;
        v[q] = isp ? __fmul_rn(a, gv[q]) : a;
      }
#pragma unroll
      for (int q = 0; q < 16; q += 4)
        *reinterpret_cast<float4*>(dst + q) = make_float4(v[q], v[q + 1], v[q + 2], v[q + 3]);
    }
  }
  __syncthreads();
  if (kp >= npred) return;
  const float* ag = AG + kp * RS;
  const float* bb = Bf + k * RS;
  float acc = 0.0f;
  DF2_UNROLL(DF2_SEL_UNROLL)
  for (int r = 0; r < R; r += 4) {
    const float4 a4 = *reinterpret_cast<const float4*>(ag + r);
    const float4 b4 = *reinterpret_cast<const float4*>(bb + r);
    acc = __fadd_rn(acc, __fmul_rn(a4.x, b4.x));
    acc = __fadd_rn(acc, __fmul_rn(a4.y, b4.y));
    acc = __fadd_rn(acc, __fmul_rn(a4.z, b4.z));
    acc = __fadd_rn(acc, __fmul_rn(a4.w, b4.w));
  }
  lattice[(((int64_t)b * N + (i - 1)) * kTopK + kp) * kTopK + k] = __fadd_rn(cv, acc);
}

__global__ __launch_bounds__(64) void select_path_kernel(
    const int32_t* __restrict__ cidx, const float* __restrict__ cval, int V,
    const int32_t* __restrict__ anchor, const float* __restrict__ temperature, uint64_t seed,
    uint64_t step, int N, const float* __restrict__ lattice, int32_t* __restrict__ tokens,
    int32_t* __restrict__ slot, float* __restrict__ q, int32_t* __restrict__ status) {
  const int b = blockIdx.x, lane = threadIdx.x;
  __shared__ float S[kMaxN][kTopK][kTopK];
  __shared__ int32_t bp[kMaxN][kTopK];
  __shared__ float dp[kTopK];
  __shared__ float uni[kMaxN];
  __shared__ int32_t path[kMaxN];
  __shared__ float mtab[kMaxN][kTopK];         // [slot][predecessor row]: the row's maximum
  __shared__ float ztab[kMaxN][kTopK];         // [slot][predecessor row]: its weights' sum
  __shared__ int32_t pick_tab[kMaxN][kTopK];   // [slot][predecessor row]: the pick
  __shared__ int32_t cid[kMaxN * kTopK];

  // Every input load is issued first, so the prologue is one memory round trip: the
  // anchor, the temperature, the candidates and their values (up to 4 per lane) and the
  // lattice (up to kMaxN float4 per lane).
  constexpr int kPerLane = kMaxN * kTopK / 64 + 1;          // candidates per lane
  constexpr int kLat4 = kMaxN * kTopK * kTopK / 4 / 64;      // lattice float4 per lane
  const int ncand = N * kTopK, nlat4 = N * kTopK * kTopK / 4;
  const int32_t anc = anchor[b];
  const float temp = temperature[b];
  int32_t cl[kPerLane];
  float vl[kPerLane];
  // (indices past the end are clamped, so that the loads carry no conditions; those
  // values are never used)
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int e = min(lane + 64 * u, ncand - 1);
    cl[u] = cidx[(int64_t)b * ncand + e];
    vl[u] = cval[(int64_t)b * ncand + e];
  }
  const float4* lat4 = reinterpret_cast<const float4*>(lattice + (int64_t)b * N * kTopK * kTopK);
  float4 lv[kLat4];
#pragma unroll
  for (int u = 0; u < kLat4; ++u) lv[u] = lat4[min(lane + 64 * u, nlat4 - 1)];

  // index validity (anchor and every candidate); the candidates stay in LDS for the end
  int bad = !(anc >= 0 && anc < V);
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int e = lane + 64 * u;
    if (e < ncand) {
      cid[e] = cl[u];
      bad |= !(cl[u] >= 0 && cl[u] < V);
    }
  }
  const bool ok = wave_or(bad) == 0;
  int st = ok ? 0 : DFLASH2_ST_BADTOKEN;

  // scores into LDS; every computed score and value must be finite
  int nonfin = 0;
  if (ok) {
    float* Sf = &S[0][0][0];
#pragma unroll
    for (int u = 0; u < kLat4; ++u) {
      const int e4 = lane + 64 * u;
      if (e4 < nlat4) {
        const float sv[4] = {lv[u].x, lv[u].y, lv[u].z, lv[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int e = 4 * e4 + h;
          const int i = e / (kTopK * kTopK) + 1, kp = (e / kTopK) % kTopK;
          Sf[e] = sv[h];
          // slot 1 has the anchor as its only predecessor (row 0)
          if (!(i == 1 && kp > 0)) nonfin |= !(fabsf(sv[h]) <= 3.40282347e38f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPerLane; ++u)
      if (lane + 64 * u < ncand) nonfin |= !(fabsf(vl[u]) <= 3.40282347e38f);
  }
  const bool finite = wave_or(nonfin) == 0;
  if (ok && !finite) st |= DFLASH2_ST_NONFINITE;
  float invT = 0.0f;
  const int mode = temp_mode(temp, &invT, &st);

  int32_t* tk = tokens + (int64_t)b * N;
  int32_t* sl = slot + (int64_t)b * N;
  float* qq = q + (int64_t)b * N * kTopK;
  if (!ok || !finite) {
    for (int e = lane; e < N * kTopK; e += 64) qq[e] = 0.0f;
    if (lane < N) {
      tk[lane] = -1;
      sl[lane] = -1;
    }
    if (lane == 0) status[b] = st;
    return;
  }
  __syncthreads();

  if (mode == 0) {
    // Viterbi. Lane (k = lane % 16, g = lane / 16) scores candidate k of the slot from the
    // four predecessors 4g .. 4g + 3, in increasing order with a strict comparison, and two
    // exchanges across g keep the larger score, the smaller predecessor on equal scores.
    // That is the first maximum over the 16 predecessors in order, the sequential rule.
    // The scores are finite, so their sums are never NaN.
    const int k = lane & (kTopK - 1), g = lane >> 4;
    if (lane < kTopK) dp[lane] = S[0][0][lane];
    __syncthreads();
    for (int i = 2; i <= N; ++i) {
      float d4[4], s4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d4[j] = dp[4 * g + j];
        s4[j] = S[i - 1][4 * g + j][k];
      }
      float best = __fadd_rn(d4[0], s4[0]);
      int arg = 4 * g;
#pragma unroll
      for (int j = 1; j < 4; ++j) {
        const float v = __fadd_rn(d4[j], s4[j]);
        if (v > best) {
          best = v;
          arg = 4 * g + j;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // lane groups g ^ 1, then g ^ 2 (lanes l ^ 16, l ^ 32)
        const uint32_t bb = __float_as_uint(best), aa = (uint32_t)arg;
        const float ob = __uint_as_float(h == 0 ? lane_xor16(bb, lane) : lane_xor32(bb, lane));
        const int oa = (int)(h == 0 ? lane_xor16(aa, lane) : lane_xor32(aa, lane));
        if (ob > best || (ob == best && oa < arg)) {
          best = ob;
          arg = oa;
        }
      }
      __syncthreads();  // every lane has read dp
      if (lane < kTopK) {
        bp[i - 1][lane] = arg;
        dp[lane] = best;
      }
      __syncthreads();
    }
    // the last slot's first maximum over the 16 candidates, the same way
    float best = dp[k];
    int last = k;
    auto take = [&](float ob, int ol) {
      if (ob > best || (ob == best && ol < last)) {
        best = ob;
        last = ol;
      }
    };
    take(__uint_as_float(dpp_row<kDppRowRor8>(__float_as_uint(best))),
         (int)dpp_row<kDppRowRor8>((uint32_t)last));
    take(__uint_as_float(dpp_row<kDppRowRor4>(__float_as_uint(best))),
         (int)dpp_row<kDppRowRor4>((uint32_t)last));
    take(__uint_as_float(dpp_row<kDppQuadXor2>(__float_as_uint(best))),
         (int)dpp_row<kDppQuadXor2>((uint32_t)last));
    take(__uint_as_float(dpp_row<kDppQuadXor1>(__float_as_uint(best))),
         (int)dpp_row<kDppQuadXor1>((uint32_t)last));
    if (lane == 0) {
      path[N - 1] = last;
      for (int i = N; i >= 2; --i) path[i - 2] = bp[i - 1][path[i - 1]];
    }
    __syncthreads();
    for (int e = lane; e < N * kTopK; e += 64) qq[e] = (e % kTopK) == path[e / kTopK] ? 1.0f : 0.0f;
  } else {
    // Inverse-CDF walk. Slot i draws from the row of its predecessor, which the walk
    // reaches only through slots 1..i-1; but every row's weights and pick can be formed
    // before the walk, independently. Lane l takes the (slot, predecessor row) pairs l,
    // l + 64, ...: the row's maximum, its 16 weights exp_c((s - max) / T), their running
    // sums in k order, and the pick (the first k whose running sum exceeds u_i Z). The
    // walk then only follows the picks, and q = weight / Z is formed for the rows it took
    // (their weights formed again, the same way). Slot 1 has only row 0 (the anchor).
    if (lane < N) uni[lane] = uniform24(philox_draw(seed, step, (uint32_t)b, (uint32_t)(lane + 1)).w[0]);
    __syncthreads();
    for (int pr = lane; pr < N * kTopK; pr += 64) {
      const int i = pr / kTopK + 1, row = pr % kTopK;
      if (i > 1 || row == 0) {
        float sv[kTopK];
#pragma unroll
        for (int k4 = 0; k4 < kTopK; k4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(&S[i - 1][row][k4]);
          sv[k4] = v4.x;
          sv[k4 + 1] = v4.y;
          sv[k4 + 2] = v4.z;
          sv[k4 + 3] = v4.w;
        }
        float m = sv[0];
#pragma unroll
        for (int k = 1; k < kTopK; ++k) m = sv[k] > m ? sv[k] : m;  // exact in any order
        float C[kTopK];
        float Z = 0.0f;
#pragma unroll
        for (int k = 0; k < kTopK; ++k) {
          const float e = exp_c(__fmul_rn(__fsub_rn(sv[k], m), invT));
          Z = __fadd_rn(Z, e);
          C[k] = Z;
        }
        const float tau = __fmul_rn(uni[i - 1], Z);
        int pick = -1;
#pragma unroll
        for (int k = kTopK - 1; k >= 0; --k)
          if (C[k] > tau) pick = k;
        pick_tab[i - 1][row] = pick < 0 ? kTopK - 1 : pick;
        mtab[i - 1][row] = m;
        ztab[i - 1][row] = Z;
      }
    }
    __syncthreads();
    if (lane == 0) {
      int prev = 0;
      for (int i = 1; i <= N; ++i) {
        prev = pick_tab[i - 1][i == 1 ? 0 : prev];
        path[i - 1] = prev;
      }
    }
    __syncthreads();
    for (int e = lane; e < N * kTopK; e += 64) {
      const int i = e / kTopK + 1, row = i == 1 ? 0 : path[i - 2];
      const float w = exp_c(__fmul_rn(__fsub_rn(S[i - 1][row][e % kTopK], mtab[i - 1][row]), invT));
      qq[e] = __fdiv_rn(w, ztab[i - 1][row]);
    }
  }
  if (lane < N) {
    sl[lane] = path[lane];
    tk[lane] = cid[lane * kTopK + path[lane]];
  }
  if (lane == 0) status[b] = st;
}

// Draft tree by best-first expansion over the lattice ("qwen35: DSpark speculative decoding
// (Qwen3.8-27B drafters) - #625", the DDTree commit: candidates scored as draft log-prob
// plus the selector's compatibility with the branch's actual parent, log-softmax
// normalised per position, expanded best-first under a node budget). One wave per
// sequence: the lattice rows are normalised (d = s - max, Z = sum exp_c(d) in k order,
// ls = d - log_c(Z)), then each of `budget` rounds takes the frontier entry with the
// largest score (ties: the earliest added) by one 64-bit wave maximum over packed
// (score key, ~entry) words, records it, and appends its 16 children in k order.
constexpr int kMaxBudget = 64;
constexpr int kMaxFrontier = kTopK + kMaxBudget * kTopK;

__global__ __launch_bounds__(64) void ddtree_kernel(
    const int32_t* __restrict__ cidx, const float* __restrict__ cval, int V,
    const int32_t* __restrict__ anchor, int N, int budget, const float* __restrict__ lattice,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth, int32_t* __restrict__ slotk,
    int32_t* __restrict__ token, float* __restrict__ score, int32_t* __restrict__ status) {
  const int b = blockIdx.x, lane = threadIdx.x;
  __shared__ float LS[kMaxN][kTopK][kTopK];
  __shared__ int32_t cid[kMaxN * kTopK];
  __shared__ float fs[kMaxFrontier];
  __shared__ uint32_t fmeta[kMaxFrontier];  // depth | k << 4 | (parent + 1) << 8 | alive << 16
  __shared__ int32_t opar[kMaxBudget], odep[kMaxBudget], oslt[kMaxBudget], otok[kMaxBudget];
  __shared__ float osc[kMaxBudget];

  // every input load first (as in the path kernel), indices past the end clamped
  constexpr int kPerLane = kMaxN * kTopK / 64 + 1;
  constexpr int kLat4 = kMaxN * kTopK * kTopK / 4 / 64;
  const int ncand = N * kTopK, nlat4 = N * kTopK * kTopK / 4;
  const int32_t anc = anchor[b];
  int32_t cl[kPerLane];
  float vl[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int e = min(lane + 64 * u, ncand - 1);
    cl[u] = cidx[(int64_t)b * ncand + e];
    vl[u] = cval[(int64_t)b * ncand + e];
  }
  const float4* lat4 = reinterpret_cast<const float4*>(lattice + (int64_t)b * N * kTopK * kTopK);
  float4 lv[kLat4];
#pragma unroll
  for (int u = 0; u < kLat4; ++u) lv[u] = lat4[min(lane + 64 * u, nlat4 - 1)];

  int bad = !(anc >= 0 && anc < V);
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) {
    const int e = lane + 64 * u;
    if (e < ncand) {
      cid[e] = cl[u];
      bad |= !(cl[u] >= 0 && cl[u] < V);
    }
  }
  const bool ok = wave_or(bad) == 0;
  int st = ok ? 0 : DFLASH2_ST_BADTOKEN;
  int nonfin = 0;
  if (ok) {
    float* Sf = &LS[0][0][0];
#pragma unroll
    for (int u = 0; u < kLat4; ++u) {
      const int e4 = lane + 64 * u;
      if (e4 < nlat4) {
        const float sv[4] = {lv[u].x, lv[u].y, lv[u].z, lv[u].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int e = 4 * e4 + h;
          const int i = e / (kTopK * kTopK) + 1, kp = (e / kTopK) % kTopK;
          Sf[e] = sv[h];
          if (!(i == 1 && kp > 0)) nonfin |= !(fabsf(sv[h]) <= 3.40282347e38f);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kPerLane; ++u)
      if (lane + 64 * u < ncand) nonfin |= !(fabsf(vl[u]) <= 3.40282347e38f);
  }
  const bool finite = wave_or(nonfin) == 0;
  if (ok && !finite) st |= DFLASH2_ST_NONFINITE;
  const int64_t o = (int64_t)b * budget;
  if (!ok || !finite) {
    for (int t = lane; t < budget; t += 64) {
      parent[o + t] = depth[o + t] = slotk[o + t] = token[o + t] = -1;
      score[o + t] = 0.0f;
    }
    if (lane == 0) status[b] = st;
    return;
  }
  __syncthreads();

  // normalise every parent row: slot 1 has only the anchor's row
  const int nrows = 1 + (N - 1) * kTopK;
  for (int q = lane; q < nrows; q += 64) {
    const int i = q == 0 ? 1 : 2 + (q - 1) / kTopK, kp = q == 0 ? 0 : (q - 1) % kTopK;
    float* row = &LS[i - 1][kp][0];
    float v[kTopK];
#pragma unroll
    for (int k = 0; k < kTopK; ++k) v[k] = row[k];
    float m = v[0];
#pragma unroll
    for (int k = 1; k < kTopK; ++k) m = v[k] > m ? v[k] : m;
    float Z = 0.0f;
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      v[k] = __fsub_rn(v[k], m);
      Z = __fadd_rn(Z, exp_c(v[k]));
    }
    const float lz = log_c(Z);
#pragma unroll
    for (int k = 0; k < kTopK; ++k) row[k] = __fsub_rn(v[k], lz);
  }
  __syncthreads();

  if (lane < kTopK) {
    fs[lane] = __fadd_rn(0.0f, LS[0][0][lane]);
    fmeta[lane] = 1u | ((uint32_t)lane << 4) | (1u << 16);
  }
  int F = kTopK;
  __syncthreads();
  for (int t = 0; t < budget; ++t) {
    uint64_t key = 0;
    for (int f = lane; f < F; f += 64) {
      if (fmeta[f] >> 16) {
        const uint64_t w = ((uint64_t)KeyF32::canon(__float_as_uint(fs[f])) << 32) |
                           (uint64_t)(~(uint32_t)f);
        key = w > key ? w : key;
      }
    }
    key = wave_max_u64(key);
    if (key == 0) {  // the whole tree is taken
      if (lane == 0) {
        opar[t] = odep[t] = oslt[t] = otok[t] = -1;
        osc[t] = 0.0f;
      }
      __syncthreads();
      continue;
    }
    const int f = (int)(~(uint32_t)key);
    const float sf = fs[f];
    const uint32_t meta = fmeta[f];
    const int dd = meta & 15u, kk = (meta >> 4) & 15u, pp = (int)((meta >> 8) & 255u) - 1;
    __syncthreads();  // every lane has read the entry
    if (lane == 0) {
      fmeta[f] = meta & 0xffffu;  // taken
      opar[t] = pp;
      odep[t] = dd;
      oslt[t] = kk;
      otok[t] = cid[(dd - 1) * kTopK + kk];
      osc[t] = sf;
    }
    if (dd < N) {
      if (lane < kTopK) {
        fs[F + lane] = __fadd_rn(sf, LS[dd][kk][lane]);
        fmeta[F + lane] =
            (uint32_t)(dd + 1) | ((uint32_t)lane << 4) | ((uint32_t)(t + 1) << 8) | (1u << 16);
      }
      F += kTopK;
    }
    __syncthreads();
  }
  for (int t = lane; t < budget; t += 64) {
    parent[o + t] = opar[t];
    depth[o + t] = odep[t];
    slotk[o + t] = oslt[t];
    token[o + t] = otok[t];
    score[o + t] = osc[t];
  }
  if (lane == 0) status[b] = st;
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_select_workspace_bytes(int B, int N) {
  if (B < 1 || N < 1 || N > kMaxN) return 0;
  return round_up((size_t)B * N * kTopK * kTopK * sizeof(float), kWsAlign);
}

namespace df2 {
namespace {

// Both selector entry points: the host checks are done, `lattice` holds at least
// dflash2_select_workspace_bytes(B, N) bytes of device memory.
int select_launch(const int32_t* cand_idx, const float* cand_val, const float* gate,
                  const uint16_t* pred_cb, const uint16_t* succ_cb, int V, int R,
                  const int32_t* anchor, const float* temperature, uint64_t seed, uint64_t step,
                  int B, int N, int32_t* tokens, int32_t* slot, float* q, int32_t* status,
                  float* lattice, hipStream_t stream) {
  const int RS = lat_row_stride(R);
  // predecessor and successor rows (bf16), the gate, and the products fl(A g) (f32)
  const size_t lds = (size_t)2 * kTopK * RS * sizeof(uint16_t) + (size_t)RS * sizeof(float) +
                     (size_t)kTopK * RS * sizeof(float);
  const bool vec = R % 8 == 0 && aligned(pred_cb, 16) && aligned(succ_cb, 16) && aligned(gate, 16);
  if (vec && R <= 256)
    select_lattice_kernel<true, 4><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  else if (vec)
    select_lattice_kernel<true, 8><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  else
    select_lattice_kernel<false, 1><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  select_path_kernel<<<B, 64, 0, stream>>>(cand_idx, cand_val, V, anchor, temperature, seed, step,
                                           N, lattice, tokens, slot, q, status);
  return launch_status();
}

int select_check(const int32_t* cand_idx, const float* cand_val, const float* gate,
                 const uint16_t* pred_cb, const uint16_t* succ_cb, int V, int R,
                 const int32_t* anchor, const float* temperature, int B, int N,
                 const int32_t* tokens, const int32_t* slot, const float* q,
                 const int32_t* status) {
  if (!cand_idx || !cand_val || !gate || !pred_cb || !succ_cb || !anchor || !temperature ||
      !tokens || !slot || !q || !status)
    return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || R < 1 || V < kTopK) return DFLASH2_EINVAL;
  if (N > kMaxN || R > kMaxR || B > 65535) return DFLASH2_EUNSUPPORTED;
  return DFLASH2_OK;
}

// The allocation-free selector's lattice: a file-scope device array, one copy per GPU the
// library runs on, held until the process ends. Host code never passes `scratch` itself
// (on the host that name is not a device address); it passes the address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr size_t kSelectScratchBytes = (size_t)4 << 20;
__device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Address of this device's `scratch`, or nullptr on a HIP error.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace df2

extern "C" int dflash2_select(const int32_t* cand_idx, const float* cand_val, const float* gate,
                              const uint16_t* pred_cb, const uint16_t* succ_cb, int V, int R,
                              const int32_t* anchor, const float* temperature, uint64_t seed,
                              uint64_t step, int B, int N, int32_t* tokens, int32_t* slot,
                              float* q, int32_t* status, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  const int rc = select_check(cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor,
                              temperature, B, N, tokens, slot, q, status);
  if (rc != DFLASH2_OK) return rc;
  if (!ws) return DFLASH2_EINVAL;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_select_workspace_bytes(B, N))
    return DFLASH2_EWORKSPACE;
  return select_launch(cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, temperature,
                       seed, step, B, N, tokens, slot, q, status, (float*)ws, stream);
}

extern "C" size_t dflash2_select_noalloc_max_bytes(void) { return kSelectScratchBytes; }

extern "C" int dflash2_select_noalloc(const int32_t* cand_idx, const float* cand_val,
                                      const float* gate, const uint16_t* pred_cb,
                                      const uint16_t* succ_cb, int V, int R,
                                      const int32_t* anchor, const float* temperature,
                                      uint64_t seed, uint64_t step, int B, int N,
                                      int32_t* tokens, int32_t* slot, float* q, int32_t* status,
                                      hipStream_t stream) {
  const int rc = select_check(cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor,
                              temperature, B, N, tokens, slot, q, status);
  if (rc != DFLASH2_OK) return rc;
  if (dflash2_select_workspace_bytes(B, N) > kSelectScratchBytes) return DFLASH2_EWORKSPACE;
  void* lattice = scratch_for_current_device();
  if (!lattice) return DFLASH2_EHIP;
  return select_launch(cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, temperature,
                       seed, step, B, N, tokens, slot, q, status, (float*)lattice, stream);
}

extern "C" int dflash2_select_q8(const int32_t* cand_idx, const float* cand_val,
                                 const float* gate, const uint8_t* pred_codes,
                                 const uint16_t* pred_scale, const uint16_t* pred_bias,
                                 const uint8_t* succ_codes, const uint16_t* succ_scale,
                                 const uint16_t* succ_bias, int V, int R, const int32_t* anchor,
                                 const float* temperature, uint64_t seed, uint64_t step, int B,
                                 int N, int32_t* tokens, int32_t* slot, float* q, int32_t* status,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cand_idx || !cand_val || !gate || !pred_codes || !pred_scale || !pred_bias ||
      !succ_codes || !succ_scale || !succ_bias || !anchor || !temperature || !tokens || !slot ||
      !q || !status || !ws)
    return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || R < 1 || V < kTopK) return DFLASH2_EINVAL;
  if (N > kMaxN || R > kMaxR || R % 64 != 0 || B > 65535) return DFLASH2_EUNSUPPORTED;
  if (!aligned(pred_codes, 16) || !aligned(succ_codes, 16) || !aligned(gate, 16) ||
      !aligned(pred_scale, 2) || !aligned(pred_bias, 2) || !aligned(succ_scale, 2) ||
      !aligned(succ_bias, 2))
    return DFLASH2_EUNSUPPORTED;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_select_workspace_bytes(B, N))
    return DFLASH2_EWORKSPACE;
  float* lattice = (float*)ws;
  const size_t lds = (size_t)2 * kTopK * (R + 4) * sizeof(float);
  if (R <= 256)
    select_lattice_q8_kernel<2><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_codes, pred_scale, pred_bias, succ_codes, succ_scale,
        succ_bias, V, R, anchor, N, lattice);
  else
    select_lattice_q8_kernel<4><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_codes, pred_scale, pred_bias, succ_codes, succ_scale,
        succ_bias, V, R, anchor, N, lattice);
  select_path_kernel<<<B, 64, 0, stream>>>(cand_idx, cand_val, V, anchor, temperature, seed, step,
                                           N, lattice, tokens, slot, q, status);
  return launch_status();
}

extern "C" size_t dflash2_ddtree_workspace_bytes(int B, int N) {
  return dflash2_select_workspace_bytes(B, N);
}

extern "C" int dflash2_ddtree(const int32_t* cand_idx, const float* cand_val, const float* gate,
                              const uint16_t* pred_cb, const uint16_t* succ_cb, int V, int R,
                              const int32_t* anchor, int B, int N, int budget, int32_t* parent,
                              int32_t* depth, int32_t* slot, int32_t* token, float* score,
                              int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!cand_idx || !cand_val || !gate || !pred_cb || !succ_cb || !anchor || !parent || !depth ||
      !slot || !token || !score || !status || !ws)
    return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || R < 1 || V < kTopK || budget < 1) return DFLASH2_EINVAL;
  if (N > kMaxN || R > kMaxR || B > 65535 || budget > kMaxBudget) return DFLASH2_EUNSUPPORTED;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_ddtree_workspace_bytes(B, N))
    return DFLASH2_EWORKSPACE;
  float* lattice = (float*)ws;
  const int RS = lat_row_stride(R);
  const size_t lds = (size_t)2 * kTopK * RS * sizeof(uint16_t) + (size_t)RS * sizeof(float) +
                     (size_t)kTopK * RS * sizeof(float);
  const bool vec = R % 8 == 0 && aligned(pred_cb, 16) && aligned(succ_cb, 16) && aligned(gate, 16);
  if (vec && R <= 256)
    select_lattice_kernel<true, 4><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  else if (vec)
    select_lattice_kernel<true, 8><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  else
    select_lattice_kernel<false, 1><<<dim3(N, B), 256, lds, stream>>>(
        cand_idx, cand_val, gate, pred_cb, succ_cb, V, R, anchor, N, lattice);
  ddtree_kernel<<<B, 64, 0, stream>>>(cand_idx, cand_val, V, anchor, N, budget, lattice, parent,
                                      depth, slot, token, score, status);
  return launch_status();
}
