// dflash2_block_attn: attention of the P block positions over their sliding context
// window and the whole block ("Geramy/LSE docs/DFLASH2.md", drafter geometry paragraph:
// 32 query heads, 8 KV heads, head dim 128; attention noncausal within the draft block,
// including future mask positions; context keys obey the 2048-position sliding window).
//
// bf16 path (MFMA). The P block positions times the G = Hq/Hkv query heads of one KV head
// form one 32-row query tile (8 x 4 = 32 at the drafter geometry), so the context ring of
// each (sequence, KV head) is streamed from HBM once for all of them. A workgroup of four
// waves owns one split of that ring and walks it in stages of 64 keys: the 256 threads
// load a stage's K and V rows with 16-byte coalesced loads into padded LDS tiles, and the
// next stage's loads are issued before the current stage is computed, so one stage (32 KiB)
// is always in flight. Wave w takes 32-key tile (w & 1) of the stage and half (w >> 1) of
// the head dimension: it computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows,
// queries as columns, so each lane owns one query's scores and the online softmax stays
// in-lane apart from one exchange with the other half-wave), then uses its probabilities
// directly as the B operand of O^T = V^T P^T for its 64 output columns; the key order in
// that contraction is permuted to match the accumulator layout and V is read from LDS in
// the same order (wave w covers columns [(w >> 1) D/2, (w >> 1 + 1) D/2)). At the end the
// two tiles' states are merged through LDS. With one split
// the workgroup writes the bf16 output; with several it writes an unnormalised partial and
// its (max, sum), and a second kernel combines the splits.
// Context position j of sequence b is in ring row j mod S; slot i sees positions j with
// L_b + i - j < W, plus all P block keys.
//
// f32 path: a plain VALU kernel (one wave per query row), used for small f32 problems.
#include "common.hpp"

// Split partials stored nontemporally (1) or through L2 (0); the combine kernel reads them
// right after.
#ifndef DF2_ATTN_NT_PARTIAL
#define DF2_ATTN_NT_PARTIAL 0
#endif

namespace df2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;    // query rows per tile
constexpr int kMaxSplits = 32;  // most splits of one (sequence, KV head)
constexpr int kStage = 64;   // keys per stage (two 32-key tiles)

// Split planning: aim for kAttnTargetWGs workgroups, with at least kAttnMinStages stages
// per split; stages in flight per workgroup: kAttnPrefetch (1 or 2).
#ifndef DF2_ATTN_TARGET_WGS
#define DF2_ATTN_TARGET_WGS 512
#endif
#ifndef DF2_ATTN_MIN_STAGES
#define DF2_ATTN_MIN_STAGES 2
#endif
#ifndef DF2_ATTN_PREFETCH
#define DF2_ATTN_PREFETCH 1
#endif
constexpr int kAttnTargetWGs = DF2_ATTN_TARGET_WGS;
constexpr int kAttnMinStages = DF2_ATTN_MIN_STAGES;
constexpr int kAttnPrefetch = DF2_ATTN_PREFETCH;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

template <int D>
struct AttnShape {
  static constexpr int KRS = D + 8;               // LDS row stride of K (elements)
  static constexpr int VRS = D + 16;              // LDS row stride of V
  static constexpr int VPR = D / 8;               // 16-byte vectors per key row
  static constexpr int LOADS = kStage * VPR / 256;  // vectors per thread per tensor per stage
  static constexpr int KS = D / 16;               // k-steps of QK^T
  static constexpr int DTH = D / 64;              // 32-wide d tiles per half of D
};

template <int D>
struct AttnSmem {
  union {
    struct {
      uint16_t k[kStage * AttnShape<D>::KRS];
      uint16_t v[kStage * AttnShape<D>::VRS];
    } kv;
    struct {
      float o[2][AttnShape<D>::DTH][16][64];  // partner wave's O^T accumulators
      float m[2][32], l[2][32];
    } x;
  };
};

template <int D>
__global__ __launch_bounds__(256) void attn_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vr, const int32_t* __restrict__ ctx_len, int P, int Hq, int Hkv,
    int S, int W, float scale_log2, int nsplit, int stages_per_split, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, uint16_t* __restrict__ out) {
  using SH = AttnShape<D>;
  __shared__ AttnSmem<D> sm;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int tt = w & 1, dh = w >> 1;
  const int G = Hq / Hkv, rows = P * G;
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  const int lo = L - W + 1 > 0 ? L - W + 1 : 0;  // oldest position any slot can see
  const int c0 = split * stages_per_split * kStage + lo;   // first context key of the split
  int c1 = c0 + stages_per_split * kStage;
  c1 = c1 < L ? c1 : L;
  const int nctx_st = c1 > c0 ? (c1 - c0 + kStage - 1) / kStage : 0;
  // split 0 also takes the block keys, as its first stage (its loads go out with the rest)
  const int blk_st = split == 0 ? 1 : 0;
  const int nst = nctx_st + blk_st;

  // Q^T as the B operand: lane (n, hh) holds q[n][16 ks + 8 hh .. +7]
  const bool qvalid = n < rows;
  const int slot_n = qvalid ? n / G : 0;
  const int head_n = g * G + (qvalid ? n % G : 0);
  const uint16_t* qrow = q + (((int64_t)b * P + slot_n) * Hq + head_n) * D;
  bf16x8_t qop[SH::KS];
#pragma unroll
  for (int ks = 0; ks < SH::KS; ++ks) {
    u32x4_t v = qvalid ? ld16(qrow + 16 * ks + 8 * hh) : u32x4_t{0, 0, 0, 0};
    qop[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
  const int jmin = L + slot_n - W + 1;  // this query's oldest visible position

  // Stage loads: vector vi = t + 256 u covers stage key vi / VPR, columns (vi % VPR) * 8.
  // The thread's stage keys are kk0 + 256/VPR * u; their ring rows are found from one
  // modulo per stage.
  constexpr int KSTEP = 256 / SH::VPR;  // stage-key stride between a thread's vectors
  const int kk0 = t / SH::VPR, d0 = (t % SH::VPR) * 8;
  const int64_t head_off = (int64_t)g * D + d0;
  auto load_stage = [&](int st, u32x4_t (&kreg)[SH::LOADS], u32x4_t (&vreg)[SH::LOADS]) {
    if (st < blk_st) {
#pragma unroll
      for (int u = 0; u < SH::LOADS; ++u) {
        const int kk = kk0 + KSTEP * u;
        const bool ok = kk < P;
        const int64_t row = ((int64_t)b * P + (ok ? kk : 0)) * Hkv * D + head_off;
        kreg[u] = ok ? ld16(kb + row) : u32x4_t{0, 0, 0, 0};
        vreg[u] = ok ? ld16(vb + row) : u32x4_t{0, 0, 0, 0};
      }
      return;
    }
    const int j0 = c0 + (st - blk_st) * kStage + kk0;
    int jm = j0 % S;
    const int kstep_mod = KSTEP % S;  // < S, so one wrap check keeps jm in [0, S)
#pragma unroll
    for (int u = 0; u < SH::LOADS; ++u) {
      const bool ok = j0 + KSTEP * u < c1;
      const int64_t row = ((int64_t)b * S + (ok ? jm : 0)) * Hkv * D + head_off;
      kreg[u] = ok ? ld16(kr + row) : u32x4_t{0, 0, 0, 0};
      vreg[u] = ok ? ld16(vr + row) : u32x4_t{0, 0, 0, 0};
      jm += kstep_mod;
      jm = jm >= S ? jm - S : jm;
    }
  };

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[SH::DTH];
#pragma unroll
  for (int i = 0; i < SH::DTH; ++i) o[i] = f32x16_t{};

  auto compute_stage = [&](int st) {
    const bool blk = st < blk_st;
    const int jb = c0 + (st - blk_st) * kStage;
    // S^T for tile tt: accumulator i of lane (n, hh) is key 32 tt + 8(i/4) + 4hh + i%4
    f32x16_t s = f32x16_t{};
    const uint16_t* krow = &sm.kv.k[(32 * tt + n) * SH::KRS + 8 * hh];
#pragma unroll
    for (int ks = 0; ks < SH::KS; ++ks)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + 16 * ks)), qop[ks], s,
          0, 0, 0);
    // visible keys of this tile: a block stage keeps keys [0, P); a context stage keeps
    // positions j in [max(jb, jmin), c1), i.e. tile keys [klo, khi)
    const int klo = blk ? 0 : (jmin > jb ? jmin - jb : 0);
    const int khi = blk ? P : c1 - jb;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = 32 * tt + 8 * (i >> 2) + 4 * hh + (i & 3);
      const bool vis = kk >= klo && kk < khi;
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
    for (int i = 0; i < SH::DTH; ++i) o[i] *= alpha;
    // P^T as the B operand, k-step u: own accumulators 8u .. 8u+7 = keys 16u + 8(e/4) + 4hh + e%4
    bf16x8_t pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[u][e] = (__bf16)s[8 * u + e];
#pragma unroll
    for (int i = 0; i < SH::DTH; ++i) {
      const int d = (D / 2) * dh + 32 * i + n;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8_t va;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kk = 32 * tt + 16 * u + 8 * (e >> 2) + 4 * hh + (e & 3);
          va[e] = __builtin_bit_cast(__bf16, sm.kv.v[kk * SH::VRS + d]);
        }
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[u], o[i], 0, 0, 0);
      }
    }
  };
  auto store_stage = [&](const u32x4_t (&kreg)[SH::LOADS], const u32x4_t (&vreg)[SH::LOADS]) {
#pragma unroll
    for (int u = 0; u < SH::LOADS; ++u) {
      const int kk = kk0 + KSTEP * u;
      *reinterpret_cast<u32x4_t*>(&sm.kv.k[kk * SH::KRS + d0]) = kreg[u];
      *reinterpret_cast<u32x4_t*>(&sm.kv.v[kk * SH::VRS + d0]) = vreg[u];
    }
  };

  if constexpr (kAttnPrefetch == 2) {
    // two stages in flight: registers A hold even stages, B odd ones
    u32x4_t ka[SH::LOADS], va_[SH::LOADS], kb2[SH::LOADS], vb2[SH::LOADS];
    if (nst > 0) load_stage(0, ka, va_);
    if (nst > 1) load_stage(1, kb2, vb2);
    for (int st = 0; st < nst; st += 2) {
      store_stage(ka, va_);
      __syncthreads();
      if (st + 2 < nst) load_stage(st + 2, ka, va_);
      compute_stage(st);
      __syncthreads();
      if (st + 1 >= nst) break;
      store_stage(kb2, vb2);
      __syncthreads();
      if (st + 3 < nst) load_stage(st + 3, kb2, vb2);
      compute_stage(st + 1);
      __syncthreads();
    }
  } else {
    // one stage in flight
    u32x4_t ka[SH::LOADS], va_[SH::LOADS];
    if (nst > 0) load_stage(0, ka, va_);
    for (int st = 0; st < nst; ++st) {
      store_stage(ka, va_);
      __syncthreads();
      if (st + 1 < nst) load_stage(st + 1, ka, va_);
      compute_stage(st);
      __syncthreads();
    }
  }

  // merge tile 1 into tile 0 (same d half): waves 1 and 3 hand their state to 0 and 2
  if (tt == 1) {
#pragma unroll
    for (int i = 0; i < SH::DTH; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.x.o[dh][i][r][lane] = o[i][r];
    if (hh == 0) {
      sm.x.m[dh][n] = m;
      sm.x.l[dh][n] = l;
    }
  }
  __syncthreads();
  if (tt == 1) return;
  {
    const float m1 = sm.x.m[dh][n], l1 = sm.x.l[dh][n];
    const float M = fmaxf(m, m1);
    const float a0 = M == -INFINITY ? 0.0f : exp2f(m - M);
    const float a1 = M == -INFINITY ? 0.0f : exp2f(m1 - M);
    l = l * a0 + l1 * a1;
    m = M;
#pragma unroll
    for (int i = 0; i < SH::DTH; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[i][r] = o[i][r] * a0 + sm.x.o[dh][i][r][lane] * a1;
  }
  // accumulator r of d tile i is column d = (D/2) dh + 32 i + 8(r/4) + 4hh + r%4
  if (nsplit == 1) {
    if (!qvalid) return;
    const float inv = 1.0f / l;
    uint16_t* dst = out + (((int64_t)b * P + slot_n) * Hq + head_n) * D;
#pragma unroll
    for (int i = 0; i < SH::DTH; ++i)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = (D / 2) * dh + 32 * i + 8 * a + 4 * hh;
        const uint32_t lo2 = (uint32_t)f32_to_bf16(o[i][4 * a] * inv) |
                             ((uint32_t)f32_to_bf16(o[i][4 * a + 1] * inv) << 16);
        const uint32_t hi2 = (uint32_t)f32_to_bf16(o[i][4 * a + 2] * inv) |
                             ((uint32_t)f32_to_bf16(o[i][4 * a + 3] * inv) << 16);
        store_nt(reinterpret_cast<u32x2_t*>(dst + d), u32x2_t{lo2, hi2});
      }
    return;
  }
  const int64_t part = ((int64_t)b * Hkv + g) * nsplit + split;
  float* po = ws_o + (part * kRows + n) * D;
#pragma unroll
  for (int i = 0; i < SH::DTH; ++i)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int d = (D / 2) * dh + 32 * i + 8 * a + 4 * hh;
      *reinterpret_cast<float4*>(po + d) =
          make_float4(o[i][4 * a], o[i][4 * a + 1], o[i][4 * a + 2], o[i][4 * a + 3]);
    }
  if (dh == 0 && hh == 0) ws_ml[part * kRows + n] = make_float2(m, l);
}

// ---------------------------------------------------------------------------------------
// D = 128 streaming kernel. The keys of one (sequence, KV head) are listed as the visible
// context window (oldest first) followed by the P block keys, and cut into 32-key tiles.
// A workgroup owns a contiguous range of tiles (one split); each of its four waves takes
// every fourth tile and works on its own: it streams the tile's K and V rows (8 KiB each)
// straight from HBM into its own pair of LDS buffers with global_load_lds (16 bytes per
// lane, no registers held while the load is in flight), the next tile's copy overlapping
// the current tile's arithmetic, so no barrier is needed until the end. Per tile a wave
// computes S^T = K Q^T (8 MFMA 32x32x16), the online softmax in-lane, and O^T += V^T P^T
// for all 128 columns (8 MFMA), with the V^T operand read by ds_read_b64_tr_b16, which
// hands each lane four keys of one column. Rows land in LDS with their 16-byte chunks
// XOR-swizzled by the row index, so that both the K reads (16 rows, one chunk) and the
// transposed V reads (4 rows, 4 chunks per half-wave) hit distinct banks. At the end the
// waves' states are merged through LDS, each wave producing its share of the columns.
// NW (waves per workgroup) is 4 when the grid is about one workgroup per compute unit
// (128 KiB of tile buffers each), and 2 for large batches, so that two workgroups share a
// unit and the whole grid is resident in one round.
constexpr int kTileKeys = 32;
constexpr int kStreamD = 128;
constexpr int kTileElems = kTileKeys * kStreamD;     // one tensor's tile (8 KiB of bf16)
constexpr int kMergeStride = 40;                      // floats per d row of a merge state
constexpr float kLazyLog2 = 8.0f;  // largest growth of a query's maximum before a rescale

#define DF2_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int NW>
struct StreamSmem {
  union {
    uint16_t kv[NW][2][2][kTileElems];           // [wave][buffer][K, V][tile]
    float o[NW][kStreamD][kMergeStride];         // [wave][d][query row]
  };
  float m[NW][kRows], l[NW][kRows];
};

// chunk swizzle of tile row r: 16 consecutive rows get 16 distinct values, and 4
// consecutive rows (aligned to 4) land in 4 different groups of four chunks
__device__ __forceinline__ int tile_swz(int r) { return ((r & 3) << 2) ^ ((r >> 2) & 3); }

template <int NW>
__global__ __launch_bounds__(64 * NW) void attn_stream_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kb,
    const uint16_t* __restrict__ vb, const uint16_t* __restrict__ kr,
    const uint16_t* __restrict__ vr, const int32_t* __restrict__ ctx_len, int P, int Hq, int Hkv,
    int S, int W, float scale_log2, int nsplit, int tiles_per_split, float* __restrict__ ws_o,
    float2* __restrict__ ws_ml, uint16_t* __restrict__ out) {
  constexpr int D = kStreamD;
  __shared__ StreamSmem<NW> sm;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, so tile math is scalar
  const int G = Hq / Hkv, rows = P * G;
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  const int lo = L - W + 1 > 0 ? L - W + 1 : 0;   // oldest visible context position
  const int nctx = L - lo;                         // context keys in the list
  const int nkeys = nctx + P;
  const int ntiles = (nkeys + kTileKeys - 1) / kTileKeys;
  const int tbeg = split * tiles_per_split;
  int tend = tbeg + tiles_per_split;
  tend = tend < ntiles ? tend : ntiles;
  // this wave's tiles: tbeg + w, tbeg + w + NW, ...
  const int nmine = tend - tbeg - w > 0 ? (tend - tbeg - w + NW - 1) / NW : 0;

  // Q^T as the B operand: lane (n, hh) holds q[n][16 ks + 8 hh .. +7]
  const bool qvalid = n < rows;
  const int slot_n = qvalid ? n / G : 0;
  const int head_n = g * G + (qvalid ? n % G : 0);
  const uint16_t* qrow = q + (((int64_t)b * P + slot_n) * Hq + head_n) * D;
  bf16x8_t qop[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    u32x4_t v = qvalid ? ld16(qrow + 16 * ks + 8 * hh) : u32x4_t{0, 0, 0, 0};
    qop[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
  // list index of this query's oldest visible context key (block keys are always visible),
  // and the largest such index over all slots: a tile of context keys from there on is
  // visible to every query
  const int kmin = L + slot_n - W + 1 - lo;
  const int kmin_all = L + P - W - lo;

  // Copy of tile `tile` into buffer `buf`: instruction i moves rows 4i .. 4i+3; lane l
  // fetches chunk (l & 15) ^ swz(row) of row 4i + l / 16 into LDS slot l.
  const int64_t ring_b = (int64_t)b * S * Hkv * D + (int64_t)g * D;
  const int64_t blk_b = (int64_t)b * P * Hkv * D + (int64_t)g * D;
  const int lrow = lane >> 4;
  // Context tiles that do not wrap around the ring (nearly all of them) take a cheap path:
  // ring rows jm .. jm + 31 are consecutive, so lane l's row 4i + l/16 sits at a 32-bit byte
  // offset (jm + l/16) * rowb + 4 i rowb from the sequence's ring base, plus its chunk, which
  // depends on i only through i & 3.
  const uint32_t rowb = (uint32_t)(Hkv * D * 2);
  const char* kr_b = reinterpret_cast<const char*>(kr + ring_b);
  const char* vr_b = reinterpret_cast<const char*>(vr + ring_b);
  uint32_t coffb[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) coffb[k] = 16u * (uint32_t)(((lane & 15) ^ (lrow << 2)) ^ k);
  auto issue = [&](int tile, int buf) {
    const int kk0 = tile * kTileKeys;
    const int jm = kk0 < nctx ? (lo + kk0) % S : 0;  // ring row of list entry kk0 (if context)
    uint16_t* dk = &sm.kv[w][buf][0][0];
    uint16_t* dv = &sm.kv[w][buf][1][0];
    if (kk0 + kTileKeys <= nctx && jm + kTileKeys <= S) {
      const uint32_t rowbase = (uint32_t)(jm + lrow) * rowb;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t off = rowbase + (uint32_t)(4 * i) * rowb + coffb[i & 3];
        __builtin_amdgcn_global_load_lds((const void*)(kr_b + off), DF2_LDS(dk + i * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vr_b + off), DF2_LDS(dv + i * 512), 16, 0, 0);
      }
      return;
    }
    const uint16_t* ksrc[8];
    const uint16_t* vsrc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + lrow;
      const int kk = kk0 + r;
      int jr = jm + r;
      if (S >= kTileKeys) {
        jr = jr >= S ? jr - S : jr;
      } else {
        jr = jr % S;
      }
      const int p = kk - nctx >= 0 && kk - nctx < P ? kk - nctx : 0;  // padding: block row 0
      const bool ctx = kk < nctx;
      const int64_t roff = ctx ? ring_b + (int64_t)jr * Hkv * D : blk_b + (int64_t)p * Hkv * D;
      const int64_t coff = 8 * ((lane & 15) ^ tile_swz(r));
      ksrc[i] = (ctx ? kr : kb) + (roff + coff);
      vsrc[i] = (ctx ? vr : vb) + (roff + coff);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_global_load_lds((const void*)ksrc[i], DF2_LDS(dk + i * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)vsrc[i], DF2_LDS(dv + i * 512), 16, 0, 0);
    }
  };

  float m = -INFINITY, l = 0.0f;
  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};

  auto compute = [&](int tile, int buf, bool first) {
    const uint16_t* tk = &sm.kv[w][buf][0][0];
    const uint16_t* tv = &sm.kv[w][buf][1][0];
    // S^T: accumulator i of lane (n, hh) is tile key 8(i/4) + 4hh + i%4; two independent
    // MFMA chains (even and odd k-steps) halve the dependent latency
    f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
    const int swn = tile_swz(n);
#pragma unroll
    for (int ks = 0; ks < 8; ks += 2) {
      const u32x4_t k0 =
          *reinterpret_cast<const u32x4_t*>(tk + n * D + 8 * ((2 * ks + hh) ^ swn));
      const u32x4_t k1 =
          *reinterpret_cast<const u32x4_t*>(tk + n * D + 8 * ((2 * ks + 2 + hh) ^ swn));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k0), qop[ks], s0,
                                                  0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, k1), qop[ks + 1],
                                                  s1, 0, 0, 0);
    }
    // V^T operand of k-step u, d tile dt: lane (j = lane & 15 of group gq) points at row
    // 16u + 8 iota + 4hh + j/4, columns 32 dt + 16 (gq & 1) + 4 (j & 3) .. +3. The reads are
    // issued now (inline assembly, waited for explicitly before the PV products), so their
    // latency overlaps the softmax; this tile's copy has already landed.
    const int gq = lane >> 4, j = lane & 15;
    const uint32_t tv_base = (uint32_t)reinterpret_cast<uintptr_t>(DF2_LDS(tv));
    uint64_t vt[4][2][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + 16 * (gq & 1) + 4 * (j & 3);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int io = 0; io < 2; ++io) {
          const int r = 16 * u + 8 * io + 4 * hh + (j >> 2);
          const int c = (d >> 3) ^ tile_swz(r);
          const uint32_t a = tv_base + 2u * (uint32_t)(r * D + 8 * c + (d & 7));
          asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(vt[dt][u][io]) : "v"(a));
        }
    }
    f32x16_t sc = s0 + s1;
    const int kk0 = tile * kTileKeys;
    // A tile of context keys visible to every query (all but the window's first tile and
    // the tiles holding block keys) needs no mask, and with a positive scale the scaling
    // folds into the exponent's fma: max(scale s) = scale max(s). Otherwise the scores are
    // masked and scaled first (sl = 1 then).
    const bool fused = kk0 >= kmin_all && kk0 + kTileKeys <= nctx && scale_log2 > 0.0f;
    float sl = scale_log2;
    if (!fused) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kk0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        const bool vis = kk < nctx ? kk >= kmin : kk < nkeys;
        sc[i] = vis ? sc[i] * scale_log2 : -INFINITY;
      }
      sl = 1.0f;
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    mx = fmaxf(mx, __uint_as_float(lane_xor32(__float_as_uint(mx), lane)));
    const float mnew = fmaxf(m, mx * sl);
    // Lazy rescale: the running maximum m is moved (and o, l rescaled) only when some
    // query's maximum has grown by more than kLazyLog2 since; until then the stale m is
    // the exponent base, so every weight stays below 2^kLazyLog2. The softmax is the same
    // for any base; only the rounding of the intermediate sums differs.
    if (__ballot(mnew > m + kLazyLog2) != 0) {
      const float nb = mnew == -INFINITY ? 0.0f : mnew;
      const float alpha = exp2f(m - nb);
      if (!first) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
      }
      l *= alpha;
      m = mnew;
    }
    const float base = m == -INFINITY ? 0.0f : m;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sc[i] = exp2f(fmaf(sc[i], sl, -base));
      psum += sc[i];
    }
    psum += __uint_as_float(lane_xor32(__float_as_uint(psum), lane));
    l += psum;
    bf16x8_t pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[u][e] = (__bf16)sc[8 * u + e];
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(vt[0][0][0]), "+v"(vt[0][0][1]), "+v"(vt[0][1][0]), "+v"(vt[0][1][1]),
                   "+v"(vt[1][0][0]), "+v"(vt[1][0][1]), "+v"(vt[1][1][0]), "+v"(vt[1][1][1]),
                   "+v"(vt[2][0][0]), "+v"(vt[2][0][1]), "+v"(vt[2][1][0]), "+v"(vt[2][1][1]),
                   "+v"(vt[3][0][0]), "+v"(vt[3][0][1]), "+v"(vt[3][1][0]), "+v"(vt[3][1][1]));
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const u32x4_t w4 = {(uint32_t)vt[dt][u][0], (uint32_t)(vt[dt][u][0] >> 32),
                            (uint32_t)vt[dt][u][1], (uint32_t)(vt[dt][u][1] >> 32)};
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w4), pb[u],
                                                       o[dt], 0, 0, 0);
      }
    }
  };

  // two tiles in flight from the start; tile k + 2 reuses tile k's buffer once it is read
  if (nmine > 0) issue(tbeg + w, 0);
  if (nmine > 1) issue(tbeg + w + NW, 1);
  for (int k = 0; k < nmine; ++k) {
    const int tile = tbeg + w + NW * k;
    if (k + 1 < nmine)
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");  // tile k + 1's 16 copies may fly on
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    compute(tile, k & 1, k == 0);
    if (k + 2 < nmine) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // tile k's LDS reads have returned
      issue(tile + 2 * NW, k & 1);
    }
  }

  // merge: every wave stores its state; wave w then combines columns [32w, 32w + 32)
  __syncthreads();  // all tile reads are done before the buffers are reused
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * dt + 8 * (r >> 2) + 4 * hh + (r & 3);
      sm.o[w][d][n] = o[dt][r];
    }
  if (hh == 0) {
    sm.m[w][n] = m;
    sm.l[w][n] = l;
  }
  __syncthreads();
  float mw[NW], M = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    mw[v] = sm.m[v][n];
    M = fmaxf(M, mw[v]);
  }
  float aw[NW], Lsum = 0.0f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    aw[v] = M == -INFINITY ? 0.0f : exp2f(mw[v] - M);
    Lsum += aw[v] * sm.l[v][n];
  }
  // lane (n, hh): query row n, CPL columns from d0
  constexpr int CPL = D / NW / 2;
  const int d0 = (D / NW) * w + CPL * hh;
  float acc[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    float a = 0.0f;
#pragma unroll
    for (int v = 0; v < NW; ++v) a += aw[v] * sm.o[v][d0 + e][n];
    acc[e] = a;
  }
  if (nsplit == 1) {
    if (!qvalid) return;
    const float inv = 1.0f / Lsum;
    uint16_t* dst = out + (((int64_t)b * P + slot_n) * Hq + head_n) * D + d0;
    u32x4_t pk[CPL / 8];
#pragma unroll
    for (int h = 0; h < CPL / 2; ++h)
      pk[h >> 2][h & 3] = (uint32_t)f32_to_bf16(acc[2 * h] * inv) |
                          ((uint32_t)f32_to_bf16(acc[2 * h + 1] * inv) << 16);
#pragma unroll
    for (int v = 0; v < CPL / 8; ++v) store_nt(reinterpret_cast<u32x4_t*>(dst + 8 * v), pk[v]);
    return;
  }
  const int64_t part = ((int64_t)b * Hkv + g) * nsplit + split;
  float* po = ws_o + (part * kRows + n) * D + d0;
#pragma unroll
  for (int e = 0; e < CPL; e += 4) {
#if DF2_ATTN_NT_PARTIAL
    store_nt(reinterpret_cast<u32x4_t*>(po + e),
             u32x4_t{__float_as_uint(acc[e]), __float_as_uint(acc[e + 1]),
                     __float_as_uint(acc[e + 2]), __float_as_uint(acc[e + 3])});
#else
    *reinterpret_cast<float4*>(po + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
#endif
  }
  if (w == 0 && hh == 0) ws_ml[part * kRows + n] = make_float2(M, Lsum);
}

// Combines the splits of one (sequence, KV head, slice of CPW columns). Each thread (query
// row n, 4 columns) issues the loads of all its split partials first; meanwhile the
// (max, sum) pairs of all splits are read into LDS and turned into weights. Small batches
// use narrow slices, so that enough workgroups share the reads.
template <int D, int MS, int CPW>
__global__ __launch_bounds__(kRows * CPW / 4) void attn_combine_kernel(
    const float* __restrict__ ws_o, const float2* __restrict__ ws_ml, int P, int Hq, int Hkv,
    int nsplit, uint16_t* __restrict__ out) {
  constexpr int TPR = CPW / 4;       // threads per query row
  constexpr int NT = kRows * TPR;    // threads per workgroup
  __shared__ float wgt[MS][kRows], lsum[MS][kRows];
  __shared__ float inv_den[kRows];
  const int g = blockIdx.x, b = blockIdx.y, slice = blockIdx.z;
  const int t = threadIdx.x;
  const int G = Hq / Hkv, rows = P * G;
  const int64_t p0 = ((int64_t)b * Hkv + g) * nsplit;
  const int n = t / TPR, c = t % TPR;
  const int d = slice * CPW + c * 4;
  float4 v[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const int sc = s < nsplit ? s : nsplit - 1;  // in range, so the loads carry no conditions
    v[s] = *reinterpret_cast<const float4*>(ws_o + ((p0 + sc) * kRows + n) * D + d);
  }
  for (int e = t; e < MS * kRows; e += NT) {
    const int s = e / kRows;
    const float2 ml = s < nsplit ? ws_ml[p0 * kRows + e] : make_float2(-INFINITY, 0.0f);
    wgt[s][e % kRows] = ml.x;
    lsum[s][e % kRows] = ml.y;
  }
  __syncthreads();
  if (t < kRows) {
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < MS; ++s) M = fmaxf(M, wgt[s][t]);
    float den = 0.0f;
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const float ms = wgt[s][t];
      const float w = ms == -INFINITY ? 0.0f : exp2f(ms - M);
      den += w * lsum[s][t];
      wgt[s][t] = w;  // splits past nsplit (and empty ones) weigh 0
    }
    inv_den[t] = 1.0f / den;
  }
  __syncthreads();
  if (n >= rows) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const float w = wgt[s][n];
    acc.x += w * v[s].x;
    acc.y += w * v[s].y;
    acc.z += w * v[s].z;
    acc.w += w * v[s].w;
  }
  const float inv = inv_den[n];
  const int slot = n / G, head = g * G + n % G;
  uint16_t* dst = out + (((int64_t)b * P + slot) * Hq + head) * D + d;
  const uint32_t lo2 = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi2 = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  store_nt(reinterpret_cast<u32x2_t*>(dst), u32x2_t{lo2, hi2});
}

template <int D, int CPW>
void launch_combine_w(const float* ws_o, const float2* ws_ml, int B, int P, int Hq, int Hkv,
                      int nsplit, uint16_t* out, hipStream_t stream) {
  const dim3 grid(Hkv, B, D / CPW);
  constexpr int NT = kRows * CPW / 4;
  if (nsplit <= 4)
    attn_combine_kernel<D, 4, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else if (nsplit <= 8)
    attn_combine_kernel<D, 8, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else if (nsplit <= 12)
    attn_combine_kernel<D, 12, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else if (nsplit <= 16)
    attn_combine_kernel<D, 16, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else if (nsplit <= 20)
    attn_combine_kernel<D, 20, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else if (nsplit <= 24)
    attn_combine_kernel<D, 24, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
  else
    attn_combine_kernel<D, 32, CPW><<<grid, NT, 0, stream>>>(ws_o, ws_ml, P, Hq, Hkv, nsplit, out);
}

template <int D>
void launch_combine(const float* ws_o, const float2* ws_ml, int B, int P, int Hq, int Hkv,
                    int nsplit, uint16_t* out, hipStream_t stream) {
#ifndef DF2_COMBINE_CPW_SMALL
#define DF2_COMBINE_CPW_SMALL 32
#endif
  // small batches may use narrower slices (more workgroups share the reads)
  if ((int64_t)B * Hkv * (D / 32) < 256)
    launch_combine_w<D, DF2_COMBINE_CPW_SMALL>(ws_o, ws_ml, B, P, Hq, Hkv, nsplit, out, stream);
  else
    launch_combine_w<D, 32>(ws_o, ws_ml, B, P, Hq, Hkv, nsplit, out, stream);
}

// f32: keys in LDS tiles of 64; a lane scores one key per row, then accumulates columns.
constexpr int kF32Waves = 16;                    // one workgroup per (sequence, KV head)
constexpr int kF32RowsPerWave = 64 / kF32Waves;  // query rows per wave (at most 64 rows)

template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kb, const float* __restrict__ vb,
    const float* __restrict__ kr, const float* __restrict__ vr, const int32_t* __restrict__ ctx_len,
    int P, int Hq, int Hkv, int S, int W, float scale, float* __restrict__ out) {
  // binary32 path (small shapes: at most 64 query rows per KV head, D 64 or 128). The keys of
  // one (sequence, KV head) are listed as slot 0's window (the widest) then the P block
  // keys, and go through LDS in tiles of 64, each one coalesced round trip. Per tile, lane
  // j of a wave scores key j against one query row, the wave takes the tile's maximum and
  // sum by shuffles (online softmax), and lane d accumulates output columns d and d + 64
  // over the tile's keys. A key outside a row's window gets weight 0. The dot products and
  // the column sums each run four partial sums (fixed order), so the LDS reads pipeline.
  constexpr int T = 64;
  __shared__ float qs[64][D];
  __shared__ float ks[T][D + 1];  // padded: lanes read 64 different rows of one column
  __shared__ float vs[T][D];
  __shared__ float ps[kF32Waves][T];
  const int g = blockIdx.x, b = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int G = Hq / Hkv, rows = P * G;
  int L = ctx_len[b];
  L = L < 0 ? 0 : L;
  const int j0 = L - W + 1 > 0 ? L - W + 1 : 0;  // oldest context position of slot 0
  const int nctx = L - j0, nkeys = nctx + P;
  for (int e = t; e < rows * D; e += 64 * kF32Waves) {
    const int n = e / D, d = e - n * D;
    qs[n][d] = q[(((int64_t)b * P + n / G) * Hq + g * G + n % G) * D + d];
  }
  // per-row online-softmax state; wave w owns rows w, w + kF32Waves, ...
  float m[kF32RowsPerWave], l[kF32RowsPerWave], o0[kF32RowsPerWave], o1[kF32RowsPerWave];
#pragma unroll
  for (int r = 0; r < kF32RowsPerWave; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0f;
    o0[r] = 0.0f;
    o1[r] = 0.0f;
  }
  for (int k0 = 0; k0 < nkeys; k0 += T) {
    __syncthreads();  // the previous tile is no longer read (and qs is written)
    for (int e = t; e < T * D; e += 64 * kF32Waves) {
      const int j = e / D, d = e - j * D, kk = k0 + j;
      float kv = 0.0f, vv = 0.0f;
      if (kk < nkeys) {
        const int64_t r = kk < nctx
            ? (((int64_t)b * S + (j0 + kk) % S) * Hkv + g) * D
            : (((int64_t)b * P + (kk - nctx)) * Hkv + g) * D;
        kv = (kk < nctx ? kr : kb)[r + d];
        vv = (kk < nctx ? vr : vb)[r + d];
      }
      ks[j][d] = kv;
      vs[j][d] = vv;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kF32RowsPerWave; ++r) {
      const int n = w + kF32Waves * r;
      if (n >= rows) continue;  // uniform over the wave
      const int slot = n / G;
      const int kk = k0 + lane;
      // context key kk (position j0 + kk) is in slot's window iff j0 + kk >= L + slot - W + 1
      const bool vis = kk < nctx ? j0 + kk >= L + slot - W + 1 : kk < nkeys;
      float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < D; d += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) s4[u] += qs[n][d + u] * ks[lane][d + u];
      float sc = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      sc = vis ? sc * scale : -INFINITY;
      float tmax = sc;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
      const float mn = fmaxf(m[r], tmax);
      const float base = mn == -INFINITY ? 0.0f : mn;
      const float a = expf(m[r] - base);
      const float pj = vis ? expf(sc - base) : 0.0f;
      float psum = pj;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) psum += __shfl_xor(psum, o, 64);
      ps[w][lane] = pj;
      __builtin_amdgcn_wave_barrier();
      float a0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, a1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < T; j += 4)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float pv = ps[w][j + u];
          a0[u] += pv * vs[j + u][lane];
          if constexpr (D > 64) a1[u] += pv * vs[j + u][lane + 64];
        }
      const float acc0 = (a0[0] + a0[1]) + (a0[2] + a0[3]);
      const float acc1 = (a1[0] + a1[1]) + (a1[2] + a1[3]);
      __builtin_amdgcn_wave_barrier();  // ps is rewritten for the next row
      l[r] = l[r] * a + psum;
      o0[r] = o0[r] * a + acc0;
      o1[r] = o1[r] * a + acc1;
      m[r] = mn;
    }
  }
#pragma unroll
  for (int r = 0; r < kF32RowsPerWave; ++r) {
    const int n = w + kF32Waves * r;
    if (n >= rows) continue;
    float* dst = out + (((int64_t)b * P + n / G) * Hq + g * G + n % G) * D;
    dst[lane] = o0[r] / l[r];
    if constexpr (D > 64) dst[lane + 64] = o1[r] / l[r];
  }
}

struct SplitPlan {
  int nsplit;
  int stages_per_split;
  int nw;  // waves per workgroup (streaming kernel)
};

// Enough workgroups to cover the chip at small batch, one split per (sequence, KV head)
// once the batch alone does.
SplitPlan plan_splits(int B, int Hkv, int W) {
  const int stages = (W - 1 + kStage - 1) / kStage;  // stages of the widest window
  const int want = (kAttnTargetWGs + B * Hkv - 1) / (B * Hkv);
  int cap = stages / kAttnMinStages > 1 ? stages / kAttnMinStages : 1;
  cap = cap < kMaxSplits ? cap : kMaxSplits;
  int ns = want < cap ? want : cap;
  ns = ns < 1 ? 1 : ns;
  SplitPlan p;
  p.stages_per_split = (stages + ns - 1) / ns;
  p.stages_per_split = p.stages_per_split < 1 ? 1 : p.stages_per_split;
  p.nsplit = (stages + p.stages_per_split - 1) / p.stages_per_split;
  p.nsplit = p.nsplit < 1 ? 1 : p.nsplit;
  p.nw = 4;
  return p;
}

// D = 128 streaming kernel. Up to one (sequence, KV head) per compute unit, workgroups of
// four waves, split so that a launch has about kStreamTargetWGs workgroups (one per unit:
// the tile buffers allow one such workgroup per unit) with at least one tile per wave.
// Beyond that, workgroups of two waves, two per unit, one per (sequence, KV head).
#ifndef DF2_STREAM_TARGET_WGS
#define DF2_STREAM_TARGET_WGS 256
#endif
#ifndef DF2_STREAM_NW
#define DF2_STREAM_NW 0  // 0: by the batch
#endif
constexpr int kComputeUnits = 256;
SplitPlan plan_stream(int B, int Hkv, int P, int W) {
  const int ntiles = (W - 1 + P + kTileKeys - 1) / kTileKeys;  // tiles of the longest list
  const int units = B * Hkv;
  const int nw = DF2_STREAM_NW ? DF2_STREAM_NW : (units > kComputeUnits ? 2 : 4);
  int ns = (DF2_STREAM_TARGET_WGS + units - 1) / units;
  const int by_tiles = (ntiles + nw - 1) / nw;
  ns = ns < by_tiles ? ns : by_tiles;
  ns = ns < kMaxSplits ? ns : kMaxSplits;
  ns = ns < 1 ? 1 : ns;
  SplitPlan p;
  p.stages_per_split = (ntiles + ns - 1) / ns;  // tiles per split
  p.nsplit = (ntiles + p.stages_per_split - 1) / p.stages_per_split;
  p.nw = nw;
  return p;
}

SplitPlan plan_for(int B, int Hkv, int P, int D, int W) {
  return D == kStreamD ? plan_stream(B, Hkv, P, W) : plan_splits(B, Hkv, W);
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_block_attn_workspace_bytes(int B, int P, int Hq, int Hkv, int D, int S,
                                                     int W, int dtype) {
  (void)Hq;
  (void)S;
  if (B < 1 || Hkv < 1 || W < 1 || P < 1 || (D != 64 && D != 128)) return 0;
  if (dtype != DFLASH2_BF16) return 0;
  const SplitPlan sp = plan_for(B, Hkv, P, D, W);
  if (sp.nsplit == 1) return 0;
  const size_t parts = (size_t)B * Hkv * sp.nsplit;
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
    if (D == 64)
      attn_f32_kernel<64><<<dim3(Hkv, B), 64 * kF32Waves, 0, stream>>>(
          (const float*)q, (const float*)k_blk, (const float*)v_blk, (const float*)k_ring,
          (const float*)v_ring, ctx_len, P, Hq, Hkv, S, W, scale, (float*)out);
    else
      attn_f32_kernel<128><<<dim3(Hkv, B), 64 * kF32Waves, 0, stream>>>(
          (const float*)q, (const float*)k_blk, (const float*)v_blk, (const float*)k_ring,
          (const float*)v_ring, ctx_len, P, Hq, Hkv, S, W, scale, (float*)out);
    return launch_status();
  }
  if (dtype != DFLASH2_BF16) return DFLASH2_EUNSUPPORTED;
  if (rows > kRows) return DFLASH2_EUNSUPPORTED;
  for (const void* p : {q, k_blk, v_blk, k_ring, v_ring, (const void*)out})
    if (!aligned(p, 16)) return DFLASH2_EUNSUPPORTED;
  const size_t need = dflash2_block_attn_workspace_bytes(B, P, Hq, Hkv, D, S, W, dtype);
  if (need && (!ws || !aligned(ws, kWsAlign) || ws_bytes < need)) return DFLASH2_EWORKSPACE;
  const SplitPlan sp = plan_for(B, Hkv, P, D, W);
  const size_t parts = (size_t)B * Hkv * sp.nsplit;
  // workspace: partial outputs, then their (max, sum)
  float* ws_o = need ? (float*)ws : nullptr;
  float2* ws_ml =
      need ? (float2*)((char*)ws + round_up(parts * kRows * D * sizeof(float), kWsAlign)) : nullptr;
  const float sl2 = scale * kLog2e;
  dim3 grid(sp.nsplit, Hkv, B);
  if (D == 128) {
    if (sp.nw == 2)
      attn_stream_kernel<2><<<grid, 128, 0, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_blk, (const uint16_t*)v_blk,
          (const uint16_t*)k_ring, (const uint16_t*)v_ring, ctx_len, P, Hq, Hkv, S, W, sl2,
          sp.nsplit, sp.stages_per_split, ws_o, ws_ml, (uint16_t*)out);
    else
      attn_stream_kernel<4><<<grid, 256, 0, stream>>>(
          (const uint16_t*)q, (const uint16_t*)k_blk, (const uint16_t*)v_blk,
          (const uint16_t*)k_ring, (const uint16_t*)v_ring, ctx_len, P, Hq, Hkv, S, W, sl2,
          sp.nsplit, sp.stages_per_split, ws_o, ws_ml, (uint16_t*)out);
    if (sp.nsplit > 1) launch_combine<128>(ws_o, ws_ml, B, P, Hq, Hkv, sp.nsplit, (uint16_t*)out, stream);
  } else {
    attn_split_kernel<64><<<grid, 256, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k_blk, (const uint16_t*)v_blk,
        (const uint16_t*)k_ring, (const uint16_t*)v_ring, ctx_len, P, Hq, Hkv, S, W, sl2,
        sp.nsplit, sp.stages_per_split, ws_o, ws_ml, (uint16_t*)out);
    if (sp.nsplit > 1) launch_combine<64>(ws_o, ws_ml, B, P, Hq, Hkv, sp.nsplit, (uint16_t*)out, stream);
  }
  return launch_status();
}
