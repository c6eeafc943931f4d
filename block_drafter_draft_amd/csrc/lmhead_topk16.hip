// dflash2_lmhead_topk16: the drafter's vocabulary projection fused with the top-16. The
// drafter reuses the target's output head ("Geramy/LSE docs/DFLASH2.md", drafter-geometry
// paragraph), and the selector consumes only the top-k head candidates of each block
// position ("qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625", DFlash 2
// commit: top-k lm_head candidates per block position):
//
//   logit[m, v] = sum_c hidden[m, c] * weight[v, c]   (binary32 accumulation of exact
//                                                     bf16 x bf16 products, any order)
//
// and the 16 first (v, logit) of each row m under the top-16 order (the order of
// dflash2_topk16 on binary32 values). The logits are never written to memory.
//
// At small batch the call is one stream of the weight (V x C bf16, 2.54 GB at the drafter
// geometry), so it is bound by HBM. Each wave owns blocks of 32 vocabulary rows (vocabulary
// block j of wave g is g + j * waves) and streams every block in 128-column chunks through
// its own ring of four LDS buffers (8 KiB each) with global_load_lds, three chunks in
// flight while the fourth is multiplied: logit^T[32 v x 32 m] += W[32 v x 128 c] h^T[128 c x 32 m]
// as eight v_mfma_f32_32x32x16_bf16 per chunk, with the W operand read from LDS (16-byte
// chunks XOR-swizzled by row, so the reads hit distinct banks) and the hidden-state operand
// loaded straight into registers (it is small and stays in L2). After a block's last chunk
// each lane holds 16 logits of one hidden row and folds them into its own sorted list of
// the 16 best packed (key, ~index) words. At the end the lists of a workgroup are merged
// (bitonic merges of sorted 16-lists) into one per hidden row, and the shared merge kernel
// picks the exact top-16 of the workgroups' lists. The waves share the vocabulary blocks
// evenly (970 waves of 8 blocks at V = 248320). Hidden rows are taken 32 at a time; more
// rows take more passes over the weight.
#include <type_traits>

#include "common.hpp"
#include "merge16.hpp"

namespace df2 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kLmWaves = 4;                  // waves per workgroup
constexpr int kLmRows = 32;                  // vocabulary rows per block (MFMA M)
constexpr int kLmCols = 32;                  // hidden rows per pass (MFMA N)
constexpr int kLmChunk = 128;                // columns per pipeline item
#ifndef DF2_LMHEAD_BUFS
#define DF2_LMHEAD_BUFS 4
#endif
constexpr int kLmBufs = DF2_LMHEAD_BUFS;     // LDS buffers per wave (3 or 4)
static_assert(kLmBufs == 3 || kLmBufs == 4, "ring depth");
constexpr int kLmTile = kLmRows * kLmChunk;  // bf16 elements per buffer (8 KiB)
#ifndef DF2_LMHEAD_MAX_WAVES
#define DF2_LMHEAD_MAX_WAVES 1024
#endif
constexpr int kLmMaxWaves = DF2_LMHEAD_MAX_WAVES;  // one workgroup of four per compute unit
constexpr int kLmMaxWGs = kLmMaxWaves / kLmWaves;

#define DF2_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt vmcnt(N) for a compile-time N (the instruction takes an immediate)
template <int N>
__device__ __forceinline__ void wait_vmcnt_n() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// chunk swizzle of tile row r (16 chunks of 16 bytes per row)
__device__ __forceinline__ int lm_swz(int r) { return ((r & 3) << 2) ^ ((r >> 2) & 3); }

template <int S>
using Slot = std::integral_constant<int, S>;

__device__ __forceinline__ void cx_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// a := the 16 largest of a and b (both sorted descending), sorted descending: the
// elementwise maximum of a and reversed b is bitonic and holds them, then a bitonic merge.
__device__ __forceinline__ void merge_top16(uint64_t (&a)[kTopK], const uint64_t (&b)[kTopK]) {
#pragma unroll
  for (int i = 0; i < kTopK; ++i) a[i] = a[i] > b[kTopK - 1 - i] ? a[i] : b[kTopK - 1 - i];
#pragma unroll
  for (int d = kTopK / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < kTopK; ++i)
      if ((i & d) == 0) cx_desc(a[i], a[i + d]);
}

// a sorted descending by a bitonic sorting network (80 compare-exchanges, no branches)
__device__ __forceinline__ void sort16_desc(uint64_t (&a)[kTopK]) {
#pragma unroll
  for (int k = 2; k <= kTopK; k <<= 1)
#pragma unroll
    for (int d = k >> 1; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < kTopK; ++i)
        if ((i & d) == 0) {
          if ((i & k) == 0) cx_desc(a[i], a[i + d]);
          else cx_desc(a[i + d], a[i]);
        }
}

// Eight 16-byte loads at p + 16 k elements, k = 0..7, in inline assembly: the compiler
// would otherwise wait for every load in flight before the first use. The caller's explicit
// vmcnt waits cover them (loads retire in order), and tie8 then marks the registers as
// defined at that point, so that no use is scheduled before the wait.
__device__ __forceinline__ void load_h8(u32x4_t (&r)[8], const uint16_t* p) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r[0]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:32" : "=v"(r[1]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:64" : "=v"(r[2]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:96" : "=v"(r[3]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:128" : "=v"(r[4]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:160" : "=v"(r[5]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:192" : "=v"(r[6]) : "v"(p));
  asm volatile("global_load_dwordx4 %0, %1, off offset:224" : "=v"(r[7]) : "v"(p));
}
__device__ __forceinline__ void tie8(u32x4_t (&r)[8]) {
  asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]),
               "+v"(r[6]), "+v"(r[7]));
}

__global__ __launch_bounds__(64 * kLmWaves) void lmhead_stream_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int V, int nwaves, uint64_t* __restrict__ lists) {
  __shared__ uint16_t buf[kLmWaves][kLmBufs][kLmTile];
  const int t = threadIdx.x, lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int gw = blockIdx.x * kLmWaves + w;
  const int nblocks = (V + kLmRows - 1) / kLmRows;
  const int nch = C / kLmChunk;
  const int myblocks = gw < nblocks && gw < nwaves ? (nblocks - 1 - gw) / nwaves + 1 : 0;
  const int items = myblocks * nch;

  // hidden row of MFMA column n in this pass; columns past M read a valid row, and their
  // logits are ignored
  const int m = blockIdx.y * kLmCols + n;
  const bool mvalid = m < M;
  const int mc = mvalid ? m : M - 1;
  const uint16_t* hrow = hid + (int64_t)(mc / N) * hss + (int64_t)(row0 + mc % N) * hrs;

  u32x4_t hreg[kLmBufs][8];
  const int lrow = lane >> 4;
  // item i is chunk i % nch of this wave's block i / nch. The W copy moves rows 4q .. 4q+3
  // per instruction q: lane l fetches chunk (l & 15) ^ swz(row) of row 4q + l / 16 into
  // LDS slot l. The hidden operand of lane (n, hh) for k-step ks is h[m][c0 + 16 ks + 8 hh ..].
  auto issue = [&](int item, auto slot) {
    constexpr int S = decltype(slot)::value;
    item = item < items ? item : items - 1;  // past the end: a copy of the last item, never used
    const int j = item / nch, k = item - j * nch;
    const int v0 = (gw + j * nwaves) * kLmRows;
    const int c0 = k * kLmChunk;
    uint16_t* dst = &buf[w][S][0];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = 4 * q + lrow;
      const int v = v0 + r < V ? v0 + r : V - 1;
      const uint16_t* src = wt + (int64_t)v * C + c0 + 8 * ((lane & 15) ^ lm_swz(r));
      __builtin_amdgcn_global_load_lds((const void*)src, DF2_LDS(dst + q * 512), 16, 0, 0);
    }
    load_h8(hreg[S], hrow + c0 + 8 * hh);
  };

  uint64_t lst[kTopK];
#pragma unroll
  for (int i = 0; i < kTopK; ++i) lst[i] = 0;
  f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
  const int swn = lm_swz(n);

  auto compute = [&](int item, auto slot) {
    constexpr int S = decltype(slot)::value;
    const int j = item / nch, k = item - j * nch;
    const uint16_t* tk = &buf[w][S][0];
    // this item's hidden operand has landed (the caller's vmcnt wait)
    tie8(hreg[S]);
#pragma unroll
    for (int ks = 0; ks < 8; ks += 2) {
      const u32x4_t a0 =
          *reinterpret_cast<const u32x4_t*>(tk + n * kLmChunk + 8 * ((2 * ks + hh) ^ swn));
      const u32x4_t a1 =
          *reinterpret_cast<const u32x4_t*>(tk + n * kLmChunk + 8 * ((2 * ks + 2 + hh) ^ swn));
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a0),
                                                     __builtin_bit_cast(bf16x8_t, hreg[S][ks]),
                                                     acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                     __builtin_bit_cast(bf16x8_t, hreg[S][ks + 1]),
                                                     acc1, 0, 0, 0);
    }
    if (k == nch - 1) {
      // logit of vocabulary row v0 + 8(i/4) + 4hh + i%4 and hidden row m in register i
      const f32x16_t s = acc0 + acc1;
      const int v0 = (gw + j * nwaves) * kLmRows;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        uint64_t c = 0;
        if (mvalid && v < V) c = pack_cand(KeyF32::canon(__float_as_uint(s[i])), (uint32_t)v);
        if (__ballot(c > lst[kTopK - 1])) {
          // insertion into the sorted list; a word below the 16th drops off the end
#pragma unroll
          for (int e = 0; e < kTopK; ++e) {
            const uint64_t hi = lst[e] > c ? lst[e] : c;
            c = lst[e] > c ? c : lst[e];
            lst[e] = hi;
          }
        }
      }
      acc0 = f32x16_t{};
      acc1 = f32x16_t{};
    }
  };

  // With D = kLmBufs buffers, item i + D - 1 goes into the buffer item i - 1 used (its LDS
  // reads were consumed by the MFMAs of item i - 1); then item i's 16 loads are waited for,
  // with the 16 (D - 1) of the next D - 1 items still in flight. Items past the end are
  // issued too (copies of the last one), so every wait is the same and the loop has no
  // data-dependent branches around its loads.
  auto stage = [&](int i, auto slot) {
    constexpr int S = decltype(slot)::value;
    issue(i + kLmBufs - 1, Slot<(S + kLmBufs - 1) % kLmBufs>{});
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(16 * (kLmBufs - 1)) : "memory");
    if (i < items) compute(i, slot);
  };
  if (items > 0) {
    issue(0, Slot<0>{});
    issue(1, Slot<1>{});
    if constexpr (kLmBufs == 4) issue(2, Slot<2>{});
    for (int i = 0; i < items; i += kLmBufs) {
      stage(i, Slot<0>{});
      stage(i + 1, Slot<1>{});
      stage(i + 2, Slot<2>{});
      if constexpr (kLmBufs == 4) stage(i + 3, Slot<3>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // One list per workgroup and hidden row: the two half-waves' lists meet through a lane
  // exchange, then the four waves' lists pairwise through LDS (the tile buffers are free).
  {
    uint64_t o[kTopK];
#pragma unroll
    for (int e = 0; e < kTopK; ++e) {
      const uint32_t lo = __shfl_xor((uint32_t)lst[e], 32, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(lst[e] >> 32), 32, 64);
      o[e] = ((uint64_t)hi << 32) | lo;
    }
    merge_top16(lst, o);
  }
  __syncthreads();  // every wave is done with its tile buffers
  uint64_t* sh = reinterpret_cast<uint64_t*>(&buf[0][0][0]);  // [wave][column][16]
  auto put = [&]() {
    if (hh == 0)
#pragma unroll
      for (int e = 0; e < kTopK; ++e) sh[(w * kLmCols + n) * kTopK + e] = lst[e];
  };
  auto take = [&](int from) {
    uint64_t o[kTopK];
#pragma unroll
    for (int e = 0; e < kTopK; ++e) o[e] = sh[(from * kLmCols + n) * kTopK + e];
    merge_top16(lst, o);
  };
  put();
  __syncthreads();
  if ((w & 1) == 0) {
    take(w + 1);
    put();
  }
  __syncthreads();
  if (w == 0) {
    take(2);
    if (mvalid && hh == 0) {
      uint64_t* out = lists + ((int64_t)m * gridDim.x + blockIdx.x) * kTopK;
#pragma unroll
      for (int e = 0; e < kTopK; e += 2)
        *reinterpret_cast<u32x4_t*>(out + e) =
            u32x4_t{(uint32_t)lst[e], (uint32_t)(lst[e] >> 32), (uint32_t)lst[e + 1],
                    (uint32_t)(lst[e + 1] >> 32)};
    }
  }
}

// More than 32 hidden rows: the workgroup's four waves run in lockstep over the same
// 64-column chunks of 4 BPW neighbouring vocabulary blocks (BPW per wave, 32 rows each),
// and share a tile of 128 hidden rows x 64 columns that the four waves copy into LDS
// together (a quarter each). Per chunk a wave does 4 k-steps x BPW blocks x 4 column
// blocks = 16 BPW MFMA into 4 BPW accumulators. Head tiles (from HBM) and hidden tiles
// (from L2) go through rings of RB LDS buffers, RB - 1 chunks in flight: after the
// barrier that follows chunk i's wait, chunk i + RB - 1 is issued into the buffers chunk
// i - 1 used (every wave has finished it by then). Two blocks per wave (rings of three,
// 144 KiB) measured 7 % faster than one (rings of four) at 448 rows. Loads retire in order, so one wait count serves both
// rings; a deeper head ring would not help, since waiting for a hidden tile also waits
// for every head tile issued before it. 16-byte chunks of the 128-byte LDS rows are XOR-swizzled by (row / 2) % 8, so
// both operands' reads hit distinct banks. Each lane keeps four sorted lists (one per
// column block); at the end the workgroup merges them as in the small kernel.
constexpr int kTlCols = 128;                   // hidden rows per pass
constexpr int kTlChunk = 64;                   // columns per chunk
#ifndef DF2_LMHEAD_BPW
#define DF2_LMHEAD_BPW 2  // vocabulary blocks per wave in the tiled kernel (1 or 2)
#endif
constexpr int kTlW = kLmRows * kTlChunk;       // head tile, bf16 elements (4 KiB)
constexpr int kTlH = kTlCols * kTlChunk;       // hidden tile, bf16 elements (16 KiB)
constexpr int kTlNB = kTlCols / kLmCols;       // column blocks per wave (4)

__device__ __forceinline__ int tl_swz(int r) { return (r >> 1) & 7; }

// BPW: vocabulary blocks per wave; RB: ring depth (RB - 1 chunks in flight)
template <int BPW, int RB>
struct TiledSmem {
  union {
    struct {
      uint16_t w[kLmWaves][RB][BPW * kTlW];    // 64 KiB (BPW 1, RB 4) or 96 KiB (2, 3)
      uint16_t h[RB][kTlH];                    // 64 KiB or 48 KiB
    } ring;
    uint64_t lists[kLmWaves][kTlCols][kTopK];  // 64 KiB, for the final merge
  };
};

// position in a workgroup's sequence of (block group, column chunk) items; it stops at
// the last item, so copies issued past the end repeat the last one (never used)
struct TlCursor {
  int g = 0, k = 0, n = 0;
  __device__ __forceinline__ void next(int nch, int items) {  // selects, no branches
    const int step = n + 1 < items ? 1 : 0;
    n += step;
    k += step;
    const int wrap = k == nch ? 1 : 0;
    k = wrap ? 0 : k;
    g += wrap;
  }
};

// Grid: 1-D, nwg workgroups per pass over the head times npass passes of 128 hidden rows.
// The passes of one workgroup slot x run on the same XCD, dispatched eight apart (index
// (x / 8) 8 npass + 8 p + x % 8; the hardware deals workgroups to the 8 XCDs by index),
// so they stream the same head tiles at about the same time and the XCD's L2 serves all
// but the first read.
template <int BPW, int RB>
__global__ __launch_bounds__(64 * kLmWaves) void lmhead_tiled_kernel(
    const uint16_t* __restrict__ hid, int64_t hss, int64_t hrs, int row0, int N, int M,
    const uint16_t* __restrict__ wt, int C, int V, int ngroups, int nwg, int npass,
    uint64_t* __restrict__ lists) {
  __shared__ TiledSmem<BPW, RB> sm;
  const int L = blockIdx.x;
  const int bx = (L / (8 * npass)) * 8 + L % 8, by = (L / 8) % npass;
  if (bx >= nwg) return;  // the padding of the last group of eight slots
  const int t = threadIdx.x, lane = t & 63, n = lane & 31, hh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int nch = C / kTlChunk;
  // block group g (4 BPW neighbouring blocks; wave w takes blocks BPW w .. BPW w + BPW - 1
  // of it) of workgroup x is x + g * nwg
  const int mygroups = bx < ngroups ? (ngroups - 1 - bx) / nwg + 1 : 0;
  const int items = mygroups * nch;
  const int mbase = by * kTlCols;

  // copy lanes: 8 per 128-byte row, rows 8q + lane/8 of a 32-row quarter, q < 4
  const int lrow = lane >> 3;
  const uint16_t* hsrc[4];  // this wave's quarter of the hidden tile (rows clamped to M - 1)
  int wsw[4];               // swizzled column of the head copy lanes, in elements
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int r = 8 * q + lrow;
    int mr = mbase + 32 * w + r;
    mr = mr < M ? mr : M - 1;
    hsrc[q] = hid + (int64_t)(mr / N) * hss + (int64_t)(row0 + mr % N) * hrs +
              8 * ((lane & 7) ^ tl_swz(32 * w + r));
    wsw[q] = 8 * ((lane & 7) ^ tl_swz(r));
  }
  auto issue_w = [&](const TlCursor& c, int slot) {
    // rows at or past the end read row V - 1 (their products are never used)
    int v0 = (4 * (bx + c.g * nwg) + w) * BPW * kLmRows;
    v0 = v0 < V ? v0 : V - 1;
    const int lim = V - 1 - v0;
    const uint16_t* base = wt + (int64_t)v0 * C + c.k * kTlChunk;
    uint16_t* dw = &sm.ring.w[w][slot][0];
#pragma unroll
    for (int q = 0; q < 4 * BPW; ++q) {
      const int r = 8 * q + lrow;
      const int off = (r < lim ? r : lim) * C + wsw[q & 3];  // (the swizzle repeats every 32 rows)
      __builtin_amdgcn_global_load_lds((const void*)(base + off), DF2_LDS(dw + q * 512), 16,
                                       0, 0);
    }
  };
  auto issue_h = [&](const TlCursor& c, int slot) {
    uint16_t* dh = &sm.ring.h[slot][(32 * w) * kTlChunk];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(hsrc[q] + c.k * kTlChunk),
                                       DF2_LDS(dh + q * 512), 16, 0, 0);
  };

  uint64_t lst[kTlNB][kTopK];
#pragma unroll
  for (int nb = 0; nb < kTlNB; ++nb)
#pragma unroll
    for (int e = 0; e < kTopK; ++e) lst[nb][e] = 0;
  f32x16_t acc[BPW][kTlNB];
#pragma unroll
  for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
    for (int nb = 0; nb < kTlNB; ++nb) acc[bb][nb] = f32x16_t{};
  const int swn = tl_swz(n);

  auto compute = [&](int item, int slot) {
    const int g = item / nch, k = item - g * nch;
    const uint16_t* tw = &sm.ring.w[w][slot][0];
    const uint16_t* th = &sm.ring.h[slot][0];
    // one wave per SIMD: LDS latency is hidden only by reads in flight, so the operand
    // reads run ahead of the products (the schedule is fixed below)
    u32x4_t a[kTlChunk / 16][BPW], bop[kTlChunk / 16][kTlNB];
#pragma unroll
    for (int ks = 0; ks < kTlChunk / 16; ++ks) {
      const int ch = 8 * ((2 * ks + hh) ^ swn);
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb)
        a[ks][bb] = *reinterpret_cast<const u32x4_t*>(tw + (bb * kLmRows + n) * kTlChunk + ch);
#pragma unroll
      for (int nb = 0; nb < kTlNB; ++nb)
        bop[ks][nb] =
            *reinterpret_cast<const u32x4_t*>(th + (nb * kLmCols + n) * kTlChunk + ch);
    }
#pragma unroll
    for (int ks = 0; ks < kTlChunk / 16; ++ks)
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
        for (int nb = 0; nb < kTlNB; ++nb)
          acc[bb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[ks][bb]), __builtin_bit_cast(bf16x8_t, bop[ks][nb]),
              acc[bb][nb], 0, 0, 0);
    // reads of two k-steps ahead, then each k-step's products behind the next one's reads
    constexpr int kRd = BPW + kTlNB, kMf = BPW * kTlNB;  // per k-step
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kRd, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * kMf, 0);
    if (k == nch - 1) {
#pragma unroll
      for (int bb = 0; bb < BPW; ++bb) {
        const int v0 = ((4 * (bx + g * nwg) + w) * BPW + bb) * kLmRows;
#pragma unroll
        for (int nb = 0; nb < kTlNB; ++nb) {
          const bool mvalid = mbase + nb * kLmCols + n < M;
          uint64_t cand[16], cmax = 0;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int v = v0 + 8 * (i >> 2) + 4 * hh + (i & 3);
            cand[i] = mvalid && v < V ? pack_cand(KeyF32::canon(__float_as_uint(acc[bb][nb][i])),
                                                  (uint32_t)v)
                                      : 0ull;
            cmax = cand[i] > cmax ? cand[i] : cmax;
          }
          if (__ballot(cmax > lst[nb][kTopK - 1])) {
            sort16_desc(cand);
            merge_top16(lst[nb], cand);
          }
          acc[bb][nb] = f32x16_t{};
        }
      }
    }
  };

  if (items > 0) {
    TlCursor ci;  // next chunk to issue
#pragma unroll
    for (int j = 0; j < RB - 1; ++j) {
      issue_w(ci, j);
      issue_h(ci, j);
      ci.next(nch, items);
    }
    constexpr int kPerItem = 4 * BPW + 4;  // copies per chunk and wave
    int slot = 0, nslot = RB - 1;          // chunk i's buffers; chunk i + RB - 1's
    for (int i = 0; i < items; ++i) {
      wait_vmcnt_n<(RB - 2) * kPerItem>();  // chunk i's copies have landed
      __builtin_amdgcn_s_barrier();          // ... everyone's, and i - 1 is done
      issue_w(ci, nslot);
      issue_h(ci, nslot);
      ci.next(nch, items);
      compute(i, slot);
      slot = slot + 1 == RB ? 0 : slot + 1;
      nslot = nslot + 1 == RB ? 0 : nslot + 1;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // one list per workgroup and hidden row (half-waves, then waves, by bitonic merges)
#pragma unroll
  for (int nb = 0; nb < kTlNB; ++nb) {
    uint64_t o[kTopK];
#pragma unroll
    for (int e = 0; e < kTopK; ++e) {
      const uint32_t lo = __shfl_xor((uint32_t)lst[nb][e], 32, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(lst[nb][e] >> 32), 32, 64);
      o[e] = ((uint64_t)hi << 32) | lo;
    }
    merge_top16(lst[nb], o);
  }
  __syncthreads();  // every wave is done with the rings
  auto put = [&]() {
    if (hh == 0)
#pragma unroll
      for (int nb = 0; nb < kTlNB; ++nb)
#pragma unroll
        for (int e = 0; e < kTopK; ++e) sm.lists[w][nb * kLmCols + n][e] = lst[nb][e];
  };
  auto take = [&](int from) {
#pragma unroll
    for (int nb = 0; nb < kTlNB; ++nb) {
      uint64_t o[kTopK];
#pragma unroll
      for (int e = 0; e < kTopK; ++e) o[e] = sm.lists[from][nb * kLmCols + n][e];
      merge_top16(lst[nb], o);
    }
  };
  put();
  __syncthreads();
  if ((w & 1) == 0) {
    take(w + 1);
    put();
  }
  __syncthreads();
  if (w == 0) {
    take(2);
    if (hh == 0) {
#pragma unroll
      for (int nb = 0; nb < kTlNB; ++nb) {
        const int m = mbase + nb * kLmCols + n;
        if (m < M) {
          uint64_t* out = lists + ((int64_t)m * nwg + bx) * kTopK;
#pragma unroll
          for (int e = 0; e < kTopK; e += 2)
            *reinterpret_cast<u32x4_t*>(out + e) =
                u32x4_t{(uint32_t)lst[nb][e], (uint32_t)(lst[nb][e] >> 32),
                        (uint32_t)lst[nb][e + 1], (uint32_t)(lst[nb][e + 1] >> 32)};
        }
      }
    }
  }
}

// binary32 value of a canonical key (NaN keys give a quiet NaN)
struct KeyValue {
  __device__ float operator()(int, uint32_t, uint32_t key) const {
    if (key == KeyF32::kNaN) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
  }
};

// Waves that share the vocabulary blocks evenly: the fewest waves (at most kLmMaxWaves)
// for the smallest number of blocks per wave, so no wave has a block more than another.
int lm_waves(int V) {
  const int nblocks = (V + kLmRows - 1) / kLmRows;
  const int per = (nblocks + kLmMaxWaves - 1) / kLmMaxWaves;
  return (nblocks + per - 1) / per;
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_lmhead_topk16_workspace_bytes(int B, int N, int V, int C) {
  if (B < 1 || N < 1 || V < kTopK || C < kLmChunk) return 0;
  return round_up((size_t)B * N * kLmMaxWGs * kTopK * sizeof(uint64_t), kWsAlign);
}

extern "C" int dflash2_lmhead_topk16(const void* hidden, int64_t hid_seq_stride,
                                     int64_t hid_row_stride, int row0, const void* weight, int C,
                                     int V, int B, int N, int32_t* idx, float* val, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!hidden || !weight || !idx || !val || !ws) return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || row0 < 0 || V < kTopK || C < 1 || hid_seq_stride < 0 ||
      hid_row_stride < 0)
    return DFLASH2_EINVAL;
  if (C % kLmChunk != 0) return DFLASH2_EUNSUPPORTED;
  if ((int64_t)B * N > 65535 || V > (1 << 30) / 4) return DFLASH2_EUNSUPPORTED;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || hid_seq_stride % 8 != 0 ||
      hid_row_stride % 8 != 0)
    return DFLASH2_EUNSUPPORTED;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_lmhead_topk16_workspace_bytes(B, N, V, C))
    return DFLASH2_EWORKSPACE;
  const int M = B * N;
  uint64_t* lists = (uint64_t*)ws;
  int nlists;  // one per workgroup
  if (M <= kLmCols) {
    const int nwaves = lm_waves(V);
    nlists = (nwaves + kLmWaves - 1) / kLmWaves;
    lmhead_stream_kernel<<<dim3(nlists, 1), 64 * kLmWaves, 0, stream>>>(
        (const uint16_t*)hidden, hid_seq_stride, hid_row_stride, row0, N, M,
        (const uint16_t*)weight, C, V, nwaves, lists);
  } else {
    // groups of 4 BPW vocabulary blocks shared evenly by at most kLmMaxWGs workgroups
    constexpr int BPW = DF2_LMHEAD_BPW;
    const int ngroups = ((V + kLmRows - 1) / kLmRows + kLmWaves * BPW - 1) / (kLmWaves * BPW);
    const int per = (ngroups + kLmMaxWGs - 1) / kLmMaxWGs;
    nlists = (ngroups + per - 1) / per;
    const int npass = (M + kTlCols - 1) / kTlCols;
    lmhead_tiled_kernel<BPW, BPW == 1 ? 4 : 3>
        <<<dim3((nlists + 7) / 8 * 8 * npass), 64 * kLmWaves, 0, stream>>>(
            (const uint16_t*)hidden, hid_seq_stride, hid_row_stride, row0, N, M,
            (const uint16_t*)weight, C, V, ngroups, nlists, npass, lists);
  }
  merge16_kernel<KeyValue><<<M, kMergeThreads, (size_t)nlists * sizeof(uint64_t), stream>>>(
      nlists, lists, idx, val, KeyValue{});
  return launch_status();
}
