// dflash2_topk16: exact top-16 per logits row ("Geramy/LSE docs/DFLASH2.md", top-k policy
// paragraph: equal scores go to the smaller index, NaNs first by index, infinities keep
// their normal order).
//
// A row is cut into wave sub-chunks of 64 x EPT elements, dealt round-robin over the
// waves of the row's workgroups (four waves each), so the workgroups of a row move
// through it side by side. Each wave works on its own, with no workgroup barrier: it
// streams its sub-chunks from HBM straight into its own three LDS buffers with
// global_load_lds (16 bytes per lane), two sub-chunks in flight while the third is
// examined, and keeps its own running candidate list in LDS. Every wave writes the 16
// best of its list as 16 packed (key, ~index) words; the union of a row's lists holds the
// row's top-16 (the order is total), and a second kernel merges them into the exact
// answer. The larger packed word comes first, so ties go to the lower index.
//
// Candidates are admitted by a threshold key T: every top-16 element of the wave's share
// has a key >= T. On the first sub-chunk T is the 16th largest lane maximum (at least 16
// elements reach it), found by a 16- or 32-step bitwise search on ballots; whenever the
// list grows long it is cut to the entries reaching its 16th largest key (found again by a
// ballot search) and T rises to that key, so later sub-chunks admit almost nothing. Any
// wave's threshold is valid for the whole row, so the waves of a workgroup share the
// highest one through LDS. A sub-chunk holding NaN or an infinity (or overflowing
// the list) is instead reduced exactly, by 16 rounds of a wave maximum of packed words
// over canonical keys, and its 16 best appended.
#include "common.hpp"
#include "merge16.hpp"

namespace df2 {
namespace {

#ifndef DF2_TOPK_THREADS
#define DF2_TOPK_THREADS 256
#endif
constexpr int kThreads = DF2_TOPK_THREADS;  // four waves share an admission threshold

#define DF2_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kWaves = kThreads / 64;
#ifndef DF2_TOPK_WCAP
#define DF2_TOPK_WCAP 128
#endif
#ifndef DF2_TOPK_REDUCE_AT
#define DF2_TOPK_REDUCE_AT 64
#endif
constexpr int kWCap = DF2_TOPK_WCAP;           // candidate slots per wave
constexpr int kReduceAt = DF2_TOPK_REDUCE_AT;  // list length that triggers a cut
#ifndef DF2_TOPK_BUFS
#define DF2_TOPK_BUFS 3
#endif
constexpr int kBufs = DF2_TOPK_BUFS;  // LDS buffers per wave (kBufs - 1 sub-chunks in flight)

// s_waitcnt vmcnt(N) for a compile-time N (the instruction takes an immediate)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <class KT, int NV>
struct WaveSmem {
  u32x4_t buf[kWaves][kBufs][NV][64];  // [wave][buffer][vector][lane]
  uint64_t list[kWaves][kWCap];
  uint64_t top[kWaves][kTopK];
  uint32_t shared_tf;  // the highest admission threshold any wave has established
};

template <class KT, int NV, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_wave_kernel(
    const typename KT::elem_t* __restrict__ scores, int64_t seq_stride, int64_t row_stride,
    int row0, int N, int V, int seg_len, int nseg, uint64_t* __restrict__ ws) {
  using E = typename KT::elem_t;
  constexpr int EPV = 16 / (int)sizeof(E);
  constexpr int EPT = NV * EPV;      // elements per lane per sub-chunk
  constexpr int WCH = 64 * EPT;      // elements per wave sub-chunk
  constexpr int KB = 8 * (int)sizeof(E);
  __shared__ WaveSmem<KT, NV> sm;
  const int seg = blockIdx.x, rowid = blockIdx.y;
  const int b = rowid / N, r = rowid % N;
  const E* row = scores + (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  // The row's wave sub-chunks are dealt round-robin: sub-chunk j of wave w of segment seg
  // is the row's sub-chunk (j nseg + seg) 4 + w, so the workgroups of a row move through it
  // side by side.
  (void)seg_len;
  const int s1 = V;
  const int ntot = (V + WCH - 1) / WCH;
  const int first = seg * kWaves + w;
  const int nsub = ntot > first ? (ntot - first + kWaves * nseg - 1) / (kWaves * nseg) : 0;
  auto wbase = [&](int j) { return ((j * nseg + seg) * kWaves + w) * WCH; };
  uint64_t* list = sm.list[w];
  uint64_t* top = sm.top[w];

  // copy of sub-chunk j into buffer slot: vector v of lane l holds elements
  // wb + v * 64 EPV + l EPV .. + EPV - 1 (wb = the sub-chunk start); rows that are not
  // 16-byte aligned go element by element through registers instead (no copy engine)
  // past the last sub-chunk: re-read the row's last whole sub-chunk (unused, and the same
  // for every wave of the row, so it comes from cache)
  const int wb_dummy = V - WCH > 0 ? V - WCH : 0;
  const E* lane_row = row + lane * EPV;
  auto issue = [&](int j, int slot) {
    const int wb = j < nsub ? wbase(j) : wb_dummy;  // wave-uniform
    if (wb + WCH <= V) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
        __builtin_amdgcn_global_load_lds((const void*)(lane_row + wb + v * 64 * EPV),
                                         DF2_LDS(&sm.buf[w][slot][v][0]), 16, 0, 0);
    } else {
      // the row's partial last sub-chunk: vectors past the end re-read the last one
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        int off = wb + v * 64 * EPV + lane * EPV;
        off = off + EPV <= V ? off : V - EPV;
        __builtin_amdgcn_global_load_lds((const void*)(row + off),
                                         DF2_LDS(&sm.buf[w][slot][v][0]), 16, 0, 0);
      }
    }
  };

  uint32_t Tf = 0;  // admission threshold on raw keys
  int cnt = 0;      // list length (wave-uniform)
  // Any wave's threshold is valid for the whole row: at least 16 of the row's elements
  // reach it. So the waves of a workgroup share the highest one through LDS; a stale read
  // only means a lower (still valid) threshold.
  auto publish = [&]() {
    if (lane == 0) __hip_atomic_fetch_max(&sm.shared_tf, Tf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  // cut the list to its best 16; the threshold rises to the 16th key
  auto reduce = [&]() {
    if (lane < kTopK) top[lane] = 0;
    for (int c = lane; c < cnt; c += 64) {
      const uint64_t v = list[c];
      int rank = 0;
      for (int o = 0; o < cnt; ++o) rank += list[o] > v;
      if (rank < kTopK) top[rank] = v;
    }
    if (lane < kTopK) list[lane] = top[lane];
    if (cnt >= kTopK) {
      const uint32_t T = cand_key(list[kTopK - 1]);
      Tf = T == KT::kPosZero ? T - 1 : T;  // -0 ranks equal to +0
      publish();
    }
    cnt = cnt < kTopK ? cnt : kTopK;
  };

  // Cheaper cut while streaming: keep the entries whose key reaches the list's 16th largest
  // key (found by a bitwise search on ballots over all entries; at least 16 are kept, more
  // only with ties) and raise the threshold to that key. If ties keep the list long, the
  // exact cut follows.
  auto shrink = [&]() {
    uint64_t e[kWCap / 64];
#pragma unroll
    for (int i = 0; i < kWCap / 64; ++i) {
      const int c = lane + 64 * i;
      e[i] = c < cnt ? list[c] : 0ull;
    }
    uint32_t prefix = 0;
#pragma unroll
    for (int bit = KB - 1; bit >= 0; --bit) {
      const uint32_t c = prefix | (1u << bit);
      int n = 0;
#pragma unroll
      for (int i = 0; i < kWCap / 64; ++i) n += __popcll(__ballot(cand_key(e[i]) >= c));
      if (n >= kTopK) prefix = c;
    }
    const uint64_t below = (1ull << lane) - 1;
    int pos = 0;
#pragma unroll
    for (int i = 0; i < kWCap / 64; ++i) {
      const bool take = e[i] != 0 && cand_key(e[i]) >= prefix;
      const uint64_t m = __ballot(take);
      if (take) list[pos + __popcll(m & below)] = e[i];
      pos += __popcll(m);
    }
    cnt = pos;
    if (prefix > 0) {
      Tf = prefix == KT::kPosZero ? prefix - 1 : prefix;  // -0 ranks equal to +0
      publish();
    }
    if (cnt > kReduceAt / 2) reduce();
  };

  // any sub-chunk, element by element (partial sub-chunks, f32 rows)
  auto process_any = [&](const uint32_t (&bits)[EPT], int j) {
    const int wb = wbase(j);
    uint32_t key[EPT];
    uint32_t kmax = 0, valid = 0;
    bool special = false;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int x = wb + (e / EPV) * 64 * EPV + lane * EPV + (e % EPV);
      const bool ok = x < s1;
      uint32_t k = KT::raw(bits[e]);
      k = ok ? k : 0u;
      valid |= (uint32_t)ok << e;
      special |= ok && (k <= KT::kNegInf || k >= KT::kPosInf);
      key[e] = k;
      kmax = k > kmax ? k : kmax;
    }
    const bool any_special = __ballot(special) != 0;
    if (j == 0) {
      const uint32_t T = wave_kth16<KB>(kmax);
      Tf = T == KT::kPosZero ? T - 1 : T;
      publish();
    }
    const int cnt0 = cnt;
    if (!any_special) {
      const uint64_t below = (1ull << lane) - 1;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const bool take = ((valid >> e) & 1u) && key[e] >= Tf;
        const uint64_t m = __ballot(take);
        if (m) {
          const int pos = cnt + __popcll(m & below);
          if (take && pos < kWCap) {
            const int x = wb + (e / EPV) * 64 * EPV + lane * EPV + (e % EPV);
            const uint32_t k = key[e] == KT::kNegZeroRaw ? KT::kPosZero : key[e];
            list[pos] = pack_cand(k, (uint32_t)x);
          }
          cnt += __popcll(m);
        }
      }
    }
    if (any_special || cnt > kWCap) {
      // exact top-16 of this sub-chunk on canonical keys, appended after the kept list
      uint64_t pk[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int x = wb + (e / EPV) * 64 * EPV + lane * EPV + (e % EPV);
        pk[e] = x < s1 ? pack_cand(KT::canon(bits[e]), (uint32_t)x) : 0ull;
      }
      for (int k = 0; k < kTopK; ++k) {
        uint64_t m = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) m = pk[e] > m ? pk[e] : m;
        const uint64_t g = wave_max_u64_all(m, lane);  // the branch is wave-uniform
        if (lane == 0) list[cnt0 + k] = g;  // 0 (no candidate) ranks last
#pragma unroll
        for (int e = 0; e < EPT; ++e)
          if (g != 0 && pk[e] == g) pk[e] = 0;
      }
      cnt = cnt0 + kTopK;
      reduce();
    } else if (cnt > kReduceAt) {
      shrink();
    }
  };

  // a whole bf16 sub-chunk: keys of two elements per 32-bit operation (the sign-magnitude
  // flip of both halves, then packed 16-bit max and min), so the common case costs about
  // three VALU operations per element; the rare lanes holding a key >= T append after.
  // returns false when the sub-chunk must go through process_any instead (NaN or an
  // infinity present, or the list overflowed; the list is then as it was on entry)
  auto process_bf16 = [&](const u32x4_t (&q)[NV], int j) -> bool {
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const int wb = wbase(j);
    uint32_t key2[NV * 4];
    u16x2_t mx2 = {0, 0}, mn2 = {0xffff, 0xffff};
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t u = q[v][i];
        typedef short i16x2_t __attribute__((ext_vector_type(2)));
        // per half: 0xffff if negative, else 0 (packed arithmetic shift)
        const uint32_t neg = __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2_t, u) >> 15);
        const uint32_t k2 = u ^ (0x80008000u | neg);
        key2[4 * v + i] = k2;
        const u16x2_t kk = __builtin_bit_cast(u16x2_t, k2);
        mx2 = __builtin_elementwise_max(mx2, kk);
        mn2 = __builtin_elementwise_min(mn2, kk);
      }
    const uint32_t kmax = mx2[0] > mx2[1] ? mx2[0] : mx2[1];
    const uint32_t kmin = mn2[0] < mn2[1] ? mn2[0] : mn2[1];
    if (__ballot(kmin <= KT::kNegInf || kmax >= KT::kPosInf)) return false;
    if (j == 0) {
      const uint32_t T = wave_kth16<KB>(kmax);
      Tf = T == KT::kPosZero ? T - 1 : T;
      publish();
    }
    if (__ballot(kmax >= Tf) == 0) return true;
    cnt = __builtin_amdgcn_readfirstlane(cnt);  // wave-uniform: lets the count live in an SGPR
    const int cnt0_fast = cnt;
    // each element position's ballot comes from one 16-bit compare of its half word
    const uint16_t tf16 = (uint16_t)Tf;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint16_t k = (e & 1) ? (uint16_t)(key2[e / 2] >> 16) : (uint16_t)key2[e / 2];
      const bool take = k >= tf16;
      const uint64_t m = __ballot(take);
      if (m) {
        // this lane's rank among the takers: a masked bit count of the lanes below it
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                  (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (take && pos < kWCap) {
          const int x = wb + (e / EPV) * 64 * EPV + lane * EPV + (e % EPV);
          list[pos] = pack_cand(k == KT::kNegZeroRaw ? KT::kPosZero : k, (uint32_t)x);
        }
        cnt += __popcll(m);
      }
    }
    if (cnt > kWCap) {
      cnt = cnt0_fast;  // the kept list is intact below cnt0_fast
      return false;
    }
    if (cnt > kReduceAt) shrink();
    return true;
  };

  // Once the threshold key is above +0, only positive values can be admitted, and raw
  // bf16 bits decide: positive values order like their bits read as signed 16-bit
  // integers, and every negative value reads below them. So one signed packed maximum gives
  // a lane's largest positive value, and one unsigned packed maximum finds -inf or a
  // negative NaN (bits >= 0xff80); a positive NaN or +inf shows as a signed maximum
  // >= 0x7f80. Two VALU operations per two elements, against four for the keys. Returns
  // false, as process_bf16 does, when the sub-chunk must go the exact way.
  auto process_bf16_pos = [&](const u32x4_t (&q)[NV], int j) -> bool {
    typedef short i16x2_t __attribute__((ext_vector_type(2)));
    typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
    const int wb = wbase(j);
    i16x2_t smx = {-32768, -32768};
    u16x2_t umx = {0, 0};
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // (through a named word: a bit cast of a vector element itself compiled to a read
        // of element 0 only)
        const uint32_t u = q[v][i];
        smx = __builtin_elementwise_max(smx, __builtin_bit_cast(i16x2_t, u));
        umx = __builtin_elementwise_max(umx, __builtin_bit_cast(u16x2_t, u));
      }
    const int smax = smx[0] > smx[1] ? smx[0] : smx[1];
    const uint32_t umax = umx[0] > umx[1] ? umx[0] : umx[1];
    if (__ballot(smax >= 0x7f80 || umax >= 0xff80u)) return false;
    const int traw = (int)(Tf ^ 0x8000u);  // the threshold as raw bits of a positive value
    if (__ballot(smax >= traw) == 0) return true;
    cnt = __builtin_amdgcn_readfirstlane(cnt);
    const int cnt0_pos = cnt;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const uint32_t wd = q[e / EPV][(e % EPV) / 2];
      const int r = (e & 1) ? ((int)wd >> 16) : (int)(int16_t)(wd & 0xffffu);
      const bool take = r >= traw;
      const uint64_t m = __ballot(take);
      if (m) {
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                  (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (take && pos < kWCap) {
          const int x = wb + (e / EPV) * 64 * EPV + lane * EPV + (e % EPV);
          list[pos] = pack_cand((uint32_t)r | 0x8000u, (uint32_t)x);  // a positive value's key
        }
        cnt += __popcll(m);
      }
    }
    if (cnt > kWCap) {
      cnt = cnt0_pos;  // the kept list is intact below cnt0_pos
      return false;
    }
    if (cnt > kReduceAt) shrink();
    return true;
  };

  // kBufs buffers: sub-chunks j + 1 .. j + kBufs - 1 are in flight while j is examined.
  // Every iteration issues exactly NV copies (clamped past the end), so "all but the
  // newest (kBufs - 1) NV copies have landed" means sub-chunk j is in LDS.
  if (threadIdx.x == 0) sm.shared_tf = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kBufs - 1; ++i) issue(i, i);
  for (int j = 0; j < nsub; ++j) {
    if (j > 0) {
      const uint32_t st = __hip_atomic_load(&sm.shared_tf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      Tf = st > Tf ? st : Tf;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // sub-chunk j - 1's reads are done
    issue(j + kBufs - 1, (j + kBufs - 1) % kBufs);
    wait_vmcnt<(kBufs - 1) * NV>();
    u32x4_t q[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) q[v] = sm.buf[w][j % kBufs][v][lane];
    const bool whole = wbase(j) + WCH <= s1;
    bool done = false;
    if constexpr (sizeof(E) == 2) {
      if (whole) {
        if (j > 0 && __builtin_amdgcn_readfirstlane(Tf) > KT::kPosZero)
          done = process_bf16_pos(q, j);
        else
          done = process_bf16(q, j);
      }
    }
    if (!done) {
      uint32_t bits[EPT];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          if constexpr (sizeof(E) == 2)
            bits[v * EPV + e] = (q[v][e / 2] >> (16 * (e & 1))) & 0xffffu;
          else
            bits[v * EPV + e] = q[v][e];
        }
      process_any(bits, j);
    }
  }
  // no copy may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (cnt > 0) reduce();  // the best 16, sorted
  uint64_t* out = ws + (((int64_t)rowid * nseg + seg) * kWaves + w) * kTopK;
  if (lane < kTopK) out[lane] = lane < cnt ? list[lane] : 0ull;
}

// Rows that are not 16-byte aligned (or whose length is not a whole number of 16-byte
// vectors): the same per-wave search, with elements loaded through registers.
template <class KT>
__global__ __launch_bounds__(kThreads) void topk_wave_scalar_kernel(
    const typename KT::elem_t* __restrict__ scores, int64_t seq_stride, int64_t row_stride,
    int row0, int N, int V, int seg_len, int nseg, uint64_t* __restrict__ ws) {
  using E = typename KT::elem_t;
  constexpr int EPT = 8;
  constexpr int WCH = 64 * EPT;
  const int seg = blockIdx.x, rowid = blockIdx.y;
  const int b = rowid / N, r = rowid % N;
  const E* row = scores + (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s0 = seg * seg_len;
  const int s1 = s0 + seg_len < V ? s0 + seg_len : V;
  // the wave's exact top-16 kept in lanes 0..15 of `best` (sorted), merged per sub-chunk
  uint64_t best = 0;
  for (int wb = s0 + w * WCH; wb < s1; wb += kWaves * WCH) {
    uint64_t pk[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int x = wb + e * 64 + lane;
      const int xc = x < V ? x : V - 1;
      uint32_t u;
      if constexpr (sizeof(E) == 2)
        u = reinterpret_cast<const uint16_t*>(row)[xc];
      else
        u = __float_as_uint(reinterpret_cast<const float*>(row)[xc]);
      pk[e] = x < s1 ? pack_cand(KT::canon(u), (uint32_t)x) : 0ull;
    }
    // 16 rounds of a wave maximum over this sub-chunk and the kept list
    uint64_t kept = lane < kTopK ? best : 0ull;
    uint64_t nb = 0;
    for (int k = 0; k < kTopK; ++k) {
      uint64_t m = kept;
#pragma unroll
      for (int e = 0; e < EPT; ++e) m = pk[e] > m ? pk[e] : m;
      const uint64_t g = wave_max_u64(m);
      if (lane == k) nb = g;
      if (g != 0) {
        if (kept == g) kept = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e)
          if (pk[e] == g) pk[e] = 0;
      }
    }
    best = nb;
  }
  uint64_t* out = ws + (((int64_t)rowid * nseg + seg) * kWaves + w) * kTopK;
  if (lane < kTopK) out[lane] = best;
}

// The value reported for a merged candidate: the row element itself, widened to binary32.
template <class KT>
struct ElementValue {
  const typename KT::elem_t* scores;
  int64_t seq_stride, row_stride;
  int row0, N;
  // The lists hold canonical order keys, which give back the element's bits by undoing the
  // sign-magnitude flip, except the NaN key (payload lost) and the zero key (sign lost):
  // only those two read the element from the row.
  __device__ float operator()(int rowid, uint32_t x, uint32_t key) const {
    if (key != KT::kNaN && key != KT::kPosZero) {
      constexpr uint32_t kSign = KT::kPosZero;  // the key's top bit: a non-negative element
      const uint32_t mask = sizeof(typename KT::elem_t) == 2 ? 0xffffu : 0xffffffffu;
      return KT::widen((key & kSign) ? (key ^ kSign) : (~key & mask));
    }
    const int b = rowid / N, r = rowid % N;
    const typename KT::elem_t* row = scores + (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
    uint32_t u;
    if constexpr (sizeof(typename KT::elem_t) == 2)
      u = reinterpret_cast<const uint16_t*>(row)[x];
    else
      u = __float_as_uint(reinterpret_cast<const float*>(row)[x]);
    return KT::widen(u);
  }
};

struct Plan {
  int nv;       // 16-byte vectors per lane per wave sub-chunk
  int vec;      // rows are 16-byte aligned and a whole number of vectors long
  int seg_len;  // elements per workgroup on average (sizes the grid; a multiple of 4 sub-chunks)
  int nseg;     // workgroups per row
};

// Workgroups per launch the grid aims at: 1024 up to 128 rows, 2048 beyond (measured on
// MI355X: at 112 rows 1024 takes 23.8 us per call against 26.2; at 448 rows 2048 takes
// 54.5 against 62.8; batch 1 gets the same plan either way).
#ifndef DF2_TOPK_TARGET_WGS
#define DF2_TOPK_TARGET_WGS 0  // 0: by the number of rows
#endif
#ifndef DF2_TOPK_NV
#define DF2_TOPK_NV 0  // 0: chosen by the batch
#endif

Plan make_plan(int B, int N, int V, int dtype, const void* scores, int64_t seq_stride,
               int64_t row_stride) {
  Plan p;
  const int esz = dtype == DFLASH2_BF16 ? 2 : 4;
  const int epv = 16 / esz;
  const int64_t rows = (int64_t)B * N;
  // two 16-byte vectors per lane per sub-chunk (measured best on MI355X at batch 1 and 64)
  p.nv = DF2_TOPK_NV ? DF2_TOPK_NV : 2;
  const int ch = kThreads * epv * p.nv;
  const int64_t target = DF2_TOPK_TARGET_WGS ? DF2_TOPK_TARGET_WGS : (rows <= 128 ? 1024 : 2048);
  const int64_t want = (target + rows - 1) / rows;  // segments per row wanted
  int64_t seg = (V + want - 1) / want;
  seg = (seg + ch - 1) / ch * ch;
  p.seg_len = (int)seg;
  p.nseg = (int)((V + seg - 1) / seg);
  bool vec = scores == nullptr || aligned(scores, 16);
  vec = vec && ((seq_stride * esz) % 16 == 0) && ((row_stride * esz) % 16 == 0) && V % epv == 0;
  p.vec = vec;
  return p;
}

template <class KT>
void launch_all(const Plan& p, const void* scores, int64_t ss, int64_t rs, int row0, int B, int N,
                int V, uint64_t* ws, int32_t* idx, float* val, hipStream_t st) {
  using E = typename KT::elem_t;
  const dim3 grid(p.nseg, B * N);
  const E* sc = (const E*)scores;
  if (!p.vec)
    topk_wave_scalar_kernel<KT><<<grid, kThreads, 0, st>>>(sc, ss, rs, row0, N, V, p.seg_len,
                                                           p.nseg, ws);
  else if (p.nv == 1)
    topk_wave_kernel<KT, 1, true><<<grid, kThreads, 0, st>>>(sc, ss, rs, row0, N, V, p.seg_len,
                                                             p.nseg, ws);
  else if (p.nv == 2)
    topk_wave_kernel<KT, 2, true><<<grid, kThreads, 0, st>>>(sc, ss, rs, row0, N, V, p.seg_len,
                                                             p.nseg, ws);
  else
    topk_wave_kernel<KT, 4, true><<<grid, kThreads, 0, st>>>(sc, ss, rs, row0, N, V, p.seg_len,
                                                             p.nseg, ws);
  const int nlists = p.nseg * kWaves;
  const size_t lds = (size_t)nlists * sizeof(uint64_t);
  merge16_kernel<ElementValue<KT>><<<B * N, kMergeThreads, lds, st>>>(
      nlists, ws, idx, val, ElementValue<KT>{sc, ss, rs, row0, N});
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_topk16_workspace_bytes(int B, int N, int V, int dtype) {
  if (B < 1 || N < 1 || V < kTopK) return 0;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_F32) return 0;
  const Plan p = make_plan(B, N, V, dtype, nullptr, 0, 0);
  return round_up((size_t)B * N * p.nseg * kWaves * kTopK * sizeof(uint64_t), kWsAlign);
}

extern "C" int dflash2_topk16(const void* scores, int dtype, int B, int N, int row0,
                              int64_t seq_stride, int64_t row_stride, int V, int32_t* idx,
                              float* val, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!scores || !idx || !val || !ws) return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || row0 < 0 || V < kTopK || seq_stride < 0 || row_stride < 0)
    return DFLASH2_EINVAL;
  if ((int64_t)B * N > 65535) return DFLASH2_EUNSUPPORTED;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_F32) return DFLASH2_EUNSUPPORTED;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_topk16_workspace_bytes(B, N, V, dtype))
    return DFLASH2_EWORKSPACE;
  Plan p = make_plan(B, N, V, dtype, scores, seq_stride, row_stride);
  if ((size_t)p.nseg * kWaves * sizeof(uint64_t) > 32 * 1024) return DFLASH2_EUNSUPPORTED;
  if (dtype == DFLASH2_BF16)
    launch_all<KeyBF16>(p, scores, seq_stride, row_stride, row0, B, N, V, (uint64_t*)ws, idx, val,
                        stream);
  else
    launch_all<KeyF32>(p, scores, seq_stride, row_stride, row0, B, N, V, (uint64_t*)ws, idx, val,
                       stream);
  return launch_status();
}
