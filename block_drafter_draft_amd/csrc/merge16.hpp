// Final merge of per-wave candidate lists into the exact top-16 of a row, shared by
// dflash2_topk16 and dflash2_lmhead_topk16. A candidate is a packed (key << 32) | ~index
// word (larger first, so equal keys go to the lower index); a list is 16 words, best
// first, and 0 marks an empty slot. The union of a row's lists holds the row's top-16.
#pragma once

#include "common.hpp"

namespace df2 {
namespace {

// the 16th largest of the wave's 64 values (bitwise search on ballots; all lanes call)
template <int KB>
__device__ __forceinline__ uint32_t wave_kth16(uint32_t v) {
  uint32_t prefix = 0;
#pragma unroll
  for (int bit = KB - 1; bit >= 0; --bit) {
    const uint32_t c = prefix | (1u << bit);
    if (__popcll(__ballot(v >= c)) >= kTopK) prefix = c;
  }
  return prefix;
}

constexpr int kMergeThreads = 256;
constexpr int kMergeWaves = kMergeThreads / 64;
constexpr int kMCap = 512;

// One workgroup per row (blockIdx.x); the row's lists are ws[rowid][nlists][16]. Writes
// idx/val[rowid][16] with val from VAL (row, index, key). A threshold key Tk is found
// first: each thread takes the largest key among its lists' maxima, and Tk is the largest
// over the waves of the 16th largest of those (ballot search), so at least 16 list maxima
// reach it and every top-16 entry has a key >= Tk. Only lists whose maximum reaches Tk are
// read, and their entries with a key >= Tk are ranked directly. If ties make that set too
// large, the exact 16th largest list maximum T is used instead: at most 16 lists have a
// maximum >= T. Dynamic LDS: nlists words.
template <class VAL>
__global__ __launch_bounds__(kMergeThreads) void merge16_kernel(int nlists,
                                                                const uint64_t* __restrict__ ws,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ val, VAL vf) {
  extern __shared__ uint64_t cmax[];  // nlists list maxima
  __shared__ uint64_t cand[kMCap];
  __shared__ uint32_t wthr[kMergeWaves];
  __shared__ uint64_t thr;
  __shared__ int count;
  const int rowid = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint64_t* src = ws + (int64_t)rowid * nlists * kTopK;
  // A row of at most kRegEntries * 256 entries is loaded whole, in one round trip: thread t
  // holds entries t, t + 256, ... of the row's lists laid end to end; the holders of each
  // list's first entry (its maximum) put it in LDS. Longer rows read the maxima first and
  // then only the lists that can hold winners.
  constexpr int kRegEntries = 4;
  const int ne = nlists * kTopK;
  const bool whole = ne <= kRegEntries * kMergeThreads;
  uint64_t e[kRegEntries];
  if (t == 0) count = 0;
  if (whole) {
#pragma unroll
    for (int i = 0; i < kRegEntries; ++i) {
      const int f = t + kMergeThreads * i;
      e[i] = f < ne ? src[f] : 0ull;
    }
#pragma unroll
    for (int i = 0; i < kRegEntries; ++i) {
      const int f = t + kMergeThreads * i;
      if (f < ne && f % kTopK == 0) cmax[f / kTopK] = e[i];
    }
    __syncthreads();
  } else {
    for (int c = t; c < nlists; c += kMergeThreads) cmax[c] = src[(int64_t)c * kTopK];
  }
  uint32_t kl = 0;
  for (int c = t; c < nlists; c += kMergeThreads) {
    const uint32_t k = cand_key(cmax[c]);
    kl = k > kl ? k : kl;
  }
  const uint32_t tw = wave_kth16<32>(kl);
  if (lane == 0) wthr[w] = tw;
  __syncthreads();
  uint32_t Tk = wthr[0];
#pragma unroll
  for (int i = 1; i < kMergeWaves; ++i) Tk = wthr[i] > Tk ? wthr[i] : Tk;
  uint64_t T = (uint64_t)Tk << 32;  // the smallest packed word with key Tk
  for (int pass = 0; pass < 2; ++pass) {
    if (whole) {
#pragma unroll
      for (int i = 0; i < kRegEntries; ++i) {
        if (e[i] != 0 && e[i] >= T) {
          const int pos = atomicAdd(&count, 1);
          if (pos < kMCap) cand[pos] = e[i];
        }
      }
    } else {
      for (int c = t; c < nlists; c += kMergeThreads) {
        if (cmax[c] == 0 || cmax[c] < T) continue;
        const u32x4_t* l4 = reinterpret_cast<const u32x4_t*>(src + (int64_t)c * kTopK);
        u32x4_t q[kTopK / 2];
#pragma unroll
        for (int i = 0; i < kTopK / 2; ++i) q[i] = l4[i];
#pragma unroll
        for (int i = 0; i < kTopK; ++i) {
          const uint64_t v = ((uint64_t)q[i / 2][2 * (i & 1) + 1] << 32) | q[i / 2][2 * (i & 1)];
          if (v != 0 && v >= T) {
            const int pos = atomicAdd(&count, 1);
            if (pos < kMCap) cand[pos] = v;
          }
        }
      }
    }
    __syncthreads();
    if (count <= kMCap || pass == 1) break;
    // too many ties: the exact 16th largest list maximum
    if (t == 0) thr = 0;
    __syncthreads();
    for (int c = t; c < nlists; c += kMergeThreads) {
      const uint64_t v = cmax[c];
      int rank = 0;
      for (int o = 0; o < nlists; ++o) rank += cmax[o] > v;
      if (rank == kTopK - 1) thr = v;
    }
    __syncthreads();
    T = thr;
    if (t == 0) count = 0;
    __syncthreads();
  }
  const int m = count < kMCap ? count : kMCap;
  for (int c = t; c < m; c += kMergeThreads) {
    const uint64_t v = cand[c];
    const uint32_t x = cand_idx(v);
    const float value = vf(rowid, x, cand_key(v));  // requested before the rank is known
    int rank = 0;
    for (int o = 0; o < m; ++o) rank += cand[o] > v;
    if (rank < kTopK) {
      idx[(int64_t)rowid * kTopK + rank] = (int32_t)x;
      val[(int64_t)rowid * kTopK + rank] = value;
    }
  }
}

}  // namespace
}  // namespace df2
