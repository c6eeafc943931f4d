// dflash2_topk16: exact top-16 per logits row ("Geramy/LSE docs/DFLASH2.md", top-k policy
// paragraph: equal scores go to the smaller index, NaNs first by index, infinities keep
// their normal order).
//
// A row is cut into chunks; one 256-thread workgroup reads one chunk once from HBM with
// 16-byte loads and keeps it in registers, finds the chunk's own top-16, and writes it as
// 16 packed (key, ~index) words. A second kernel merges the chunk lists of a row. The
// union of the chunk top-16 lists holds the row's top-16 (the order is total), so the
// result is exact.
//
// Chunk top-16, fast path: every lane takes the maximum key of its elements; each wave
// sorts its 64 lane maxima and takes the 16th, and the workgroup threshold T is the
// largest of the four. At least 16 elements have a key >= T, so every top-16 element has
// a key >= T. The few elements at or above T are compacted into LDS and each one's rank is
// counted directly. Slow path (NaN or ±inf present, or too many candidates, e.g. a row of
// equal values): 16 rounds of a workgroup-wide maximum of packed words.
#include "common.hpp"

namespace df2 {
namespace {

constexpr int kThreads = kChunkThreads;
constexpr int kCap = 512;  // candidate slots in LDS

// Workgroup maximum of a packed word (all threads must call).
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  uint64_t m = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) m = red[i] > m ? red[i] : m;
  return m;
}

template <class KT, int EPT, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_chunk_kernel(
    const typename KT::elem_t* __restrict__ scores, int64_t seq_stride, int64_t row_stride,
    int row0, int N, int V, int nchunks, uint64_t* __restrict__ ws) {
  constexpr int CH = EPT * kThreads;
  const int chunk = blockIdx.x;
  const int rowid = blockIdx.y;  // b * N + r
  const int b = rowid / N, r = rowid % N;
  const typename KT::elem_t* row =
      scores + (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
  const int base = chunk * CH;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;

  __shared__ uint64_t cand[kCap];
  __shared__ uint64_t red[kThreads / 64];
  __shared__ uint32_t wthr[kThreads / 64];
  __shared__ int count;

  uint32_t bits[EPT];
  if (VEC && base + CH <= V)
    load_chunk_full<KT, EPT>(row, base, bits);
  else
    load_chunk<KT, EPT, VEC>(row, base, V, bits);

  // raw keys; lane maximum; detection of NaN / infinities (valid elements only)
  uint32_t key[EPT];
  uint32_t kmax = 0;
  int special = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bool valid = index_of<EPT, VEC, KT>(base, e) < V;
    uint32_t k = valid ? KT::raw(bits[e]) : 0u;
    special |= valid && (k <= KT::kNegInf || k >= KT::kPosInf);
    key[e] = k;
    kmax = k > kmax ? k : kmax;
  }
  if (t == 0) count = 0;
  const int any_special = __syncthreads_or(special);

  uint64_t* out = ws + ((int64_t)rowid * nchunks + chunk) * kTopK;
  bool slow = any_special != 0;

  if (!slow) {
    uint32_t srt = wave_sort_desc_u32(kmax);
    uint32_t thr = __shfl(srt, 15, 64);
    if (lane == 0) wthr[wv] = thr;
    __syncthreads();
    uint32_t T = wthr[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i) T = wthr[i] > T ? wthr[i] : T;
    // -0 has a raw key one below +0 but ranks equal to it
    uint32_t Tf = (T == KT::kPosZero) ? T - 1 : T;
    if (kmax >= Tf) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        int x = index_of<EPT, VEC, KT>(base, e);
        if (x < V && key[e] >= Tf) {
          uint32_t k = key[e] == KT::kNegZeroRaw ? KT::kPosZero : key[e];
          int pos = atomicAdd(&count, 1);
          if (pos < kCap) cand[pos] = pack_cand(k, (uint32_t)x);
        }
      }
    }
    __syncthreads();
    const int n = count;
    if (n <= kCap) {
      if (t >= n && t < kTopK) out[t] = 0;  // slots beyond the number of candidates stay empty
      for (int c = t; c < n; c += kThreads) {
        uint64_t v = cand[c];
        int rank = 0;
        for (int o = 0; o < n; ++o) rank += cand[o] > v;
        if (rank < kTopK) out[rank] = v;
      }
      return;
    }
    slow = true;
  }

  // slow path: canonical keys, 16 rounds of a workgroup maximum
  uint64_t pk[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    int x = index_of<EPT, VEC, KT>(base, e);
    pk[e] = x < V ? pack_cand(KT::canon(bits[e]), (uint32_t)x) : 0ull;
  }
  for (int k = 0; k < kTopK; ++k) {
    uint64_t m = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) m = pk[e] > m ? pk[e] : m;
    uint64_t g = block_max_u64(m, red);
    if (t == 0) out[k] = g;
    if (g != 0) {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (pk[e] == g) pk[e] = 0;
    }
  }
}

// Merge the chunk lists of one row and write the top-16 (index and widened value). Each
// chunk list is stored best first, so entry 0 is the chunk's maximum. With more than 16
// chunks, T = the 16th largest chunk maximum bounds the answer from below; only the 16
// chunks whose maximum is >= T can hold entries >= T, so at most 256 candidates remain.
template <class KT>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(
    const typename KT::elem_t* __restrict__ scores, int64_t seq_stride, int64_t row_stride,
    int row0, int N, int nchunks, const uint64_t* __restrict__ ws, int32_t* __restrict__ idx,
    float* __restrict__ val) {
  extern __shared__ uint64_t cmax[];  // nchunks chunk maxima
  __shared__ uint64_t cand[kTopK * kTopK];
  __shared__ uint64_t thr;
  __shared__ int count;
  const int rowid = blockIdx.x;
  const int b = rowid / N, r = rowid % N;
  const int n = nchunks * kTopK;
  const uint64_t* src = ws + (int64_t)rowid * n;
  if (threadIdx.x == 0) {
    count = 0;
    thr = 0;
  }
  for (int c = threadIdx.x; c < nchunks; c += kThreads) cmax[c] = src[c * kTopK];
  __syncthreads();
  if (nchunks > kTopK) {
    for (int c = threadIdx.x; c < nchunks; c += kThreads) {
      uint64_t v = cmax[c];
      int rank = 0;
      for (int o = 0; o < nchunks; ++o) rank += cmax[o] > v;
      if (rank == kTopK - 1) thr = v;
    }
    __syncthreads();
  }
  const uint64_t T = thr;
  for (int i0 = 0; i0 < n; i0 += kThreads * 8) {
    uint64_t vals[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + threadIdx.x + kThreads * u;
      vals[u] = i < n ? src[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (vals[u] != 0 && vals[u] >= T) {
        int pos = atomicAdd(&count, 1);
        if (pos < kTopK * kTopK) cand[pos] = vals[u];
      }
    }
  }
  __syncthreads();
  const int m = count < kTopK * kTopK ? count : kTopK * kTopK;
  const typename KT::elem_t* row =
      scores + (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
  for (int c = threadIdx.x; c < m; c += kThreads) {
    uint64_t v = cand[c];
    int rank = 0;
    for (int o = 0; o < m; ++o) rank += cand[o] > v;
    if (rank < kTopK) {
      uint32_t x = cand_idx(v);
      uint32_t u;
      if constexpr (sizeof(typename KT::elem_t) == 2)
        u = reinterpret_cast<const uint16_t*>(row)[x];
      else
        u = __float_as_uint(reinterpret_cast<const float*>(row)[x]);
      idx[(int64_t)rowid * kTopK + rank] = (int32_t)x;
      val[(int64_t)rowid * kTopK + rank] = KT::widen(u);
    }
  }
}

struct Plan {
  int ept;      // elements per thread
  int vec;      // 16-byte loads
  int nchunks;
};

Plan make_plan(int B, int N, int V, int dtype, const void* scores, int64_t seq_stride,
               int64_t row_stride, int row0) {
  Plan p;
  const int esz = dtype == DFLASH2_BF16 ? 2 : 4;
  const int64_t rows = (int64_t)B * N;
  // fewer elements per thread when there are few rows, so that the grid covers the chip
  int ept = esz == 2 ? 32 : 16;
  while (ept > 8 && rows * ((V + ept * kThreads - 1) / (ept * kThreads)) < 1024) ept >>= 1;
  p.ept = ept;
  p.nchunks = (V + ept * kThreads - 1) / (ept * kThreads);
  bool vec = scores == nullptr || aligned(scores, 16);
  vec = vec && ((seq_stride * esz) % 16 == 0) && ((row_stride * esz) % 16 == 0);
  (void)row0;
  p.vec = vec;
  return p;
}

template <class KT, int EPT>
void launch_chunks(const Plan& p, const void* scores, int64_t ss, int64_t rs, int row0, int B,
                   int N, int V, uint64_t* ws, hipStream_t st) {
  dim3 grid(p.nchunks, B * N);
  using E = typename KT::elem_t;
  if (p.vec)
    topk_chunk_kernel<KT, EPT, true><<<grid, kThreads, 0, st>>>((const E*)scores, ss, rs, row0, N, V,
                                                                p.nchunks, ws);
  else
    topk_chunk_kernel<KT, EPT, false><<<grid, kThreads, 0, st>>>((const E*)scores, ss, rs, row0, N,
                                                                 V, p.nchunks, ws);
}

template <class KT>
void launch_all(const Plan& p, const void* scores, int64_t ss, int64_t rs, int row0, int B, int N,
                int V, uint64_t* ws, int32_t* idx, float* val, hipStream_t st) {
  switch (p.ept) {
    case 32: launch_chunks<KT, 32>(p, scores, ss, rs, row0, B, N, V, ws, st); break;
    case 16: launch_chunks<KT, 16>(p, scores, ss, rs, row0, B, N, V, ws, st); break;
    default: launch_chunks<KT, 8>(p, scores, ss, rs, row0, B, N, V, ws, st); break;
  }
  size_t lds = (size_t)p.nchunks * sizeof(uint64_t);
  topk_merge_kernel<KT><<<B * N, kThreads, lds, st>>>((const typename KT::elem_t*)scores, ss, rs,
                                                      row0, N, p.nchunks, ws, idx, val);
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_topk16_workspace_bytes(int B, int N, int V, int dtype) {
  if (B < 1 || N < 1 || V < kTopK) return 0;
  Plan p = make_plan(B, N, V, dtype, nullptr, 0, 0, 0);
  // the plan never picks fewer than 8 elements per thread
  int64_t nch = (V + 8 * kThreads - 1) / (8 * kThreads);
  if (p.nchunks > nch) nch = p.nchunks;
  return round_up((size_t)B * N * nch * kTopK * sizeof(uint64_t), kWsAlign);
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
  Plan p = make_plan(B, N, V, dtype, scores, seq_stride, row_stride, row0);
  if ((size_t)p.nchunks * sizeof(uint64_t) > 32 * 1024) return DFLASH2_EUNSUPPORTED;
  if (dtype == DFLASH2_BF16)
    launch_all<KeyBF16>(p, scores, seq_stride, row_stride, row0, B, N, V, (uint64_t*)ws, idx, val,
                        stream);
  else
    launch_all<KeyF32>(p, scores, seq_stride, row_stride, row0, B, N, V, (uint64_t*)ws, idx, val,
                       stream);
  return launch_status();
}
