// dflash2_verify: target verification of the N proposals ("Geramy/LSE docs/DFLASH2.md",
// usage paragraph: probability-ratio rejection with residual sampling over all seven
// proposals, greedy keeps the deterministic chain; drafter-geometry paragraph: the target
// consumes the anchor plus all proposals, so an all-accept step has a bonus row).
//
// Kernel 1 (grid: chunks x sequences) reads one row chunk per workgroup:
//   greedy  - row 0: the chunk's first element under the top-16 order (packed word). The
//             greedy chain needs row j only after proposals 1..j have all been accepted, so
//             rows 1..N wait for kernel 2;
//   sampled - the accept chain is cheap (N gathers and N Philox draws, one per lane), so
//             every workgroup of the sequence recomputes it and then reads only the row it
//             will draw from: the chunk sums of the integer weights floor(w * 2^40), both
//             for p_t itself and with the 16 candidates' residual max(0, p_t - q) swapped in.
//             The chain record (accepted count, draw position, residual or not, status
//             bits, and word 2 of the Philox draw at that position) goes to the workspace.
// Kernel 2 (grid: G workgroups per sequence):
//   greedy  - every workgroup reduces row 0's chunk maxima and checks proposal 1. Rejected:
//             workgroup 0 writes the result. Accepted: the G workgroups stream rows 1..N over
//             their share of the chunks and fold each row's best into one word per row with
//             an agent-scope atomic maximum; the last workgroup to arrive (an agent-scope
//             counter) runs the chain on those words. The words and the counter travel only
//             through agent-scope atomics, which are coherent across the XCDs' L2 caches
//             without a release fence (a fence would write back the whole L2).
//   sampled - workgroup 0 picks the chunk holding the draw from the chunk sums and scans
//             that one chunk in index order (each candidate's residual weight computed once,
//             by its own thread). Integer weights make the draw independent of the
//             summation order, so it is bit-exact.
#include <algorithm>

#include "common.hpp"

namespace df2 {
namespace {

constexpr int kThreads = kChunkThreads;
constexpr int kMaxN = 15;
constexpr int kRowWords = 16;    // per-sequence atomic row words (rows 1..N; N <= 15)
#ifndef DF2_VERIFY_RPP
#define DF2_VERIFY_RPP 4
#endif
constexpr int kRowsPerPass = DF2_VERIFY_RPP;  // rows whose chunk loads are in flight together in kernel 2

struct ChainRec {
  int32_t n_acc;   // accepted proposals
  int32_t pos;     // block position of the drawn token (1..N+1)
  int32_t resid;   // 1: draw from the residual of slot pos; 0: from p_t itself
  int32_t flags;   // status bits from the accept tests
  uint64_t draw;   // word 2 of the Philox draw at position pos (the residual draw)
};

struct Ws {
  ChainRec* chain;   // [B]
  uint64_t* best0;   // [B][nchunks] greedy row-0 chunk maxima
  uint64_t* rowmax;  // [B][kRowWords] greedy row maxima of rows 1..N (agent-scope atomics)
  uint32_t* arrive;  // [B] kernel-2 arrivals of an accepted greedy sequence (agent scope)
  uint64_t* zsum;    // [B][nchunks][2] sampled chunk sums (residual, plain)
  int32_t* zflag;    // [B][nchunks] status bits seen in the chunk
};

__host__ __device__ inline size_t ws_layout(int B, int nchunks, Ws* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  size_t o_chain = take(sizeof(ChainRec) * B);
  size_t o_best = take(sizeof(uint64_t) * (size_t)B * nchunks);
  size_t o_row = take(sizeof(uint64_t) * (size_t)B * kRowWords);
  size_t o_arr = take(sizeof(uint32_t) * (size_t)B);
  size_t o_z = take(sizeof(uint64_t) * 2 * (size_t)B * nchunks);
  size_t o_f = take(sizeof(int32_t) * (size_t)B * nchunks);
  if (w && base) {
    w->chain = (ChainRec*)(base + o_chain);
    w->best0 = (uint64_t*)(base + o_best);
    w->rowmax = (uint64_t*)(base + o_row);
    w->arrive = (uint32_t*)(base + o_arr);
    w->zsum = (uint64_t*)(base + o_z);
    w->zflag = (int32_t*)(base + o_f);
  }
  return off;
}

// Agent-scope (whole-GPU) relaxed atomics. Read-modify-write atomics are performed
// coherently for all XCDs; loads and stores at this scope bypass the non-coherent parts of
// the cache hierarchy (sc1). wait_vm makes a thread's earlier memory operations complete
// (performed) before anything after it is issued, and keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t load_agent(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void max_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vm() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Accept chain of a sampled sequence, computed by wave 0 (lane j-1 tests proposal j) and
// published in *rec (LDS). All threads must call; returns after a barrier.
// x and sl are lane t's proposal token and slot (loaded by the caller; t < N); allc/allq
// hold the sequence's candidates and q ([N][16], LDS), written by the caller before the
// call (the barrier on entry orders them).
__device__ void accept_chain(const float* __restrict__ tgt, int64_t row_stride, int V, int N,
                             int32_t x, int32_t sl, const int32_t* allc, const float* allq,
                             uint64_t seed, uint64_t step, int b, ChainRec* rec) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t < 64) {
    bool acc = false, plain = false;
    int fl = 0;
    // lane t draws for position t + 1, lane N for the bonus position N + 1 (whose word 2
    // is the residual draw of an all-accepted chain)
    Draw d = {};
    if (t <= N) d = philox_draw(seed, step, (uint32_t)b, (uint32_t)(t + 1));
    if (t < N) {
      // the target gather goes out first (at a clamped, always valid index)
      const int xc = x < 0 ? 0 : (x >= V ? V - 1 : x);
      const float pt_raw = tgt[(int64_t)t * row_stride + xc];
      const float u = uniform24(d.w[1]);
      if (x < 0 || x >= V) {
        plain = true;
      } else {
        if (sl < 0 || sl >= kTopK || allc[t * kTopK + sl] != x) {
          fl |= DFLASH2_ST_BADTOKEN;
          plain = true;
        } else {
          const float qx = prob_ok(allq[t * kTopK + sl], &fl);
          const float pt = prob_ok(pt_raw, &fl);
          acc = __fmul_rn(u, qx) < pt;
        }
      }
    }
    const uint64_t rej = __ballot(t < N && !acc);
    const int first = rej ? __ffsll((unsigned long long)rej) - 1 : N;  // lane of the rejection
    const int use = (t < N && t <= first) ? fl : 0;
    const int flags = wave_or(use);
    const int plain_first = __shfl(plain ? 1 : 0, first < N ? first : 0, 64);
    const uint32_t dlo = __shfl((uint32_t)d.w[2], first, 64);
    const uint32_t dhi = __shfl((uint32_t)(d.w[2] >> 32), first, 64);
    if (t == 0) {
      rec->n_acc = first;
      rec->pos = first + 1;
      rec->resid = (first < N && !plain_first) ? 1 : 0;
      rec->flags = flags;
      rec->draw = ((uint64_t)dhi << 32) | dlo;
    }
  }
  __syncthreads();
}

// The first element of one row chunk under the top-16 order (packed key and index), over
// the whole workgroup's wave: exact for any contents. Elements at or past V do not count.
template <class KT, int EPT, bool VEC>
__device__ __forceinline__ uint64_t chunk_best_exact(const uint32_t (&bits)[EPT], int base, int V) {
  uint32_t bk = 0, bi = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int x = index_of<EPT, VEC, KT>(base, e);
    const uint32_t k = x < V ? KT::canon(bits[e]) : 0u;
    if (k > bk) {
      bk = k;
      bi = (uint32_t)x;
    }
  }
  return wave_max_u64(bk ? pack_cand(bk, bi) : 0ull);
}

// The same for a chunk that lies wholly inside the row (16-byte loads). Keys are the plain
// sign-magnitude flip; that is the canonical key unless an element is a NaN, or a signed
// zero is a lane's largest key. A wave that sees either goes the exact way; otherwise the
// wave maximum M is found with one 32-bit reduction and its first holder in index order
// by ballots (element e of vector v of lane l sits at v*256*EPV + (64*wave + l)*EPV + e).
template <class KT, int EPT>
__device__ __forceinline__ uint64_t chunk_best_full(const uint32_t (&bits)[EPT], int base, int V) {
  constexpr int EPV = ChunkLoad<KT, EPT>::kEPV;
  constexpr int NV = EPT / EPV;
  uint32_t k[EPT];
  uint32_t mx = 0u, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    k[e] = KT::raw(bits[e]);
    mx = k[e] > mx ? k[e] : mx;
    mn = k[e] < mn ? k[e] : mn;
  }
  const bool special = mx > KT::kPosInf || mn < KT::kNegInf || mx == KT::kNegZeroRaw ||
                       mx == KT::kPosZero;
  if (__ballot(special)) return chunk_best_exact<KT, EPT, true>(bits, base, V);
  const uint32_t M = wave_max_u32_all(mx, threadIdx.x & 63);  // every lane is active here
  const int wv = threadIdx.x >> 6;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    int ef = EPV;
#pragma unroll
    for (int e = EPV - 1; e >= 0; --e) ef = k[v * EPV + e] == M ? e : ef;
    const uint64_t holders = __ballot(ef < EPV);
    if (holders) {
      const int L = __ffsll((unsigned long long)holders) - 1;
      const int e = __shfl(ef, L, 64);
      const int x = base + v * (kChunkThreads * EPV) + (64 * wv + L) * EPV + e;
      return pack_cand(M, (uint32_t)x);
    }
  }
  return 0ull;  // not reached: some lane holds M
}

// Grid: (units of CPW chunks, sequences). A greedy sequence's workgroup reduces its chunks
// of row 0; a sampled sequence's workgroup recomputes the accept chain and sums its chunks
// of the row the draw comes from. Every chunk's loads are issued before any is used, so a
// sampled workgroup spends the chain's dependent round trips once for CPW chunks.
template <class KT, int EPT, bool VEC, int CPW>
__global__ __launch_bounds__(kThreads) void verify_rows_kernel(
    const typename KT::elem_t* __restrict__ target, int64_t seq_stride, int64_t row_stride, int V,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cidx,
    const float* __restrict__ q, const int32_t* __restrict__ slot,
    const float* __restrict__ temperature, uint64_t seed, uint64_t step, int N, int nchunks,
    Ws ws) {
  constexpr int CH = EPT * kThreads;
  const int unit = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int c0 = unit * CPW;                      // first chunk of this workgroup
  const int nc = min(CPW, nchunks - c0);          // its chunks (>= 1)
  __shared__ ChainRec rec;
  __shared__ uint64_t red[kThreads / 64][CPW][2];
  __shared__ int redf[kThreads / 64];

  // a sampled chain's first loads do not depend on the temperature: issue them with it
  // (the proposals and slots, and on an f32 target every slot's candidates and q)
  __shared__ int32_t allc[kMaxN * kTopK];
  __shared__ float allq[kMaxN * kTopK];
  int32_t x_pre = -1, sl_pre = -1;
  if (t < N) {
    x_pre = tokens[(int64_t)b * N + t];
    sl_pre = slot[(int64_t)b * N + t];
  }
  int32_t ci_pre = -1;
  float q_pre = 0.0f;
  if (sizeof(typename KT::elem_t) == 4 && t < N * kTopK) {
    ci_pre = cidx[(int64_t)b * N * kTopK + t];
    q_pre = q[(int64_t)b * N * kTopK + t];
  }
  int st = 0;
  float invT = 0.0f;
  int mode = temp_mode(temperature[b], &invT, &st);
  constexpr bool kIsF32 = sizeof(typename KT::elem_t) == 4;
  if (!kIsF32) mode = 0;
  const typename KT::elem_t* tb = target + (int64_t)b * seq_stride;

  if (mode == 0) {
    // kernel 2's row words and arrival counter for this sequence start at zero
    if (unit == 0 && t < kRowWords) {
      store_agent(ws.rowmax + (int64_t)b * kRowWords + t, 0ull);
      if (t == 0) store_agent(ws.arrive + b, 0u);
    }
    uint32_t bits[CPW][EPT];
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int base = (c0 + cc) * CH;
      if (cc < nc) {
        if (VEC && base + CH <= V)
          load_chunk_full<KT, EPT>(tb, base, bits[cc]);
        else
          load_chunk<KT, EPT, VEC>(tb, base, V, bits[cc]);
      }
    }
#pragma unroll
    for (int cc = 0; cc < CPW; ++cc) {
      const int base = (c0 + cc) * CH;
      uint64_t m = 0;
      if (cc < nc)
        m = (VEC && base + CH <= V) ? chunk_best_full<KT, EPT>(bits[cc], base, V)
                                    : chunk_best_exact<KT, EPT, VEC>(bits[cc], base, V);
      if ((t & 63) == 0) red[t >> 6][cc][0] = m;
    }
    __syncthreads();
    if (t < nc) {
      uint64_t g = red[0][t][0];
      for (int w = 1; w < kThreads / 64; ++w) g = red[w][t][0] > g ? red[w][t][0] : g;
      ws.best0[(int64_t)b * nchunks + c0 + t] = g;
    }
    return;
  }

  // sampled: which row, and with which candidate corrections
  const float* tgt = reinterpret_cast<const float*>(tb);
  if (t < N * kTopK) {
    allc[t] = ci_pre;
    allq[t] = q_pre;
  }
  accept_chain(tgt, row_stride, V, N, x_pre, sl_pre, allc, allq, seed, step, b, &rec);
  if (unit == 0 && t == 0) ws.chain[b] = rec;
  const float* row = tgt + (int64_t)(rec.pos - 1) * row_stride;

  uint32_t bits[CPW][EPT];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int base = (c0 + cc) * CH;
    if (cc < nc) {
      if (VEC && base + CH <= V)
        load_chunk_full<KT, EPT>(reinterpret_cast<const typename KT::elem_t*>(row), base, bits[cc]);
      else
        load_chunk<KT, EPT, VEC>(reinterpret_cast<const typename KT::elem_t*>(row), base, V,
                                 bits[cc]);
    }
  }
  // residual corrections for the candidates of slot pos that fall in these chunks; for a
  // repeated index only its first occurrence counts. Their gathers go out with the chunks.
  bool corr = false;
  int corr_cc = 0;
  float p_c = 0.0f, q_c = 0.0f;
  if (rec.resid && t < kTopK) {
    const int32_t* ci = allc + (rec.pos - 1) * kTopK;
    const int32_t c = ci[t];
    bool first = c >= 0 && c < V;
#pragma unroll
    for (int k = 0; k < kTopK; ++k)
      if (k < t) first = first && ci[k] != c;
    if (first && c >= c0 * CH && c < (c0 + nc) * CH) {
      corr = true;
      corr_cc = c / CH - c0;
      p_c = row[c];
      q_c = allq[(rec.pos - 1) * kTopK + t];
    }
  }
  int fl = 0;
  uint64_t zp[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    const int base = (c0 + cc) * CH;
    zp[cc] = 0;
    if (cc < nc) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int x = index_of<EPT, VEC, KT>(base, e);
        if (x < V) zp[cc] += quant40(prob_ok(__uint_as_float(bits[cc][e]), &fl));
      }
    }
  }
  int64_t dz = 0;
  if (corr) {
    int dummy = 0;
    const float p = prob_ok(p_c, &dummy);
    const float qk = prob_ok(q_c, &fl);
    const float d = __fsub_rn(p, qk);
    dz = (int64_t)quant40(d > 0.0f ? d : 0.0f) - (int64_t)quant40(p);
  }
  fl = wave_or(fl);
#pragma unroll
  for (int cc = 0; cc < CPW; ++cc) {
    uint64_t zr = zp[cc] + (corr && corr_cc == cc ? (uint64_t)dz : 0ull);
    const uint64_t sp = wave_sum_u64_all(zp[cc], t & 63);  // every lane is active here
    zr = wave_sum_u64_all(zr, t & 63);
    if ((t & 63) == 0) {
      red[t >> 6][cc][0] = zr;
      red[t >> 6][cc][1] = sp;
    }
  }
  if ((t & 63) == 0) redf[t >> 6] = fl;
  __syncthreads();
  if (t < nc) {
    uint64_t a = 0, c = 0;
    int f = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      a += red[w][t][0];
      c += red[w][t][1];
      f |= redf[w];
    }
    ws.zsum[((int64_t)b * nchunks + c0 + t) * 2 + 0] = a;
    ws.zsum[((int64_t)b * nchunks + c0 + t) * 2 + 1] = c;
    ws.zflag[(int64_t)b * nchunks + c0 + t] = f;
  }
}

// inclusive scan of a u64 over the workgroup (all threads call)
__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, uint64_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t lo = __shfl_up((uint32_t)v, d, 64), hi = __shfl_up((uint32_t)(v >> 32), d, 64);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    if (lane >= d) v += o;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  uint64_t add = 0;
  for (int i = 0; i < w; ++i) add += wsum[i];
  __syncthreads();
  return v + add;
}

// Grid: B * G workgroups (see below); see the head of this file.
#ifndef DF2_VERIFY_WPE
#define DF2_VERIFY_WPE 0
#endif
template <class KT, int EPT, bool VEC>
__global__
#if DF2_VERIFY_WPE > 0
__launch_bounds__(kThreads, DF2_VERIFY_WPE)
#else
__launch_bounds__(kThreads)
#endif
void verify_finish_kernel(
    const typename KT::elem_t* __restrict__ target, int64_t seq_stride, int64_t row_stride, int V,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cidx,
    const float* __restrict__ q, const float* __restrict__ temperature, uint64_t seed,
    uint64_t step, int N, int nchunks, int G, Ws ws, int32_t* __restrict__ n_accept,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ status) {
  constexpr int CH = EPT * kThreads;
  // A 1-D grid of B * G workgroups. The first B are workgroup 0 of each sequence (the one
  // that writes a rejected or sampled sequence's result), dispatched before any other; the
  // rest go chunk-fastest, so that consecutive workgroups (which the hardware deals to
  // different XCDs) share a sequence.
  const int B = gridDim.x / G, L = blockIdx.x;
  const int Gm = G > 1 ? G - 1 : 1;  // (with G = 1 every workgroup is a first one)
  const int b = L < B ? L : (L - B) / Gm;
  const int g = L < B ? 0 : 1 + (L - B) % Gm;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ uint64_t wsum[kThreads / 64], wsum2[kThreads / 64];
  __shared__ uint64_t sh_z[2];
  __shared__ int sh_f[kThreads / 64];
  __shared__ int sh_chunk;
  __shared__ uint64_t sh_tau;
  __shared__ int sh_tok;
  __shared__ int32_t cand[kTopK];
  __shared__ float candq[kTopK];
  __shared__ int corr_off[kTopK];      // chunk offset of a candidate's first occurrence, or -1
  __shared__ uint64_t corr_w[kTopK];   // its residual weight
  __shared__ int32_t allc[kMaxN * kTopK];
  __shared__ float allq[kMaxN * kTopK];
  __shared__ int32_t dtok[kMaxN];
  __shared__ uint64_t red[kThreads / 64][kRowsPerPass];
  __shared__ uint64_t rowacc[kRowWords];
  __shared__ uint64_t sh_row0;
  __shared__ int sh_last;

  // One memory round trip: the temperature, the proposals, the status word the selector
  // left (so that the final update is a plain store), row 0's chunk maxima (wave 0, up to
  // 128 chunks: lane l takes chunks l and l + 64), and for workgroup 0 of an f32 target a
  // sampled sequence's chain record, this thread's chunk sums (chunks t*cpt .. t*cpt + cpt
  // - 1, kept in registers for up to kCptMax chunks) and every slot's candidates. The
  // workspace holds all of these for either target type; a sequence ignores what its
  // mode does not use.
  const float T = temperature[b];
  const int32_t my_tok = tokens[(int64_t)b * N + (t < N ? t : 0)];
  const int32_t st_in = t == 0 ? status[b] : 0;
  const bool few = nchunks <= 128;
  uint64_t pre0[2] = {0ull, 0ull};
  if (few && w == 0) {
    const uint64_t* src = ws.best0 + (int64_t)b * nchunks;
#pragma unroll
    for (int i = 0; i < 2; ++i) pre0[i] = src[min(lane + 64 * i, nchunks - 1)];
  }
  constexpr bool kIsF32 = sizeof(typename KT::elem_t) == 4;
  constexpr int kCptMax = 4;
  const int cpt = (nchunks + kThreads - 1) / kThreads;
  ChainRec rec_pre = {0, 1, 0, 0, 0};
  uint64_t zr_pre[kCptMax], zp_pre[kCptMax];
  int zf_pre[kCptMax];
  int32_t ci_pre = -1;
  float q_pre = 0.0f;
  if constexpr (kIsF32) {
    if (g == 0) {
      rec_pre = ws.chain[b];
#pragma unroll
      for (int i = 0; i < kCptMax; ++i) {
        const int c = min(t * cpt + i, nchunks - 1);
        zr_pre[i] = ws.zsum[((int64_t)b * nchunks + c) * 2 + 0];
        zp_pre[i] = ws.zsum[((int64_t)b * nchunks + c) * 2 + 1];
        zf_pre[i] = ws.zflag[(int64_t)b * nchunks + c];
      }
      if (t < N * kTopK) {
        ci_pre = cidx[(int64_t)b * N * kTopK + t];
        q_pre = q[(int64_t)b * N * kTopK + t];
      }
    }
  }
  int st = 0;
  float invT = 0.0f;
  int mode = temp_mode(T, &invT, &st);
  if (mode == 1 && !kIsF32) {
    st |= DFLASH2_ST_BADPROB;
    mode = 0;
  }
  const int32_t* d = tokens + (int64_t)b * N;
  int32_t* out = out_tokens + (int64_t)b * (N + 1);
  const typename KT::elem_t* tb = target + (int64_t)b * seq_stride;

  if (mode == 0) {
    // row 0's first element
    if (w == 0) {
      uint64_t m = 0;
      if (few) {
        m = lane < nchunks ? pre0[0] : 0ull;
        if (lane + 64 < nchunks) m = pre0[1] > m ? pre0[1] : m;
        m = wave_max_u64_all(m, lane);  // every lane of wave 0 is active here
      } else {
        const uint64_t* src = ws.best0 + (int64_t)b * nchunks;
        for (int c = lane; c < nchunks; c += 64) m = src[c] > m ? src[c] : m;
        m = wave_max_u64(m);
      }
      if (lane == 0) sh_row0 = m;
    }
    if (t < N) dtok[t] = my_tok;
    if (t < kRowWords) rowacc[t] = 0ull;
    __syncthreads();
    const uint64_t r0 = sh_row0;
    if (dtok[0] != (int32_t)cand_idx(r0)) {
      // proposal 1 is rejected: the chain ends at row 0
      if (g == 0 && t == 0) {
        if (cand_key(r0) == KT::kNaN) st |= DFLASH2_ST_NONFINITE;
        out[0] = (int32_t)cand_idx(r0);
        for (int j = 1; j <= N; ++j) out[j] = -1;
        n_accept[b] = 0;
        status[b] = st_in | st;
      }
      return;
    }
    // Proposal 1 is accepted: this workgroup's chunks g, g + G, ... of rows 1..N, with
    // the loads of up to kRowsPerPass rows in flight together (rows past N re-read row N,
    // ignored, so that the loads carry no conditions).
    for (int c = g; c < nchunks; c += G) {
      const int base = c * CH;
      const bool full = VEC && base + CH <= V;
      for (int rp = 1; rp <= N; rp += kRowsPerPass) {
        uint32_t bits[kRowsPerPass][EPT];
        if (full) {
#pragma unroll
          for (int rr = 0; rr < kRowsPerPass; ++rr)
            load_chunk_full<KT, EPT>(tb + (int64_t)min(rp + rr, N) * row_stride, base, bits[rr]);
        } else {
#pragma unroll
          for (int rr = 0; rr < kRowsPerPass; ++rr)
            load_chunk<KT, EPT, VEC>(tb + (int64_t)min(rp + rr, N) * row_stride, base, V,
                                     bits[rr]);
        }
#pragma unroll
        for (int rr = 0; rr < kRowsPerPass; ++rr) {
          uint64_t m = 0;
          if (rp + rr <= N)
            m = full ? chunk_best_full<KT, EPT>(bits[rr], base, V)
                     : chunk_best_exact<KT, EPT, VEC>(bits[rr], base, V);
          if (lane == 0) red[w][rr] = m;
        }
        __syncthreads();
        if (t < kRowsPerPass && rp + t <= N) {
          uint64_t x = rowacc[rp + t];
          for (int i = 0; i < kThreads / 64; ++i) x = red[i][t] > x ? red[i][t] : x;
          rowacc[rp + t] = x;
        }
        __syncthreads();
      }
    }
    // Publish: one atomic maximum per row, performed before this workgroup arrives.
    if (t >= 1 && t <= N) max_agent(ws.rowmax + (int64_t)b * kRowWords + t, rowacc[t]);
    wait_vm();
    __syncthreads();
    if (t == 0) sh_last = add_agent(ws.arrive + b, 1u) == (uint32_t)(G - 1);
    __syncthreads();
    if (!sh_last) return;
    // The last workgroup: every other one's maxima were performed before its arrival.
    if (t >= 1 && t <= N) rowacc[t] = load_agent(ws.rowmax + (int64_t)b * kRowWords + t);
    __syncthreads();
    if (t == 0) {
      int n = 1;  // proposal 1, checked above
      int32_t emitted = -1;
      if (cand_key(r0) == KT::kNaN) st |= DFLASH2_ST_NONFINITE;
      for (int j = 2; j <= N + 1; ++j) {
        const uint64_t m = rowacc[j - 1];
        const int32_t y = (int32_t)cand_idx(m);
        if (cand_key(m) == KT::kNaN) st |= DFLASH2_ST_NONFINITE;
        if (j <= N && dtok[j - 1] == y) {
          ++n;
          continue;
        }
        emitted = y;
        break;
      }
      for (int j = 0; j <= N; ++j) out[j] = j < n ? dtok[j] : (j == n ? emitted : -1);
      n_accept[b] = n;
      status[b] = st_in | st;
    }
    return;
  }
  if (g != 0) return;

  // sampled
  const ChainRec rec = rec_pre;
  st |= rec.flags;
  const float* row = reinterpret_cast<const float*>(tb) + (int64_t)(rec.pos - 1) * row_stride;
  if (t < N * kTopK) {
    allc[t] = ci_pre;
    allq[t] = q_pre;
  }
  // thread t owns chunks t*cpt .. t*cpt + cpt - 1 (in index order), so a workgroup scan of
  // the per-thread sums finds the chunk that holds the draw
  uint64_t my_zr = 0, my_zp = 0;
  {
    int f = 0;
    if (cpt <= kCptMax) {
#pragma unroll
      for (int i = 0; i < kCptMax; ++i) {
        if (i < cpt && t * cpt + i < nchunks) {
          my_zr += zr_pre[i];
          my_zp += zp_pre[i];
          f |= zf_pre[i];
        }
      }
    } else {
      for (int i = 0; i < cpt; ++i) {
        const int c = t * cpt + i;
        if (c < nchunks) {
          my_zr += ws.zsum[((int64_t)b * nchunks + c) * 2 + 0];
          my_zp += ws.zsum[((int64_t)b * nchunks + c) * 2 + 1];
          f |= ws.zflag[(int64_t)b * nchunks + c];
        }
      }
    }
    const uint64_t zr = wave_sum_u64(my_zr);
    const uint64_t zp = wave_sum_u64(my_zp);
    f = wave_or(f);
    if (lane == 0) {
      wsum[w] = zr;
      wsum2[w] = zp;
      sh_f[w] = f;
    }
    __syncthreads();
    if (t == 0) {
      uint64_t a = 0, c2 = 0;
      int ff = 0;
      for (int i = 0; i < kThreads / 64; ++i) {
        a += wsum[i];
        c2 += wsum2[i];
        ff |= sh_f[i];
      }
      sh_z[0] = a;
      sh_z[1] = c2;
      sh_f[0] = ff;
    }
    __syncthreads();
  }
  st |= sh_f[0];
  int use_resid = rec.resid;
  uint64_t Z = use_resid ? sh_z[0] : sh_z[1];
  if (Z == 0 && use_resid) {
    use_resid = 0;
    Z = sh_z[1];
  }
  if (t < kTopK) {
    // the barriers above ordered the allc/allq writes before these reads
    if (use_resid) {
      cand[t] = allc[(rec.pos - 1) * kTopK + t];
      candq[t] = allq[(rec.pos - 1) * kTopK + t];
    } else {
      cand[t] = -1;
      candq[t] = 0.0f;
    }
  }
  int32_t emitted = -1;
  if (Z == 0) {
    // no mass at all: the row's first element under the top-16 order
    st |= DFLASH2_ST_ZEROMASS;
    uint32_t bk = 0, bi = 0;
    for (int x = t; x < V; x += kThreads) {
      const uint32_t k = KeyF32::canon(__float_as_uint(row[x]));
      if (k > bk) {
        bk = k;
        bi = (uint32_t)x;
      }
    }
    uint64_t m = bk ? pack_cand(bk, bi) : 0ull;
    m = wave_max_u64(m);
    if (lane == 0) wsum[w] = m;
    __syncthreads();
    if (t == 0) {
      uint64_t g = wsum[0];
      for (int i = 1; i < kThreads / 64; ++i) g = wsum[i] > g ? wsum[i] : g;
      sh_tok = (int)cand_idx(g);
    }
    __syncthreads();
    emitted = sh_tok;
  } else {
    // every thread takes the same tau (kernel 1 made the draw); the scan of the per-thread
    // sums finds the chunk
    const uint64_t tau_all = scale_draw(rec.draw, Z);
    if (t == 0) sh_tok = -1;
    const uint64_t mine_z = use_resid ? my_zr : my_zp;
    const uint64_t incl_z = block_incl_scan_u64(mine_z, wsum);
    const uint64_t excl_z = incl_z - mine_z;
    if (excl_z <= tau_all && tau_all < incl_z) {
      uint64_t cum = excl_z;
      int c = t * cpt;
      if (cpt <= kCptMax) {
#pragma unroll
        for (int i = 0; i < kCptMax; ++i) {
          if (i >= cpt || c >= nchunks) break;
          const uint64_t zc = use_resid ? zr_pre[i] : zp_pre[i];
          if (cum + zc > tau_all) break;
          cum += zc;
          ++c;
        }
      } else {
        for (int i = 0; i < cpt && c < nchunks; ++i, ++c) {
          const uint64_t zc = ws.zsum[((int64_t)b * nchunks + c) * 2 + (use_resid ? 0 : 1)];
          if (cum + zc > tau_all) break;
          cum += zc;
        }
      }
      sh_chunk = c;
      sh_tau = tau_all - cum;
    }
    __syncthreads();
    // scan the chosen chunk in index order: thread t owns EPT consecutive elements
    const int cbase = sh_chunk * CH;
    const int c0 = cbase + t * EPT;
    uint64_t wgt[EPT];
    uint64_t mine = 0;
    int dummy = 0;
    float pv[EPT];
    if (VEC && cbase + CH <= V) {
      const float4* p4 = reinterpret_cast<const float4*>(row + c0);
      const float4 a = p4[0], z = p4[1];
      pv[0] = a.x; pv[1] = a.y; pv[2] = a.z; pv[3] = a.w;
      pv[4] = z.x; pv[5] = z.y; pv[6] = z.z; pv[7] = z.w;
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) pv[e] = c0 + e < V ? row[c0 + e] : 0.0f;
    }
    // A candidate index takes the residual weight instead, and for a repeated index its
    // first occurrence counts: thread k < 16 finds whether candidate k is the first
    // occurrence of an index inside this chunk and gathers that element with the chunk.
    int32_t ck = -1;
    float pk = 0.0f, qk = 0.0f;
    bool has = false;
    if (t < kTopK) {
      ck = cand[t];
      qk = candq[t];
      has = ck >= cbase && ck < cbase + CH && ck < V;  // (cbase >= 0; unused slots hold -1)
#pragma unroll
      for (int j = 0; j < kTopK; ++j)
        if (j < t) has = has && cand[j] != ck;
      if (has) pk = row[ck];
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      wgt[e] = c0 + e < V ? quant40(prob_ok(pv[e], &dummy)) : 0ull;
    if (t < kTopK) {
      uint64_t wk = 0;
      if (has) {
        const float df = __fsub_rn(prob_ok(pk, &dummy), prob_ok(qk, &dummy));
        wk = quant40(df > 0.0f ? df : 0.0f);
      }
      corr_off[t] = has ? ck - cbase : -1;
      corr_w[t] = wk;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      const int dd = corr_off[k] - t * EPT;
      if ((unsigned)dd < (unsigned)EPT) {
        const uint64_t wk = corr_w[k];
#pragma unroll
        for (int e = 0; e < EPT; ++e)
          if (e == dd) wgt[e] = wk;
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) mine += wgt[e];
    const uint64_t incl = block_incl_scan_u64(mine, wsum);
    const uint64_t excl = incl - mine;
    const uint64_t tau = sh_tau;
    if (excl <= tau && tau < incl) {
      uint64_t run = excl;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        run += wgt[e];
        if (run > tau) {
          sh_tok = c0 + e;
          break;
        }
      }
    }
    __syncthreads();
    emitted = sh_tok;
  }
  if (t == 0) {
    const int n = rec.n_acc;
    for (int j = 0; j <= N; ++j) out[j] = j < n ? d[j] : (j == n ? emitted : -1);
    n_accept[b] = n;
    status[b] = st_in | st;
  }
}

constexpr int kEPT = 8;  // elements per thread: one 16-byte bf16 vector or two f32 vectors

struct Plan {
  int nchunks;
  bool vec;
  int G;    // kernel-2 workgroups per sequence
  int cpw;  // kernel-1 chunks per workgroup
};

// Kernel-1 chunks per workgroup (1, 2 or 4): a chunk is 8 KB of an f32 row, and a sampled
// workgroup spends its chain's dependent round trips before its row loads, so larger
// grids take two chunks per workgroup. Measured at batch 64 (7,808 chunks, cold rows):
// kernel 1 alone 18.3 us with one chunk per workgroup, 16.5 with two, 18.5 with four; at
// batch 1 one chunk is fastest. DF2_VERIFY_CPW fixes the value; 0 chooses by grid size.
#ifndef DF2_VERIFY_CPW
#define DF2_VERIFY_CPW 0
#endif

// Kernel 2 workgroups per sequence: one per chunk by default (0), so that even a single
// accepted greedy chain streams rows 1..N over the whole chip in one or two round trips;
// a positive value aims at that many workgroups in all instead. Measured at batch 64 (32
// greedy sequences, 2 accepting proposal 1): one per chunk 32.0 us per call, about 4096 in
// all 34.7, about 2048 in all 41.4, about 1024 in all 50.6 (the accepted chains then
// stream their rows in eight latency-bound rounds).
#ifndef DF2_VERIFY_FINISH_WGS
#define DF2_VERIFY_FINISH_WGS 0
#endif
constexpr int kFinishTargetWGs = DF2_VERIFY_FINISH_WGS;  // 0: one workgroup per chunk

Plan make_plan(int B, int V, int dtype, const void* target, int64_t ss, int64_t rs) {
  Plan p;
  p.nchunks = (V + kEPT * kThreads - 1) / (kEPT * kThreads);
  p.G = kFinishTargetWGs ? std::max(1, std::min(p.nchunks, kFinishTargetWGs / B)) : p.nchunks;
  p.G = (int)std::min<int64_t>(p.G, INT32_MAX / B);  // the 1-D grid of B * G workgroups
  const int64_t wgs = (int64_t)B * p.nchunks;
  p.cpw = DF2_VERIFY_CPW ? DF2_VERIFY_CPW : (wgs >= 1024 ? 2 : 1);
  const int esz = dtype == DFLASH2_BF16 ? 2 : 4;
  p.vec = (target == nullptr || aligned(target, 16)) && (ss * esz) % 16 == 0 && (rs * esz) % 16 == 0;
  return p;
}

template <class KT, bool VEC>
void launch(const Plan& p, const void* target, int64_t ss, int64_t rs, int V,
            const int32_t* tokens, const int32_t* cidx, const float* q, const int32_t* slot,
            const float* temp, uint64_t seed, uint64_t step, int B, int N, Ws w, int32_t* n_acc,
            int32_t* out, int32_t* status, hipStream_t st) {
  using E = typename KT::elem_t;
  const dim3 g1((p.nchunks + p.cpw - 1) / p.cpw, B);
  if (p.cpw >= 4)
    verify_rows_kernel<KT, kEPT, VEC, 4><<<g1, kThreads, 0, st>>>(
        (const E*)target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, N, p.nchunks, w);
  else if (p.cpw == 2)
    verify_rows_kernel<KT, kEPT, VEC, 2><<<g1, kThreads, 0, st>>>(
        (const E*)target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, N, p.nchunks, w);
  else
    verify_rows_kernel<KT, kEPT, VEC, 1><<<g1, kThreads, 0, st>>>(
        (const E*)target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, N, p.nchunks, w);
  verify_finish_kernel<KT, kEPT, VEC><<<dim3(B * p.G), kThreads, 0, st>>>(
      (const E*)target, ss, rs, V, tokens, cidx, q, temp, seed, step, N, p.nchunks, p.G, w, n_acc,
      out, status);
}

template <class KT>
void launch_vec(const Plan& p, const void* target, int64_t ss, int64_t rs, int V,
                const int32_t* tokens, const int32_t* cidx, const float* q, const int32_t* slot,
                const float* temp, uint64_t seed, uint64_t step, int B, int N, Ws w,
                int32_t* n_acc, int32_t* out, int32_t* status, hipStream_t st) {
  if (p.vec)
    launch<KT, true>(p, target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, B, N, w, n_acc, out, status, st);
  else
    launch<KT, false>(p, target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, B, N, w, n_acc, out, status, st);
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" size_t dflash2_verify_workspace_bytes(int B, int N, int V, int dtype) {
  if (B < 1 || N < 1 || N > kMaxN || V < kTopK) return 0;
  Plan p = make_plan(B, V, dtype, nullptr, 0, 0);
  return ws_layout(B, p.nchunks, nullptr, nullptr);
}

extern "C" int dflash2_verify(const void* target, int dtype, int64_t seq_stride, int64_t row_stride,
                              int V, const int32_t* tokens, const int32_t* cand_idx, const float* q,
                              const int32_t* slot, const float* temperature, uint64_t seed,
                              uint64_t step, int B, int N, int32_t* n_accept, int32_t* out_tokens,
                              int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!target || !tokens || !cand_idx || !q || !slot || !temperature || !n_accept ||
      !out_tokens || !status || !ws)
    return DFLASH2_EINVAL;
  if (B < 1 || N < 1 || V < kTopK || seq_stride < 0 || row_stride < 0) return DFLASH2_EINVAL;
  if (N > kMaxN || B > 65535) return DFLASH2_EUNSUPPORTED;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_F32) return DFLASH2_EUNSUPPORTED;
  if (!aligned(ws, kWsAlign) || ws_bytes < dflash2_verify_workspace_bytes(B, N, V, dtype))
    return DFLASH2_EWORKSPACE;
  Plan p = make_plan(B, V, dtype, target, seq_stride, row_stride);
  Ws w;
  ws_layout(B, p.nchunks, &w, (char*)ws);
  if (dtype == DFLASH2_BF16)
    launch_vec<KeyBF16>(p, target, seq_stride, row_stride, V, tokens, cand_idx, q, slot,
                        temperature, seed, step, B, N, w, n_accept, out_tokens, status, stream);
  else
    launch_vec<KeyF32>(p, target, seq_stride, row_stride, V, tokens, cand_idx, q, slot,
                       temperature, seed, step, B, N, w, n_accept, out_tokens, status, stream);
  return launch_status();
}
