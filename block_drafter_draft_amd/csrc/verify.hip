// dflash2_verify: target verification of the N proposals ("Geramy/LSE docs/DFLASH2.md",
// usage paragraph: probability-ratio rejection with residual sampling over all seven
// proposals, greedy keeps the deterministic chain; drafter-geometry paragraph: the target
// consumes the anchor plus all proposals, so an all-accept step has a bonus row).
//
// Kernel 1 (grid: chunks x row groups x sequences) reads each needed target row chunk once:
//   greedy  - rows 0..N: the chunk's first element under the top-16 order (packed word),
//             a group of rows per workgroup;
//   sampled - the accept chain is cheap (N gathers and N Philox draws, one per lane), so
//             every workgroup of the sequence recomputes it and then reads only the row it
//             will draw from: the chunk sums of the integer weights floor(w * 2^40), both
//             for p_t itself and with the 16 candidates' residual max(0, p_t - q) swapped in.
// Kernel 2 (one workgroup per sequence) runs the greedy chain on the row maxima, or picks
// the chunk holding the draw from the chunk sums and scans that one chunk in index order.
// Integer weights make the draw independent of the summation order, so it is bit-exact.
#include "common.hpp"

namespace df2 {
namespace {

constexpr int kThreads = kChunkThreads;
constexpr int kMaxN = 15;

struct ChainRec {
  int32_t n_acc;   // accepted proposals
  int32_t pos;     // block position of the drawn token (1..N+1)
  int32_t resid;   // 1: draw from the residual of slot pos; 0: from p_t itself
  int32_t flags;   // status bits from the accept tests
};

struct Ws {
  ChainRec* chain;   // [B]
  uint64_t* best;    // [B][N+1][nchunks] greedy chunk maxima
  uint64_t* zsum;    // [B][nchunks][2] sampled chunk sums (residual, plain)
  int32_t* zflag;    // [B][nchunks] status bits seen in the chunk
};

__host__ __device__ inline size_t ws_layout(int B, int N, int nchunks, Ws* w, char* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = (off + bytes + 255) / 256 * 256;
    return o;
  };
  size_t o_chain = take(sizeof(ChainRec) * B);
  size_t o_best = take(sizeof(uint64_t) * (size_t)B * (N + 1) * nchunks);
  size_t o_z = take(sizeof(uint64_t) * 2 * (size_t)B * nchunks);
  size_t o_f = take(sizeof(int32_t) * (size_t)B * nchunks);
  if (w && base) {
    w->chain = (ChainRec*)(base + o_chain);
    w->best = (uint64_t*)(base + o_best);
    w->zsum = (uint64_t*)(base + o_z);
    w->zflag = (int32_t*)(base + o_f);
  }
  return off;
}

template <class KT>
__device__ __forceinline__ uint32_t load_bits(const typename KT::elem_t* p, int64_t i) {
  if constexpr (sizeof(typename KT::elem_t) == 2)
    return reinterpret_cast<const uint16_t*>(p)[i];
  else
    return __float_as_uint(reinterpret_cast<const float*>(p)[i]);
}

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
    if (t < N) {
      const int j = t + 1;
      // the target gather goes out first (at a clamped, always valid index)
      const int xc = x < 0 ? 0 : (x >= V ? V - 1 : x);
      const float pt_raw = tgt[(int64_t)t * row_stride + xc];
      Draw d = philox_draw(seed, step, (uint32_t)b, (uint32_t)j);
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
    if (t == 0) {
      rec->n_acc = first;
      rec->pos = first + 1;
      rec->resid = (first < N && !plain_first) ? 1 : 0;
      rec->flags = flags;
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

// Grid: (chunks, row groups, sequences). A greedy sequence's workgroup takes RG rows of
// one chunk; a sampled sequence uses row group 0 only.
template <class KT, int EPT, bool VEC, int RG>
__global__ __launch_bounds__(kThreads) void verify_rows_kernel(
    const typename KT::elem_t* __restrict__ target, int64_t seq_stride, int64_t row_stride, int V,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cidx,
    const float* __restrict__ q, const int32_t* __restrict__ slot,
    const float* __restrict__ temperature, uint64_t seed, uint64_t step, int N, int nchunks,
    Ws ws) {
  constexpr int CH = EPT * kThreads;
  const int chunk = blockIdx.x, grp = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int base = chunk * CH;
  __shared__ ChainRec rec;
  __shared__ uint64_t red[kThreads / 64][RG < 2 ? 2 : RG];  // the sampled path uses two
  __shared__ int redf[kThreads / 64];

  // a sampled chain's first loads do not depend on the temperature: issue them with it
  // (the proposals and slots, and on an f32 target every slot's candidates and q)
  __shared__ int32_t allc[kMaxN * kTopK];
  __shared__ float allq[kMaxN * kTopK];
  // (only row group 0 can need them: a sampled sequence uses no other group)
  int32_t x_pre = -1, sl_pre = -1;
  if (grp == 0 && t < N) {
    x_pre = tokens[(int64_t)b * N + t];
    sl_pre = slot[(int64_t)b * N + t];
  }
  int32_t ci_pre = -1;
  float q_pre = 0.0f;
  if (sizeof(typename KT::elem_t) == 4 && grp == 0 && t < N * kTopK) {
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
    // greedy: the chunk's first element of rows r0 .. r0 + RG - 1, all loads issued together
    const int r0 = grp * RG;
    if (r0 > N) return;
    uint32_t bits[RG][EPT];
    const bool full = VEC && base + CH <= V;
    // rows past N re-read row N (ignored below), so the loads carry no conditions
    if (full) {
#pragma unroll
      for (int rr = 0; rr < RG; ++rr) {
        const int r = r0 + rr <= N ? r0 + rr : N;
        load_chunk_full<KT, EPT>(tb + (int64_t)r * row_stride, base, bits[rr]);
      }
    } else {
#pragma unroll
      for (int rr = 0; rr < RG; ++rr) {
        const int r = r0 + rr <= N ? r0 + rr : N;
        load_chunk<KT, EPT, VEC>(tb + (int64_t)r * row_stride, base, V, bits[rr]);
      }
    }
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) {
      uint64_t m = 0;
      if (r0 + rr <= N)
        m = full ? chunk_best_full<KT, EPT>(bits[rr], base, V)
                 : chunk_best_exact<KT, EPT, VEC>(bits[rr], base, V);
      if ((t & 63) == 0) red[t >> 6][rr] = m;
    }
    __syncthreads();
    if (t < RG && r0 + t <= N) {
      uint64_t g = red[0][t];
      for (int w = 1; w < kThreads / 64; ++w) g = red[w][t] > g ? red[w][t] : g;
      ws.best[((int64_t)b * (N + 1) + r0 + t) * nchunks + chunk] = g;
    }
    return;
  }
  if (grp != 0) return;

  // sampled: which row, and with which candidate corrections
  const float* tgt = reinterpret_cast<const float*>(tb);
  if (t < N * kTopK) {
    allc[t] = ci_pre;
    allq[t] = q_pre;
  }
  accept_chain(tgt, row_stride, V, N, x_pre, sl_pre, allc, allq, seed, step, b, &rec);
  if (chunk == 0 && t == 0) ws.chain[b] = rec;
  const float* row = tgt + (int64_t)(rec.pos - 1) * row_stride;

  uint32_t bits[EPT];
  if (VEC && base + CH <= V)
    load_chunk_full<KT, EPT>(reinterpret_cast<const typename KT::elem_t*>(row), base, bits);
  else
    load_chunk<KT, EPT, VEC>(reinterpret_cast<const typename KT::elem_t*>(row), base, V, bits);
  // residual corrections for the candidates of slot pos that fall in this chunk; for a
  // repeated index only its first occurrence counts. Their gathers go out with the chunk.
  bool corr = false;
  float p_c = 0.0f, q_c = 0.0f;
  if (rec.resid && t < kTopK) {
    const int32_t* ci = allc + (rec.pos - 1) * kTopK;
    const int32_t c = ci[t];
    bool first = c >= 0 && c < V;
#pragma unroll
    for (int k = 0; k < kTopK; ++k)
      if (k < t) first = first && ci[k] != c;
    if (first && c >= base && c < base + CH) {
      corr = true;
      p_c = row[c];
      q_c = allq[(rec.pos - 1) * kTopK + t];
    }
  }
  uint64_t zp = 0;
  int fl = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int x = index_of<EPT, VEC, KT>(base, e);
    if (x < V) zp += quant40(prob_ok(__uint_as_float(bits[e]), &fl));
  }
  int64_t dz = 0;
  if (corr) {
    int dummy = 0;
    const float p = prob_ok(p_c, &dummy);
    const float qk = prob_ok(q_c, &fl);
    const float d = __fsub_rn(p, qk);
    dz = (int64_t)quant40(d > 0.0f ? d : 0.0f) - (int64_t)quant40(p);
  }
  uint64_t zr = zp + (uint64_t)dz;
  zp = wave_sum_u64_all(zp, t & 63);  // every lane is active here
  zr = wave_sum_u64_all(zr, t & 63);
  fl = wave_or(fl);
  if ((t & 63) == 0) {
    red[t >> 6][0] = zr;
    red[t >> 6][1] = zp;
    redf[t >> 6] = fl;
  }
  __syncthreads();
  if (t == 0) {
    uint64_t a = 0, c = 0;
    int f = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      a += red[w][0];
      c += red[w][1];
      f |= redf[w];
    }
    ws.zsum[((int64_t)b * nchunks + chunk) * 2 + 0] = a;
    ws.zsum[((int64_t)b * nchunks + chunk) * 2 + 1] = c;
    ws.zflag[(int64_t)b * nchunks + chunk] = f;
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

template <class KT, int EPT>
__global__ __launch_bounds__(kThreads) void verify_finish_kernel(
    const typename KT::elem_t* __restrict__ target, int64_t seq_stride, int64_t row_stride, int V,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ cidx,
    const float* __restrict__ q, const float* __restrict__ temperature, uint64_t seed,
    uint64_t step, int N, int nchunks, Ws ws, int32_t* __restrict__ n_accept,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ status) {
  constexpr int CH = EPT * kThreads;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ uint64_t rowbest[kMaxN + 1];
  __shared__ uint64_t wsum[kThreads / 64], wsum2[kThreads / 64];
  __shared__ uint64_t sh_z[2];
  __shared__ int sh_f[kThreads / 64];
  __shared__ int sh_chunk;
  __shared__ uint64_t sh_tau;
  __shared__ int sh_tok;
  __shared__ int32_t cand[kTopK];
  __shared__ float candq[kTopK];
  __shared__ int32_t allc[kMaxN * kTopK];
  __shared__ float allq[kMaxN * kTopK];

  // The greedy chain's chunk maxima are loaded before the temperature is known (for up to
  // 128 chunks: wave w takes rows w, w + 4, ..., lane l chunks l and l + 64), so that the
  // two loads are one memory round trip; a sampled sequence ignores them.
  constexpr int kRowIt = (kMaxN + 1 + kThreads / 64 - 1) / (kThreads / 64);
  uint64_t pre[kRowIt][2];
  __shared__ int32_t dtok[kMaxN];
  const int32_t my_tok = tokens[(int64_t)b * N + (t < N ? t : 0)];  // the proposals, with them
  // the status word the selector left, read now so that the final update is a plain store
  const int32_t st_in = t == 0 ? status[b] : 0;
  const bool few = nchunks <= 128;
  if (few) {
#pragma unroll
    for (int j = 0; j < kRowIt; ++j) {
      const int r = min(w + (kThreads / 64) * j, N);
      const uint64_t* src = ws.best + ((int64_t)b * (N + 1) + r) * nchunks;
#pragma unroll
      for (int i = 0; i < 2; ++i) pre[j][i] = src[min(lane + 64 * i, nchunks - 1)];
    }
  }
  constexpr bool kIsF32 = sizeof(typename KT::elem_t) == 4;
  // A sampled sequence's inputs do not depend on the temperature either: the chain record,
  // this thread's chunk sums (chunks t*cpt .. t*cpt + cpt - 1, kept in registers for up to
  // kCptMax chunks) and every slot's candidates, loaded in the same round trip. The
  // workspace holds these arrays for either target type; a greedy sequence ignores them.
  constexpr int kCptMax = 4;
  const int cpt = (nchunks + kThreads - 1) / kThreads;
  ChainRec rec_pre = {0, 1, 0, 0};
  uint64_t zr_pre[kCptMax], zp_pre[kCptMax];
  int zf_pre[kCptMax];
  int32_t ci_pre = -1;
  float q_pre = 0.0f;
  if constexpr (kIsF32) {
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
  int st = 0;
  float invT = 0.0f;
  int mode = temp_mode(temperature[b], &invT, &st);
  if (mode == 1 && !kIsF32) {
    st |= DFLASH2_ST_BADPROB;
    mode = 0;
  }
  const int32_t* d = tokens + (int64_t)b * N;
  int32_t* out = out_tokens + (int64_t)b * (N + 1);
  const typename KT::elem_t* tb = target + (int64_t)b * seq_stride;

  if (mode == 0) {
    if (few) {
#pragma unroll
      for (int j = 0; j < kRowIt; ++j) {
        const int r = w + (kThreads / 64) * j;
        uint64_t m = pre[j][0];
        if (lane + 64 < nchunks) m = pre[j][1] > m ? pre[j][1] : m;
        if (lane >= nchunks) m = 0;
        m = wave_max_u64_all(m, lane);  // every lane is active here
        if (lane == 0 && r <= N) rowbest[r] = m;
      }
    } else {
      for (int r = w; r <= N; r += kThreads / 64) {
        uint64_t m = 0;
        const uint64_t* src = ws.best + ((int64_t)b * (N + 1) + r) * nchunks;
        for (int c = lane; c < nchunks; c += 64) m = src[c] > m ? src[c] : m;
        m = wave_max_u64(m);
        if (lane == 0) rowbest[r] = m;
      }
    }
    if (t < N) dtok[t] = my_tok;
    __syncthreads();
    if (t == 0) {
      int n = 0;
      int32_t emitted = -1;
      for (int j = 1; j <= N + 1; ++j) {
        const uint64_t m = rowbest[j - 1];
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
    // every thread draws the same tau; the scan of the per-thread sums finds the chunk
    const Draw dr = philox_draw(seed, step, (uint32_t)b, (uint32_t)rec.pos);
    const uint64_t tau_all = scale_draw(dr.w[2], Z);
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
    const int c0 = sh_chunk * CH + t * EPT;
    uint64_t wgt[EPT];
    uint64_t mine = 0;
    int dummy = 0;
    float pv[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) pv[e] = c0 + e < V ? row[c0 + e] : 0.0f;
    int32_t ck[kTopK];
    float qk[kTopK];
#pragma unroll
    for (int k = 0; k < kTopK; ++k) {
      ck[k] = cand[k];
      qk[k] = candq[k];
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int x = c0 + e;
      uint64_t r = 0;
      if (x < V) {
        const float p = prob_ok(pv[e], &dummy);
        r = quant40(p);
        // a candidate index replaces the weight by the residual; for a repeated index
        // the first occurrence counts, so the candidates are applied last to first
#pragma unroll
        for (int k = kTopK - 1; k >= 0; --k) {
          if (ck[k] == x) {
            const float df = __fsub_rn(p, prob_ok(qk[k], &dummy));
            r = quant40(df > 0.0f ? df : 0.0f);
          }
        }
      }
      wgt[e] = r;
      mine += r;
    }
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
  int rg;  // rows per greedy workgroup: 1, 2 or 4 (8 with DF2_VERIFY_RG)
};

// Rows per greedy workgroup: four (measured best at batch 16 and 64: fewer registers than
// eight, so more workgroups in flight), fewer while the grid would have under about 1024
// workgroups (batch 1 takes one row per workgroup).
#ifndef DF2_VERIFY_RG
#define DF2_VERIFY_RG 0  // 0: by the batch
#endif
constexpr int kVerifyTargetWGs = 1024;

Plan make_plan(int B, int N, int V, int dtype, const void* target, int64_t ss, int64_t rs) {
  Plan p;
  p.nchunks = (V + kEPT * kThreads - 1) / (kEPT * kThreads);
  int rg = 4;
  while (rg > 1 && (int64_t)B * p.nchunks * ((N + 1 + rg - 1) / rg) < kVerifyTargetWGs) rg >>= 1;
  p.rg = DF2_VERIFY_RG ? DF2_VERIFY_RG : rg;
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
  const dim3 grid(p.nchunks, (N + 1 + p.rg - 1) / p.rg, B);
#define DF2_ROWS(RG)                                                                     \
  verify_rows_kernel<KT, kEPT, VEC, RG><<<grid, kThreads, 0, st>>>(                      \
      (const E*)target, ss, rs, V, tokens, cidx, q, slot, temp, seed, step, N, p.nchunks, w)
  switch (p.rg) {
    case 1: DF2_ROWS(1); break;
    case 2: DF2_ROWS(2); break;
    case 4: DF2_ROWS(4); break;
    default: DF2_ROWS(8); break;
  }
#undef DF2_ROWS
  verify_finish_kernel<KT, kEPT><<<B, kThreads, 0, st>>>((const E*)target, ss, rs, V, tokens, cidx,
                                                         q, temp, seed, step, N, p.nchunks, w,
                                                         n_acc, out, status);
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
  Plan p = make_plan(B, N, V, dtype, nullptr, 0, 0);
  return ws_layout(B, N, p.nchunks, nullptr, nullptr);
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
  Plan p = make_plan(B, N, V, dtype, target, seq_stride, row_stride);
  Ws w;
  ws_layout(B, N, p.nchunks, &w, (char*)ws);
  if (dtype == DFLASH2_BF16)
    launch_vec<KeyBF16>(p, target, seq_stride, row_stride, V, tokens, cand_idx, q, slot,
                        temperature, seed, step, B, N, w, n_accept, out_tokens, status, stream);
  else
    launch_vec<KeyF32>(p, target, seq_stride, row_stride, V, tokens, cand_idx, q, slot,
                       temperature, seed, step, B, N, w, n_accept, out_tokens, status, stream);
  return launch_status();
}
