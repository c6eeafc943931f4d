/*
 * dflash2_oracle.c - plain CPU oracle for the DFlash2 block-draft-and-verify step.
 *
 * TEST INFRASTRUCTURE ONLY. This is the slow, obviously-correct reference that the GPU
 * library is checked against. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it. It shares no source, header, table or helper with the HIP
 * library, and nothing on the product path may call it.
 *
 * Every function is single-threaded and written as the plain definition of what the step
 * computes: dense attention over an explicit visible-key list, a full sort for top-16, a
 * straight Viterbi recursion, a straight scan of the full vocabulary for sampling.
 *
 * The pages these definitions follow (cited by title and passage):
 *   [LSE]  "Geramy/LSE docs/DFLASH2.md": the drafter-geometry paragraph (block of eight,
 *          noncausal block, 2048-position window, two-tap conv, groups of 16, top-16,
 *          rank-256 selector), the native-test notes (attention and selector checks, the
 *          selector rounding bound) and the top-k policy paragraph (ties to the smaller
 *          index, NaNs first by index, infinities ordered normally).
 *   [PR625] "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625": the
 *          DFlash 2 commit message (two taps over the block, per-element base plus
 *          per-group dynamic coefficient; top-k, codebook gathers, path search).
 *   [VLLM] "[Spec Decode] DFlash2: local convolution + candidate selector - #52816": the
 *          PR description's two items (the conv formula; the selector edge score, best
 *          path from the verified anchor, inverse-CDF walk returning q for the lossless
 *          verify).
 *
 * Where the pages leave a step open, the reading taken is stated at the function.
 *
 * Arithmetic. Build with -O2 -ffp-contract=off and no fast-math. Attention and conv are
 * accumulated in binary64 (their results are compared within a tolerance). The selector
 * and the sampled verify decide integers (paths, accepts, tokens) from floating point, so
 * they run in binary32, the precision the pages give for activations and accumulation
 * ([LSE] conversion notes: floating activations and accumulation stay FP32), with every
 * operation rounded once, in the order written, and fmaf only where written.
 */
#define _GNU_SOURCE /* qsort_r */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BF16 0
#define OR_F32 1

#define OR_ST_NONFINITE 1
#define OR_ST_BADTOKEN 2
#define OR_ST_ZEROMASS 4
#define OR_ST_BADPROB 8
#define OR_ST_BADTEMP 16

#define OR_K 16 /* candidates per position: top-16 ([LSE] geometry paragraph) */

/* ------------------------------------------------------------------------------------ */
/* Element access                                                                        */
/* ------------------------------------------------------------------------------------ */

/* A bf16 value is the top half of a binary32; widening it is exact. */
static float or_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static float or_load(const void *p, int dtype, int64_t i) {
  if (dtype == OR_F32) return ((const float *)p)[i];
  return or_bf16_to_f32(((const uint16_t *)p)[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, */
/* 3", SC'11). The pages name no generator; the step needs a counter-based one so that   */
/* any (seed, sequence, position, step) draw can be recomputed independently.            */
/* ------------------------------------------------------------------------------------ */

static void or_mul64(uint64_t a, uint64_t b, uint64_t *hi, uint64_t *lo) {
  unsigned __int128 p = (unsigned __int128)a * (unsigned __int128)b;
  *hi = (uint64_t)(p >> 64);
  *lo = (uint64_t)p;
}

void or_philox4x64_10(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ULL, M1 = 0xCA5A826395121157ULL;
  const uint64_t W0 = 0x9E3779B97F4A7C15ULL, W1 = 0xBB67AE8584CAA73BULL;
  uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint64_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint64_t hi0, lo0, hi1, lo1;
    or_mul64(M0, c0, &hi0, &lo0);
    or_mul64(M1, c2, &hi1, &lo1);
    uint64_t n0 = hi1 ^ c1 ^ k0;
    uint64_t n1 = lo1;
    uint64_t n2 = hi0 ^ c3 ^ k1;
    uint64_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0; /* the key schedule advances by the Weyl constants between rounds */
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Draw layout (a reading: the uniforms need only be tied to the seed, the sequence and the
 * block position):
 * key = (seed, 0); counter = (step, b, j, 0). Word 0 is the selector-walk uniform for
 * slot j, word 1 the accept uniform for proposal j, word 2 the residual or bonus draw for
 * the token emitted at block position j; word 3 is unused. */
static void or_draw(uint64_t seed, uint64_t step, int b, int j, uint64_t w[4]) {
  uint64_t ctr[4] = {step, (uint64_t)b, (uint64_t)j, 0};
  uint64_t key[2] = {seed, 0};
  or_philox4x64_10(ctr, key, w);
}

/* u = top 24 bits / 2^24: exact in binary32, in [0, 1 - 2^-24]. */
static float or_uniform24(uint64_t w) { return (float)(w >> 40) * 0x1p-24f; }

/* ------------------------------------------------------------------------------------ */
/* exp_c: a binary32 exp for y <= 0, written from the mathematics so that two          */
/* independent implementations can agree bit for bit. exp(y) = 2^k * exp(r) with        */
/* k = round(y / ln 2), r = y - k ln 2 by two-constant (Cody-Waite) reduction, and       */
/* exp(r) by its degree-7 Taylor polynomial in Horner form. Results below e^-87 are     */
/* flushed to zero (they would be subnormal).                                            */
/* ------------------------------------------------------------------------------------ */

float or_exp_c(float y) {
  if (!(y >= -87.0f)) return 0.0f; /* also maps -inf (and NaN) to 0 */
  const float LOG2E = 1.44269502f;          /* fl(1/ln 2) */
  const float LN2_HI = 0.693145751953125f;  /* ln 2 with its low 8 significand bits cleared */
  const float LN2_LO = 1.42860677e-06f;     /* fl(ln 2 - LN2_HI) */
  float t = y * LOG2E;
  float k = rintf(t); /* round half to even (default rounding mode) */
  float r = fmaf(-k, LN2_HI, y);
  r = fmaf(-k, LN2_LO, r);
  /* 1/n! for n = 7..0, each rounded to binary32 */
  float p = 1.98412698e-04f;
  p = fmaf(p, r, 1.38888889e-03f);
  p = fmaf(p, r, 8.33333377e-03f);
  p = fmaf(p, r, 4.16666679e-02f);
  p = fmaf(p, r, 1.66666672e-01f);
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)k);
}

/* ------------------------------------------------------------------------------------ */
/* Block attention ([LSE] geometry paragraph; drafter width 5120, 32 query heads, 8 KV    */
/* heads, head dim 128).                                                                 */
/*                                                                                       */
/* Readings taken: slot i of sequence b sits at absolute position L_b + i (the anchor is */
/* the first position after the verified context). A context key at position j is       */
/* visible to slot i iff (L_b + i) - j < W (the usual per-query sliding window; the LSE */
/* test's live count 2055 = 2047 + 8 fits this). Context position j lives in ring row    */
/* j mod S. Every block key is visible to every slot (noncausal inside the block,        */
/* including later mask positions). Query head h reads KV head h / (Hq / Hkv). Inputs   */
/* are taken after RoPE; scale is supplied. Accumulated in binary64.                    */
/*                                                                                       */
/* q [B,P,Hq,D]; k_blk, v_blk [B,P,Hkv,D]; k_ring, v_ring [B,S,Hkv,D]; out [B,P,Hq,D].   */
/* ------------------------------------------------------------------------------------ */

void or_block_attn(const void *q, const void *k_blk, const void *v_blk, const void *k_ring,
                   const void *v_ring, const int32_t *ctx_len, double *out, int B, int P, int Hq,
                   int Hkv, int D, int S, int W, double scale, int dtype) {
  int group = Hq / Hkv;
  int max_keys = W + P;
  int64_t *key_row = (int64_t *)malloc(sizeof(int64_t) * (size_t)max_keys);
  int *key_is_blk = (int *)malloc(sizeof(int) * (size_t)max_keys);
  double *score = (double *)malloc(sizeof(double) * (size_t)max_keys);
  for (int b = 0; b < B; ++b) {
    int64_t L = ctx_len[b];
    for (int i = 0; i < P; ++i) {
      /* the visible key list for (b, i): context positions first, then the block */
      int n = 0;
      int64_t first = L + i - W + 1;
      if (first < 0) first = 0;
      for (int64_t j = first; j <= L - 1; ++j) {
        key_row[n] = j % S;
        key_is_blk[n] = 0;
        ++n;
      }
      for (int t = 0; t < P; ++t) {
        key_row[n] = t;
        key_is_blk[n] = 1;
        ++n;
      }
      for (int h = 0; h < Hq; ++h) {
        int g = h / group;
        int64_t qoff = (((int64_t)b * P + i) * Hq + h) * D;
        double mx = -INFINITY;
        for (int e = 0; e < n; ++e) {
          int64_t koff = key_is_blk[e] ? (((int64_t)b * P + key_row[e]) * Hkv + g) * D
                                       : (((int64_t)b * S + key_row[e]) * Hkv + g) * D;
          const void *kp = key_is_blk[e] ? k_blk : k_ring;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)or_load(q, dtype, qoff + d) * (double)or_load(kp, dtype, koff + d);
          score[e] = dot * scale;
          if (score[e] > mx) mx = score[e];
        }
        double denom = 0.0;
        for (int e = 0; e < n; ++e) {
          score[e] = exp(score[e] - mx);
          denom += score[e];
        }
        double *o = out + qoff;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int e = 0; e < n; ++e) {
          int64_t voff = key_is_blk[e] ? (((int64_t)b * P + key_row[e]) * Hkv + g) * D
                                       : (((int64_t)b * S + key_row[e]) * Hkv + g) * D;
          const void *vp = key_is_blk[e] ? v_blk : v_ring;
          double w = score[e] / denom;
          for (int d = 0; d < D; ++d) o[d] += w * (double)or_load(vp, dtype, voff + d);
        }
      }
    }
  }
  free(key_row);
  free(key_is_blk);
  free(score);
}

/* ------------------------------------------------------------------------------------ */
/* Dynamic two-tap convolution ([VLLM] PR description, first item; [PR625] DFlash 2      */
/* commit: two taps over the block, per-element base plus per-group dynamic coefficient).*/
/*   out[b,i,c] = sum_{t in {0,1}} (base[t,c] + delta[b,i,t,c/group]) * x[b,i-t,c]       */
/* with x[b,-1,c] = 0 (taps zero across the block boundary). Reading: tap 0 is the       */
/* current position, tap 1 its predecessor; groups are contiguous runs of `group`        */
/* channels; delta is supplied (its projection is outside the step). Binary64.           */
/*                                                                                       */
/* x [B,P,C]; base [2,C]; delta [B,P,2,C/group]; out [B,P,C].                            */
/* ------------------------------------------------------------------------------------ */

void or_dynconv2(const void *x, const float *base, const float *delta, double *out, int B, int P,
                 int C, int group, int dtype) {
  int G = C / group;
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < P; ++i)
      for (int c = 0; c < C; ++c) {
        double acc = 0.0;
        for (int t = 0; t < 2; ++t) {
          if (i - t < 0) continue; /* the block start has no predecessor */
          double w = (double)base[(int64_t)t * C + c] +
                     (double)delta[(((int64_t)b * P + i) * 2 + t) * G + c / group];
          acc += w * (double)or_load(x, dtype, ((int64_t)b * P + (i - t)) * C + c);
        }
        out[((int64_t)b * P + i) * C + c] = acc;
      }
}

/* ------------------------------------------------------------------------------------ */
/* Top-16 ([LSE] top-k policy paragraph). The order, first to last: every NaN (among     */
/* themselves by ascending index), then +inf, then finite values descending, then -inf; */
/* equal values by ascending index; -0 equals +0. The 16 first elements under this order */
/* are returned. Implemented as a full sort under that comparator.                       */
/* ------------------------------------------------------------------------------------ */

/* Returns 1 when (va, ia) comes before (vb, ib) in the order above. */
static int or_before(float va, int64_t ia, float vb, int64_t ib) {
  int na = isnan(va), nb = isnan(vb);
  if (na && nb) return ia < ib;
  if (na) return 1;
  if (nb) return 0;
  if (va > vb) return 1;
  if (va < vb) return 0;
  return ia < ib; /* equal values, including -0 == +0 and inf == inf */
}

typedef struct {
  const void *row;
  int dtype;
} or_sort_ctx;

static int or_cmp(const void *a, const void *b, void *arg) {
  const or_sort_ctx *c = (const or_sort_ctx *)arg;
  int32_t ia = *(const int32_t *)a, ib = *(const int32_t *)b;
  float va = or_load(c->row, c->dtype, ia), vb = or_load(c->row, c->dtype, ib);
  if (or_before(va, ia, vb, ib)) return -1;
  if (or_before(vb, ib, va, ia)) return 1;
  return 0;
}

/* Row r of sequence b starts at element b*seq_stride + (row0 + r)*row_stride.
 * idx/val are [B, N, 16]. */
void or_topk16(const void *scores, int dtype, int B, int N, int row0, int64_t seq_stride,
               int64_t row_stride, int V, int32_t *idx, float *val) {
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)V);
  for (int b = 0; b < B; ++b)
    for (int r = 0; r < N; ++r) {
      int64_t off = (int64_t)b * seq_stride + (int64_t)(row0 + r) * row_stride;
      const void *row = dtype == OR_F32 ? (const void *)((const float *)scores + off)
                                        : (const void *)((const uint16_t *)scores + off);
      or_sort_ctx ctx = {row, dtype};
      for (int v = 0; v < V; ++v) order[v] = v;
      qsort_r(order, (size_t)V, sizeof(int32_t), or_cmp, &ctx);
      for (int k = 0; k < OR_K; ++k) {
        idx[((int64_t)b * N + r) * OR_K + k] = order[k];
        val[((int64_t)b * N + r) * OR_K + k] = or_load(row, dtype, order[k]);
      }
    }
  free(order);
}

/* The first element of a row under the top-k order (a plain argmax with that policy). */
static int64_t or_row_first(const void *row, int dtype, int V) {
  int64_t best = 0;
  for (int64_t x = 1; x < V; ++x)
    if (or_before(or_load(row, dtype, x), x, or_load(row, dtype, best), best)) best = x;
  return best;
}

/* ------------------------------------------------------------------------------------ */
/* Temperature classes shared by select and verify (reading of [LSE] usage paragraph:    */
/* draft selection uses the request's sampling settings, greedy requests keep            */
/* deterministic selection). T == 0 is greedy; a positive finite T whose reciprocal is   */
/* finite is sampled; anything else is flagged and treated as greedy.                    */
/* ------------------------------------------------------------------------------------ */

#define OR_GREEDY 0
#define OR_SAMPLED 1

static int or_mode(float T, float *invT, int32_t *st) {
  if (T == 0.0f) return OR_GREEDY;
  if (T > 0.0f && isfinite(T)) {
    float inv = 1.0f / T;
    if (isfinite(inv)) {
      *invT = inv;
      return OR_SAMPLED;
    }
  }
  *st |= OR_ST_BADTEMP;
  return OR_GREEDY;
}

/* ------------------------------------------------------------------------------------ */
/* Selector transition ([VLLM] PR description, second item):                             */
/*   edge(p -> c) = < A[p] (*) g, B[c] > + unary[c]                                      */
/* with A the predecessor codebook, B the successor codebook (both [V,R] bf16), g the    */
/* gate for the successor's slot (the projection of the drafter state; supplied), and   */
/* unary[c] the candidate's draft logit (reading: the top-16 value; a log-softmax would  */
/* add one constant per position, which changes neither the best path nor the walk's    */
/* softmax). Binary32: prod_r = fl(fl(A[p,r] * g[r]) * B[c,r]); the dot is the           */
/* left-to-right sum t = fl(t + prod_r), r = 0..R-1; score = fl(unary + t). The pages'   */
/* selector bound (gamma_{R+2} on the absolute products plus a relative term) is the     */
/* error bound of exactly this evaluation.                                               */
/* ------------------------------------------------------------------------------------ */

static float or_transition(const float *A_row, const float *g, const float *B_row, int R) {
  float t = 0.0f;
  for (int r = 0; r < R; ++r) {
    float ag = A_row[r] * g[r];
    float pr = ag * B_row[r];
    t = t + pr;
  }
  return t;
}

/* ------------------------------------------------------------------------------------ */
/* Codebook rows. bf16 rows widen exactly. Affine Q8 rows ([LSE] conversion notes: matrix */
/* weights and selector codebooks use affine Q8 with groups of 64, BF16 scale and bias,  */
/* FP32 activations and accumulation): reading, an unsigned 8-bit code q per element and */
/* value = fl(fl(scale * q) + bias) in binary32, scale and bias of the element's group   */
/* of 64 widened from bf16.                                                               */
/* ------------------------------------------------------------------------------------ */

typedef struct {
  const uint16_t *bf16;  /* [V, R] bf16 bits, or NULL for Q8 */
  const uint8_t *codes;  /* [V, R] */
  const uint16_t *scale; /* [V, R / 64] bf16 bits */
  const uint16_t *bias;  /* [V, R / 64] bf16 bits */
} or_codebook;

static void or_row(const or_codebook *cb, int64_t v, int R, float *out) {
  if (cb->bf16) {
    for (int r = 0; r < R; ++r) out[r] = or_bf16_to_f32(cb->bf16[v * R + r]);
    return;
  }
  const int G = R / 64;
  for (int r = 0; r < R; ++r) {
    const float sc = or_bf16_to_f32(cb->scale[v * G + r / 64]);
    const float bi = or_bf16_to_f32(cb->bias[v * G + r / 64]);
    const float sq = sc * (float)cb->codes[v * R + r];
    out[r] = sq + bi;
  }
}

/* ------------------------------------------------------------------------------------ */
/* Best path ([VLLM] PR description: walk the best path from the verified anchor).       */
/* Reading: the max-sum path over the lattice (Viterbi). s1[k] is the slot-1 score of    */
/* candidate k (its only predecessor is the anchor); s[(i-2)*K*K + kp*K + k] is the      */
/* score of moving from candidate kp of slot i-1 to candidate k of slot i. Binary32:     */
/* delta_i[k] = max_kp fl(delta_{i-1}[kp] + s_i(kp,k)), scanning kp upward and replacing */
/* only on a strictly larger value; the final slot also takes the first maximum. In     */
/* exact arithmetic this returns, among the best paths, the one whose slots are smallest */
/* compared from the last slot backwards. path[i-1] = chosen candidate of slot i.        */
/* ------------------------------------------------------------------------------------ */

void or_viterbi(int K, int N, const float *s1, const float *s, int32_t *path) {
  float *dp = (float *)malloc(sizeof(float) * (size_t)K * (size_t)N);
  int32_t *bp = (int32_t *)malloc(sizeof(int32_t) * (size_t)K * (size_t)N);
  for (int k = 0; k < K; ++k) {
    dp[k] = s1[k];
    bp[k] = -1;
  }
  for (int i = 2; i <= N; ++i)
    for (int k = 0; k < K; ++k) {
      float best = 0.0f;
      int arg = -1;
      for (int kp = 0; kp < K; ++kp) {
        float v = dp[(i - 2) * K + kp] + s[((int64_t)(i - 2) * K + kp) * K + k];
        if (arg < 0 || v > best) {
          best = v;
          arg = kp;
        }
      }
      dp[(i - 1) * K + k] = best;
      bp[(i - 1) * K + k] = arg;
    }
  int last = 0;
  for (int k = 1; k < K; ++k)
    if (dp[(N - 1) * K + k] > dp[(N - 1) * K + last]) last = k;
  path[N - 1] = last;
  for (int i = N; i >= 2; --i) path[i - 2] = bp[(i - 1) * K + path[i - 1]];
  free(dp);
  free(bp);
}

/* ------------------------------------------------------------------------------------ */
/* Sampled walk ([VLLM] PR description: at T > 0 the selector walks by inverse CDF and   */
/* returns q over the K candidates for the lossless verify). For slot i with previous   */
/* choice prev: scores s_k = s_i(prev, k); m = max_k s_k; y_k = fl(fl(s_k - m) * invT);  */
/* e_k = exp_c(y_k); running sums C_k = fl(C_{k-1} + e_k) with Z = C_{K-1}; u = the     */
/* walk uniform of (b, i); tau = fl(u * Z) < Z; the choice is the smallest k with        */
/* C_k > tau (so e_k > 0); q_i[k] = fl(e_k / Z). uniforms[i-1] is the walk uniform.      */
/* score_of(i, kp, k) semantics as in or_viterbi (kp ignored for slot 1).                */
/* ------------------------------------------------------------------------------------ */

void or_walk(int K, int N, const float *s1, const float *s, float invT, const float *uniforms,
             int32_t *path, float *q) {
  float *e = (float *)malloc(sizeof(float) * (size_t)K);
  float *cum = (float *)malloc(sizeof(float) * (size_t)K);
  float *sk = (float *)malloc(sizeof(float) * (size_t)K);
  int prev = -1;
  for (int i = 1; i <= N; ++i) {
    for (int k = 0; k < K; ++k)
      sk[k] = (i == 1) ? s1[k] : s[((int64_t)(i - 2) * K + prev) * K + k];
    float m = sk[0];
    for (int k = 1; k < K; ++k)
      if (sk[k] > m) m = sk[k];
    float Z = 0.0f;
    for (int k = 0; k < K; ++k) {
      float diff = sk[k] - m;
      float y = diff * invT;
      e[k] = or_exp_c(y);
      Z = Z + e[k];
      cum[k] = Z;
    }
    float tau = uniforms[i - 1] * Z;
    int pick = K - 1;
    for (int k = 0; k < K; ++k)
      if (cum[k] > tau) {
        pick = k;
        break;
      }
    for (int k = 0; k < K; ++k) q[(int64_t)(i - 1) * K + k] = e[k] / Z;
    path[i - 1] = pick;
    prev = pick;
  }
  free(e);
  free(cum);
  free(sk);
}

/* ------------------------------------------------------------------------------------ */
/* The selector for a batch ([VLLM] PR description, second item; [LSE] geometry          */
/* paragraph: each choice conditioned on its predecessor, top-16 candidates, rank-256    */
/* codebooks; [LSE] top-k paragraph: the selector rejects nonfinite scores).             */
/*                                                                                       */
/* cand_idx, cand_val [B,N,16]; gate [B,N,R] (row i-1 is slot i's gate); pred_cb,        */
/* succ_cb [V,R] bf16 bits; anchor [B]; temperature [B]. Outputs tokens, slot [B,N]      */
/* (-1 when the sequence is rejected), q [B,N,16] (one-hot on the chosen slot when       */
/* greedy; 0 when rejected), status [B] (cleared here). lattice, if not NULL, receives   */
/* [B,N,16,16] scores; slot 1 fills row 0 (the anchor) and leaves rows 1..15 zero.       */
/* ------------------------------------------------------------------------------------ */

static void or_select_cb(const int32_t *cand_idx, const float *cand_val, const float *gate,
                         const or_codebook *pred_cb, const or_codebook *succ_cb, int V, int R,
                         const int32_t *anchor, const float *temperature, uint64_t seed,
                         uint64_t step, int B, int N, int32_t *tokens, int32_t *slot, float *q,
                         int32_t *status, float *lattice) {
  const int K = OR_K;
  float *arow = (float *)malloc(sizeof(float) * (size_t)R);
  float *brow = (float *)malloc(sizeof(float) * (size_t)R);
  float *s1 = (float *)malloc(sizeof(float) * K);
  float *s = (float *)malloc(sizeof(float) * (size_t)(N > 1 ? N - 1 : 1) * K * K);
  float *uni = (float *)malloc(sizeof(float) * (size_t)N);
  int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (size_t)N);
  float *qq = (float *)malloc(sizeof(float) * (size_t)N * K);
  for (int b = 0; b < B; ++b) {
    int32_t st = 0;
    const int32_t *ci = cand_idx + (int64_t)b * N * K;
    const float *cv = cand_val + (int64_t)b * N * K;
    int ok = anchor[b] >= 0 && anchor[b] < V;
    for (int e = 0; e < N * K; ++e)
      if (ci[e] < 0 || ci[e] >= V) ok = 0;
    if (!ok) st |= OR_ST_BADTOKEN;
    if (lattice) memset(lattice + (int64_t)b * N * K * K, 0, sizeof(float) * (size_t)N * K * K);
    int finite = 1;
    if (ok) {
      for (int i = 1; i <= N; ++i) {
        const float *g = gate + ((int64_t)b * N + (i - 1)) * R;
        int npred = (i == 1) ? 1 : K;
        for (int kp = 0; kp < npred; ++kp) {
          int64_t p = (i == 1) ? anchor[b] : ci[(i - 2) * K + kp];
          for (int k = 0; k < K; ++k) {
            int64_t c = ci[(i - 1) * K + k];
            or_row(pred_cb, p, R, arow);
            or_row(succ_cb, c, R, brow);
            float t = or_transition(arow, g, brow, R);
            float sc = cv[(i - 1) * K + k] + t;
            if (!isfinite(sc) || !isfinite(cv[(i - 1) * K + k])) finite = 0;
            if (i == 1)
              s1[k] = sc;
            else
              s[((int64_t)(i - 2) * K + kp) * K + k] = sc;
            if (lattice) lattice[(((int64_t)b * N + (i - 1)) * K + kp) * K + k] = sc;
          }
        }
      }
      if (!finite) st |= OR_ST_NONFINITE;
    }
    float invT = 0.0f;
    int mode = or_mode(temperature[b], &invT, &st);
    if (!ok || !finite) {
      for (int i = 0; i < N; ++i) {
        tokens[(int64_t)b * N + i] = -1;
        slot[(int64_t)b * N + i] = -1;
        for (int k = 0; k < K; ++k) q[((int64_t)b * N + i) * K + k] = 0.0f;
      }
      status[b] = st;
      continue;
    }
    if (mode == OR_GREEDY) {
      or_viterbi(K, N, s1, s, path);
      for (int i = 0; i < N; ++i)
        for (int k = 0; k < K; ++k) qq[i * K + k] = (k == path[i]) ? 1.0f : 0.0f;
    } else {
      for (int i = 1; i <= N; ++i) {
        uint64_t w[4];
        or_draw(seed, step, b, i, w);
        uni[i - 1] = or_uniform24(w[0]);
      }
      or_walk(K, N, s1, s, invT, uni, path, qq);
    }
    for (int i = 0; i < N; ++i) {
      tokens[(int64_t)b * N + i] = ci[i * K + path[i]];
      slot[(int64_t)b * N + i] = path[i];
      for (int k = 0; k < K; ++k) q[((int64_t)b * N + i) * K + k] = qq[i * K + k];
    }
    status[b] = st;
  }
  free(s1);
  free(s);
  free(uni);
  free(path);
  free(qq);
  free(arow);
  free(brow);
}

void or_select(const int32_t *cand_idx, const float *cand_val, const float *gate,
               const uint16_t *pred_cb, const uint16_t *succ_cb, int V, int R,
               const int32_t *anchor, const float *temperature, uint64_t seed, uint64_t step, int B,
               int N, int32_t *tokens, int32_t *slot, float *q, int32_t *status, float *lattice) {
  or_codebook a = {pred_cb, NULL, NULL, NULL}, c = {succ_cb, NULL, NULL, NULL};
  or_select_cb(cand_idx, cand_val, gate, &a, &c, V, R, anchor, temperature, seed, step, B, N,
               tokens, slot, q, status, lattice);
}

void or_select_q8(const int32_t *cand_idx, const float *cand_val, const float *gate,
                  const uint8_t *pred_codes, const uint16_t *pred_scale, const uint16_t *pred_bias,
                  const uint8_t *succ_codes, const uint16_t *succ_scale, const uint16_t *succ_bias,
                  int V, int R, const int32_t *anchor, const float *temperature, uint64_t seed,
                  uint64_t step, int B, int N, int32_t *tokens, int32_t *slot, float *q,
                  int32_t *status, float *lattice) {
  or_codebook a = {NULL, pred_codes, pred_scale, pred_bias};
  or_codebook c = {NULL, succ_codes, succ_scale, succ_bias};
  or_select_cb(cand_idx, cand_val, gate, &a, &c, V, R, anchor, temperature, seed, step, B, N,
               tokens, slot, q, status, lattice);
}

/* ------------------------------------------------------------------------------------ */
/* Draft tree by best-first expansion over the selector lattice ("qwen35: DSpark          */
/* speculative decoding (Qwen3.8-27B drafters) - #625", the DDTree commit: each expansion */
/* scores a candidate as its draft log-probability plus the selector's compatibility with */
/* the branch's actual parent, log-softmax normalised per position so that cumulative     */
/* best-first comparisons across depths stay on one scale, under a node budget).          */
/* Readings: the edge score is the selector lattice s_i(p, k) (candidate value plus the   */
/* rank-R term); for each parent row, d_k = fl(s_k - max), Z = sum_k exp_c(d_k) (k        */
/* ascending), ls_k = fl(d_k - log_c(Z)). A node is (depth i, candidate k, parent node);  */
/* its score is fl(parent score + ls), the root (the anchor) scoring 0. The frontier       */
/* starts with the root's 16 children (in k order); each of `budget` rounds takes the     */
/* frontier entry with the largest score (ties: the earliest added), records it, and if   */
/* its depth is below N adds its 16 children in k order. Outputs per tree node t (the      */
/* order taken): parent (tree index, -1 under the root), depth (1..N), slot k, token and   */
/* score. Index and finiteness checks are the selector's (BADTOKEN, NONFINITE; outputs -1 */
/* and score 0).                                                                           */
/* ------------------------------------------------------------------------------------ */

float or_log_c(float x);

void or_ddtree(const int32_t *cand_idx, const float *cand_val, const float *gate,
               const uint16_t *pred_cb, const uint16_t *succ_cb, int V, int R,
               const int32_t *anchor, int B, int N, int budget, int32_t *parent, int32_t *depth,
               int32_t *slotk, int32_t *token, float *score, int32_t *status) {
  const int K = OR_K;
  or_codebook pa = {pred_cb, NULL, NULL, NULL}, pc = {succ_cb, NULL, NULL, NULL};
  float *arow = (float *)malloc(sizeof(float) * (size_t)R);
  float *brow = (float *)malloc(sizeof(float) * (size_t)R);
  float *ls = (float *)malloc(sizeof(float) * (size_t)N * K * K);
  const int fmax = K + budget * K;
  float *fs = (float *)malloc(sizeof(float) * (size_t)fmax);
  int *fd = (int *)malloc(sizeof(int) * (size_t)fmax);
  int *fk = (int *)malloc(sizeof(int) * (size_t)fmax);
  int *fp = (int *)malloc(sizeof(int) * (size_t)fmax);
  int *alive = (int *)malloc(sizeof(int) * (size_t)fmax);
  for (int b = 0; b < B; ++b) {
    int32_t st = 0;
    const int32_t *ci = cand_idx + (int64_t)b * N * K;
    const float *cv = cand_val + (int64_t)b * N * K;
    int ok = anchor[b] >= 0 && anchor[b] < V;
    for (int e = 0; e < N * K; ++e)
      if (ci[e] < 0 || ci[e] >= V) ok = 0;
    int finite = 1;
    if (ok) {
      for (int i = 1; i <= N; ++i) {
        const float *g = gate + ((int64_t)b * N + (i - 1)) * R;
        const int npred = (i == 1) ? 1 : K;
        for (int kp = 0; kp < npred; ++kp) {
          const int64_t p = (i == 1) ? anchor[b] : ci[(i - 2) * K + kp];
          float row[OR_K];
          for (int k = 0; k < K; ++k) {
            or_row(&pa, p, R, arow);
            or_row(&pc, ci[(i - 1) * K + k], R, brow);
            row[k] = cv[(i - 1) * K + k] + or_transition(arow, g, brow, R);
            if (!isfinite(row[k]) || !isfinite(cv[(i - 1) * K + k])) finite = 0;
          }
          float m = row[0];
          for (int k = 1; k < K; ++k) m = row[k] > m ? row[k] : m;
          float d[OR_K], Z = 0.0f;
          for (int k = 0; k < K; ++k) {
            d[k] = row[k] - m;
            Z = Z + or_exp_c(d[k]);
          }
          const float lz = or_log_c(Z);
          for (int k = 0; k < K; ++k) ls[((int64_t)(i - 1) * K + kp) * K + k] = d[k] - lz;
        }
      }
    }
    if (!ok) st |= OR_ST_BADTOKEN;
    if (ok && !finite) st |= OR_ST_NONFINITE;
    int32_t *opar = parent + (int64_t)b * budget, *odep = depth + (int64_t)b * budget;
    int32_t *oslt = slotk + (int64_t)b * budget, *otok = token + (int64_t)b * budget;
    float *osc = score + (int64_t)b * budget;
    if (!ok || !finite) {
      for (int t = 0; t < budget; ++t) {
        opar[t] = odep[t] = oslt[t] = otok[t] = -1;
        osc[t] = 0.0f;
      }
      status[b] = st;
      continue;
    }
    int F = 0;
    for (int k = 0; k < K; ++k) {
      fs[F] = 0.0f + ls[k]; /* slot 1, the anchor's row */
      fd[F] = 1;
      fk[F] = k;
      fp[F] = -1;
      alive[F] = 1;
      ++F;
    }
    for (int t = 0; t < budget; ++t) {
      int best = -1;
      for (int f = 0; f < F; ++f)
        if (alive[f] && (best < 0 || fs[f] > fs[best])) best = f;
      if (best < 0) { /* nothing left (the whole tree is taken) */
        opar[t] = odep[t] = oslt[t] = otok[t] = -1;
        osc[t] = 0.0f;
        continue;
      }
      alive[best] = 0;
      opar[t] = fp[best];
      odep[t] = fd[best];
      oslt[t] = fk[best];
      otok[t] = ci[(fd[best] - 1) * K + fk[best]];
      osc[t] = fs[best];
      if (fd[best] < N) {
        for (int k = 0; k < K; ++k) {
          fs[F] = fs[best] + ls[((int64_t)fd[best] * K + fk[best]) * K + k];
          fd[F] = fd[best] + 1;
          fk[F] = k;
          fp[F] = t;
          alive[F] = 1;
          ++F;
        }
      }
    }
    status[b] = st;
  }
  free(arow);
  free(brow);
  free(ls);
  free(fs);
  free(fd);
  free(fk);
  free(fp);
  free(alive);
}

/* Q8 rows as binary32 (for tests that compare against the dequantized values). */
void or_q8_dequant(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias, int64_t V,
                   int R, float *out) {
  or_codebook cb = {NULL, codes, scale, bias};
  for (int64_t v = 0; v < V; ++v) or_row(&cb, v, R, out + v * R);
}

/* ------------------------------------------------------------------------------------ */
/* Verify ([LSE] usage paragraph: the target verifies all seven proposals with           */
/* probability-ratio rejection and residual sampling; greedy keeps a deterministic       */
/* chain. [LSE] geometry paragraph: the verifier consumes the anchor plus all seven      */
/* proposals, so row j-1 of the target checks proposal j and row N follows the last).   */
/*                                                                                       */
/* Greedy (T == 0): y_j = first element of row j-1 under the top-k order; proposals are  */
/* accepted while d_j == y_j; then y at the first mismatch is emitted, or the first      */
/* element of row N if all N matched. A NaN chosen as y sets NONFINITE.                  */
/*                                                                                       */
/* Sampled (T > 0; target rows are binary32 probabilities): proposal j with draft        */
/* probability qx (q row j-1 at its slot) and target probability pt is accepted iff      */
/* fl(u * qx) < pt, u the accept uniform of (b, j). At the first rejection the token is  */
/* drawn from the residual max(0, p_t - q_j) over the whole vocabulary (q_j is zero off  */
/* the 16 candidates), renormalised; if all N are accepted the bonus token is drawn from */
/* row N. Reading for exact, order-free sampling: each weight is quantised to            */
/* R(x) = floor(r(x) * 2^40) (exact: r*2^40 is an exact binary32 scaling), Z = sum R in  */
/* uint64, tau = floor(w2 * Z / 2^64) with w2 the 64-bit draw of (b, position), and the  */
/* token is the smallest x whose running sum of R exceeds tau. A residual of zero mass   */
/* falls back to p_t itself; if that is zero too the row's first element is emitted and  */
/* ZEROMASS is set. Probabilities outside [0, 1] (or NaN) count as 0 and set BADPROB.    */
/* A proposal outside [0, V) is a rejection; one whose slot or candidate does not match  */
/* sets BADTOKEN and is rejected with q taken as 0.                                      */
/*                                                                                       */
/* target: row r of sequence b at element b*seq_stride + r*row_stride, rows 0..N.        */
/* tokens, slot [B,N]; cand_idx, q [B,N,16]; out_tokens [B,N+1] (-1 padded); status |=.  */
/* ------------------------------------------------------------------------------------ */

static float or_prob(float p, int32_t *st) {
  if (p >= 0.0f && p <= 1.0f) return p;
  *st |= OR_ST_BADPROB;
  return 0.0f;
}

static uint64_t or_quant40(float r) { return (uint64_t)floorf(r * 0x1p40f); }

/* Draw from weights R(x) over a row, where R comes from `weight(x)`. Returns -1 when the
 * total mass is zero. */
typedef struct {
  const float *row;
  int V;
  const int32_t *cidx; /* NULL for a plain p_t row */
  const float *cq;
  int32_t *st;
} or_resid;

static uint64_t or_resid_weight(const or_resid *rs, int64_t x, int use_plain) {
  float p = or_prob(rs->row[x], rs->st);
  if (!use_plain && rs->cidx) {
    for (int k = 0; k < OR_K; ++k)
      if (rs->cidx[k] == x) {
        float qk = or_prob(rs->cq[k], rs->st);
        float d = p - qk;
        return or_quant40(d > 0.0f ? d : 0.0f);
      }
  }
  return or_quant40(p);
}

static int64_t or_draw_row(const or_resid *rs, uint64_t w2) {
  for (int use_plain = 0; use_plain < 2; ++use_plain) {
    if (use_plain && !rs->cidx) break;
    uint64_t Z = 0;
    for (int64_t x = 0; x < rs->V; ++x) Z += or_resid_weight(rs, x, use_plain);
    if (Z == 0) continue;
    uint64_t tau = (uint64_t)(((unsigned __int128)w2 * Z) >> 64);
    uint64_t run = 0;
    for (int64_t x = 0; x < rs->V; ++x) {
      run += or_resid_weight(rs, x, use_plain);
      if (run > tau) return x;
    }
  }
  return -1;
}

void or_verify(const void *target, int dtype, int64_t seq_stride, int64_t row_stride, int V,
               const int32_t *tokens, const int32_t *cand_idx, const float *q, const int32_t *slot,
               const float *temperature, uint64_t seed, uint64_t step, int B, int N,
               int32_t *n_accept, int32_t *out_tokens, int32_t *status) {
  for (int b = 0; b < B; ++b) {
    int32_t st = 0;
    float invT = 0.0f;
    int mode = or_mode(temperature[b], &invT, &st);
    if (mode == OR_SAMPLED && dtype != OR_F32) {
      st |= OR_ST_BADPROB; /* sampling needs probabilities; take the greedy chain */
      mode = OR_GREEDY;
    }
    int64_t base = (int64_t)b * seq_stride;
    int32_t *out = out_tokens + (int64_t)b * (N + 1);
    for (int j = 0; j <= N; ++j) out[j] = -1;
    const int32_t *d = tokens + (int64_t)b * N;
    int n = 0;
    int64_t emitted = -1;
    if (mode == OR_GREEDY) {
      for (int j = 1; j <= N + 1; ++j) {
        const void *row = dtype == OR_F32
                              ? (const void *)((const float *)target + base + (int64_t)(j - 1) * row_stride)
                              : (const void *)((const uint16_t *)target + base + (int64_t)(j - 1) * row_stride);
        int64_t y = or_row_first(row, dtype, V);
        if (isnan(or_load(row, dtype, y))) st |= OR_ST_NONFINITE;
        if (j <= N && d[j - 1] == y) {
          ++n;
          continue;
        }
        emitted = y;
        break;
      }
    } else {
      const float *tgt = (const float *)target + base;
      int rejected_at = 0;   /* 0: all accepted */
      int reject_plain = 0;  /* rejected with q taken as 0 */
      for (int j = 1; j <= N; ++j) {
        int32_t x = d[j - 1];
        const float *row = tgt + (int64_t)(j - 1) * row_stride;
        uint64_t w[4];
        or_draw(seed, step, b, j, w);
        float u = or_uniform24(w[1]);
        if (x < 0 || x >= V) {
          rejected_at = j;
          reject_plain = 1;
          break;
        }
        int32_t sl = slot[(int64_t)b * N + (j - 1)];
        const int32_t *ci = cand_idx + ((int64_t)b * N + (j - 1)) * OR_K;
        if (sl < 0 || sl >= OR_K || ci[sl] != x) {
          st |= OR_ST_BADTOKEN;
          rejected_at = j;
          reject_plain = 1;
          break;
        }
        float qx = or_prob(q[((int64_t)b * N + (j - 1)) * OR_K + sl], &st);
        float pt = or_prob(row[x], &st);
        if (u * qx < pt) {
          ++n;
          continue;
        }
        rejected_at = j;
        break;
      }
      int pos = rejected_at ? rejected_at : N + 1; /* block position of the drawn token */
      const float *row = tgt + (int64_t)(pos - 1) * row_stride;
      or_resid rs;
      rs.row = row;
      rs.V = V;
      rs.st = &st;
      if (rejected_at && !reject_plain) {
        rs.cidx = cand_idx + ((int64_t)b * N + (rejected_at - 1)) * OR_K;
        rs.cq = q + ((int64_t)b * N + (rejected_at - 1)) * OR_K;
      } else {
        rs.cidx = NULL;
        rs.cq = NULL;
      }
      uint64_t w[4];
      or_draw(seed, step, b, pos, w);
      emitted = or_draw_row(&rs, w[2]);
      if (emitted < 0) {
        st |= OR_ST_ZEROMASS;
        emitted = or_row_first(row, OR_F32, V);
      }
    }
    for (int j = 0; j < n; ++j) out[j] = d[j];
    out[n] = (int32_t)emitted;
    n_accept[b] = n;
    status[b] |= st;
  }
}

/* ------------------------------------------------------------------------------------ */
/* log_c(x), x > 0 finite: x = 2^e * m with m in [sqrt(1/2), sqrt(2)), and               */
/* log x = e ln 2 + 2 atanh(u), u = (m - 1) / (m + 1), |u| <= 0.1716, with               */
/* 2 atanh(u) = 2u (1 + u^2/3 + u^4/5 + u^6/7 + u^8/9) in Horner form (fmaf) and e ln 2   */
/* as e * LN2_HI + e * LN2_LO. Every step one correctly rounded binary32 operation.       */
/* ------------------------------------------------------------------------------------ */

float or_log_c(float x) {
  const float LN2_HI = 0.693145751953125f;
  const float LN2_LO = 1.42860677e-06f;
  int e = 0;
  float m = frexpf(x, &e); /* m in [0.5, 1), exact */
  if (m < 0.707106769f) {
    m = m * 2.0f;
    e -= 1;
  }
  const float u = (m - 1.0f) / (m + 1.0f);
  const float u2 = u * u;
  float p = 0.111111112f;
  p = fmaf(p, u2, 0.142857149f);
  p = fmaf(p, u2, 0.2f);
  p = fmaf(p, u2, 0.333333343f);
  p = fmaf(p, u2, 1.0f);
  const float t = (2.0f * u) * p;
  const float ef = (float)e;
  return fmaf(ef, LN2_HI, fmaf(ef, LN2_LO, t));
}

/* Vector form of or_log_c for the accuracy sweep in the tests. */
void or_log_c_many(const float *x, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_log_c(x[i]);
}

/* Vector form of or_exp_c for the accuracy sweep in the tests. */
void or_exp_c_many(const float *y, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = or_exp_c(y[i]);
}
