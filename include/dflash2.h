/*
 * dflash2.h - C ABI of the DFlash2 block-draft-and-verify step for AMD Instinct MI355X
 * (gfx950). Library: libdflash2.so.
 *
 * One draft-and-verify step of a DFlash2 drafter has five stages, each a call below:
 * block attention and the two-tap dynamic convolution inside the drafter's layers,
 * top-16 candidate extraction per block position, the predecessor-conditioned selector,
 * and target verification. The computation is the one described on these pages:
 *   - "Geramy/LSE docs/DFLASH2.md": drafter geometry paragraph (block of eight = anchor
 *     plus seven masks, noncausal block attention, 2048-position context window, two-tap
 *     conv with groups of 16, top-16 candidates, rank-256 codebooks); usage paragraph
 *     (verification of all seven proposals by probability-ratio rejection with residual
 *     sampling, deterministic greedy selection); top-k policy paragraph (ties to the
 *     smaller index, NaNs first by index, infinities ordered normally).
 *   - "[Spec Decode] DFlash2: local convolution + candidate selector - #52816": the PR
 *     description's conv formula and selector edge score, best path from the verified
 *     anchor, inverse-CDF walk returning q for the lossless verify.
 *   - "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625": the DFlash 2
 *     commit message (two taps over the block, per-element base plus per-group dynamic
 *     coefficient; top-k, codebook gathers and path search).
 *
 * Conventions (all calls):
 *   - Every array pointer is DEVICE memory owned by the caller, and must stay valid until
 *     the work enqueued on `stream` has completed. The library allocates nothing, keeps no
 *     mutable global state (calls are thread-safe), never synchronises and never falls
 *     back to the host. The one exception is dflash2_select_noalloc, whose lattice is a
 *     static device array per GPU (its per-device address is cached under a lock).
 *   - Calls enqueue kernels on `stream` (0 = the null stream) and return at once. The
 *     return value reports argument errors known on the host (DFLASH2_E*); nothing is
 *     launched when it is nonzero. Data-dependent problems are reported per sequence in
 *     the device array `status` (DFLASH2_ST_* bits).
 *   - bf16 arrays hold 16-bit patterns (the upper half of an IEEE binary32). Element
 *     strides are in elements, not bytes.
 *   - Scratch memory is passed as `ws`/`ws_bytes`; the sizes come from the
 *     *_workspace_bytes functions. It must be 256-byte aligned. Its contents between
 *     calls do not matter, and two calls in flight at once must not share it.
 *   - Random draws come from Philox4x64-10 (Salmon et al., SC'11) with key (seed, 0) and
 *     counter (step, b, j, 0), for sequence b and block position j. Word 0 drives the
 *     selector walk at slot j, word 1 the accept test of proposal j, word 2 the residual
 *     or bonus draw of the token emitted at position j.
 */
#ifndef DFLASH2_H
#define DFLASH2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define DFLASH2_BF16 0
#define DFLASH2_F32 1

/* return codes */
#define DFLASH2_OK 0
#define DFLASH2_EINVAL (-1)       /* null pointer, bad size or inconsistent shape */
#define DFLASH2_EUNSUPPORTED (-2) /* a shape or type the library does not implement */
#define DFLASH2_EWORKSPACE (-3)   /* ws too small or misaligned */
#define DFLASH2_EHIP (-4)         /* a kernel launch failed */

/* per-sequence status bits (device int32, OR-ed) */
#define DFLASH2_ST_NONFINITE 1 /* a NaN/inf selector score, or a NaN chosen by the greedy chain */
#define DFLASH2_ST_BADTOKEN 2  /* a candidate/anchor index out of range, or a proposal whose slot
                                  does not match its candidate */
#define DFLASH2_ST_ZEROMASS 4  /* the sampling row had no mass; its first element was emitted */
#define DFLASH2_ST_BADPROB 8   /* a probability outside [0, 1] or NaN (taken as 0), or sampling
                                  requested on a bf16 target (the greedy chain was used) */
#define DFLASH2_ST_BADTEMP 16  /* a temperature that is negative, NaN, infinite or whose
                                  reciprocal overflows (treated as greedy) */
#define DFLASH2_ST_RINGLOST 32 /* a rewind went back past positions the ring still holds: the
                                  next window has stale slots until W - 1 new positions are in */
#define DFLASH2_ST_BADCOUNT 64 /* a ring update count outside [0, Pn] (clamped) */

/* Temperature classes (select and verify): T == 0 selects greedy; T > 0 and finite with a
 * finite binary32 1/T selects sampling; anything else sets ST_BADTEMP and is greedy. */

/*
 * dflash2_block_attn - attention of the P block positions over their windowed context and
 * the whole block ("Geramy/LSE docs/DFLASH2.md", drafter geometry paragraph).
 *
 *   q      [B, P, Hq, D]    queries (after any rotary embedding)
 *   k_blk, v_blk [B, P, Hkv, D]  keys/values of the P block positions
 *   k_ring, v_ring [B, S, Hkv, D] context keys/values; context position j of sequence b
 *                            lives in row j mod S
 *   ctx_len [B] int32       L_b, the number of context positions (>= 0)
 *   out    [B, P, Hq, D]    result, same dtype as q
 *
 * Slot i of sequence b sits at absolute position L_b + i. It attends to every block key
 * (noncausal inside the block) and to context positions j with L_b + i - j < W and
 * 0 <= j < L_b. Query head h uses KV head h / (Hq / Hkv). Scores are scaled by `scale`
 * (pass 1/sqrt(D) for the usual scaling), softmax in binary32.
 * dtype: DFLASH2_BF16 (MFMA path) or DFLASH2_F32, for all of q, k*, v*, out.
 * The window may be split across workgroups; the workspace then holds the split partials
 * and their softmax statistics, which a second kernel combines.
 * Requires B >= 1, 2 <= P <= 16, Hq % Hkv == 0, (Hq / Hkv) * P <= 32 for bf16 (64 for
 * f32), D in {64, 128}, W >= 1, S >= W - 1 (every windowed key is still in the ring),
 * and ctx_len[b] >= 0 (negative values are clamped to 0 on the device).
 * Workspace: dflash2_block_attn_workspace_bytes.
 */
int dflash2_block_attn(const void *q, const void *k_blk, const void *v_blk, const void *k_ring,
                       const void *v_ring, const int32_t *ctx_len, void *out, int B, int P, int Hq,
                       int Hkv, int D, int S, int W, float scale, int dtype, void *ws,
                       size_t ws_bytes, hipStream_t stream);
size_t dflash2_block_attn_workspace_bytes(int B, int P, int Hq, int Hkv, int D, int S, int W,
                                          int dtype);

/*
 * dflash2_dynconv2 - grouped dynamic two-tap convolution over the block ("[Spec Decode]
 * DFlash2: local convolution + candidate selector - #52816", PR description, first item):
 *
 *   out[b,i,c] = (base[0,c] + delta[b,i,0,c/group]) * x[b,i,c]
 *              + (base[1,c] + delta[b,i,1,c/group]) * x[b,i-1,c],   x[b,-1,c] = 0
 *
 *   x, out [B, P, C] (dtype), base [2, C] f32, delta [B, P, 2, C/group] f32.
 * Arithmetic in binary32, each product and sum rounded once, result rounded to dtype.
 * Requires group == 16 and C % 16 == 0, P in [1, 16], B*P <= 65535. No workspace. out may
 * not alias x.
 */
int dflash2_dynconv2(const void *x, const float *base, const float *delta, void *out, int B, int P,
                     int C, int group, int dtype, hipStream_t stream);

/*
 * dflash2_topk16 - the 16 first elements of each logits row under the order: every NaN
 * (by ascending index), then +inf, finite values descending, -inf; equal values (and -0,
 * +0) by ascending index ("Geramy/LSE docs/DFLASH2.md", top-k policy paragraph).
 *
 *   scores  rows addressed as scores[b*seq_stride + (row0 + r)*row_stride + x], r < N, x < V
 *   idx     [B, N, 16] int32 (best first); val [B, N, 16] f32 (the element, widened)
 * Requires V >= 16, N >= 1, row0 >= 0, strides >= 0, B*N <= 65535, V <= 8388608.
 * Workspace: dflash2_topk16_workspace_bytes.
 */
int dflash2_topk16(const void *scores, int dtype, int B, int N, int row0, int64_t seq_stride,
                   int64_t row_stride, int V, int32_t *idx, float *val, void *ws, size_t ws_bytes,
                   hipStream_t stream);
size_t dflash2_topk16_workspace_bytes(int B, int N, int V, int dtype);

/*
 * dflash2_lmhead_topk16 - the drafter's output-head projection fused with the top-16
 * ("Geramy/LSE docs/DFLASH2.md", drafter-geometry paragraph: the drafter shares the
 * target's output head; "qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) -
 * #625", DFlash 2 commit: the selector takes the top-k head candidates per block position).
 *
 *   logit[b,r,v] = sum_c hidden[b*hid_seq_stride + (row0 + r)*hid_row_stride + c] * weight[v*C + c]
 *
 *   hidden  bf16, rows r < N of each of the B sequences, C elements each
 *   weight  bf16 [V, C] row-major (an output head's usual layout)
 *   idx     [B, N, 16] int32, val [B, N, 16] f32: the 16 first (v, logit) under the order
 *           of dflash2_topk16, taken on the binary32 logits
 * The bf16 products are exact; they are summed in binary32 in an unspecified order, so a
 * logit may differ from the exact sum by at most about C * 2^-24 * sum_c |h_c w_c| (and
 * candidates whose logits lie that close may trade places). The logits are never stored.
 * A NaN logit is reported as a quiet NaN. Requires C % 128 == 0, 16-byte aligned hidden
 * and weight with strides that are multiples of 8, V >= 16, B*N <= 65535. Hidden rows are
 * processed 32 per pass over the weight. Workspace: dflash2_lmhead_topk16_workspace_bytes.
 */
int dflash2_lmhead_topk16(const void *hidden, int64_t hid_seq_stride, int64_t hid_row_stride,
                          int row0, const void *weight, int C, int V, int B, int N, int32_t *idx,
                          float *val, void *ws, size_t ws_bytes, hipStream_t stream);
size_t dflash2_lmhead_topk16_workspace_bytes(int B, int N, int V, int C);

/*
 * dflash2_proj - the drafter's linear projections on either side of the path: the dynamic
 * conv's per-group coefficients, taken from one projection of the sublayer's input, and
 * the selector gate, a projection of each block slot's hidden state that multiplies the
 * predecessor codebook row elementwise ("[Spec Decode] DFlash2: local convolution +
 * candidate selector - #52816", PR description, both items; "qwen35: DSpark speculative
 * decoding (Qwen3.8-27B drafters) - #625", DFlash 2 commit: kernel projections, hproj).
 *
 *   out[b*out_seq_stride + r*out_row_stride + o]
 *       = sum_c hidden[b*hid_seq_stride + (row0 + r)*hid_row_stride + c] * weight[o*C + c]
 *
 *   hidden  bf16, rows r < N of each of the B sequences, C elements each (strides may be 0)
 *   weight  bf16 [O, C] row-major (a linear layer's usual layout)
 *   out     f32; the B*N output rows of O values must not overlap (sequence-major or
 *           row-major placement, else DFLASH2_EINVAL); out may not alias the inputs
 * The bf16 products are exact; they are summed in binary32 in a fixed order (the result
 * does not vary between calls), within C * 2^-24 * sum_c |h_c w_c| of the exact sum for
 * ordinary magnitudes. Conv coefficients: with a sublayer's coefficient weight [4G, C]
 * ordered (conv s, tap t, group g) -> (2s + t)G + g, the first 2G rows give the conv
 * before the sublayer and the last 2G the conv after it, each [B, P, 2, G] as
 * dflash2_dynconv2 takes delta (one call per half, weight offset by 2G*C). Selector gate:
 * weight [R, C], rows row0 = 1 .. N of the block, out [B, N, R]. Requires C % 8 == 0,
 * 16-byte aligned hidden and weight, hidden strides multiples of 8, B*N <= 2^20,
 * O <= 2^26. Workspace: dflash2_proj_workspace_bytes (0 when the call needs none; then ws
 * may be null). Small calls split the contraction over workgroups and add the partials
 * there in a fixed order.
 */
int dflash2_proj(const void *hidden, int64_t hid_seq_stride, int64_t hid_row_stride, int row0,
                 const void *weight, int C, int O, int B, int N, float *out,
                 int64_t out_seq_stride, int64_t out_row_stride, void *ws, size_t ws_bytes,
                 hipStream_t stream);
size_t dflash2_proj_workspace_bytes(int B, int N, int O, int C);

/*
 * dflash2_ring_update - keeps a drafter context ring in step with the committed sequence
 * after verification ("Geramy/LSE docs/DFLASH2.md", native-test notes: cache rewind,
 * replacement and reset). Position p of sequence b lives in ring slot p mod S (the layout
 * dflash2_block_attn reads). For each b, in this order:
 *   1. back[b] < 0 resets the sequence (ctx_len[b] = 0); otherwise the sequence is rewound
 *      by min(back[b], ctx_len[b]) positions. If the rewound window (positions
 *      max(0, L' - W + 1) .. L' - 1) is not empty and reaches below the oldest position the
 *      ring held (max(0, L - S)), DFLASH2_ST_RINGLOST is set: those slots hold later positions.
 *   2. rows j < n_new[b] of new_k/new_v are written to slots (L' + j) mod S, and
 *      ctx_len[b] = L' + n_new[b]. A count outside [0, Pn] sets DFLASH2_ST_BADCOUNT and is
 *      clamped.
 *   new_k, new_v [B, Pn, Hkv, D] (dtype); k_ring, v_ring [B, S, Hkv, D]; ctx_len [B] in/out;
 *   n_new, back [B]; status [B] OR-ed. Requires Pn <= 16, Pn <= S, S >= W - 1, Hkv*D*size
 *   a multiple of 16 bytes and 16-byte aligned arrays. Negative ctx_len values count as 0.
 */
int dflash2_ring_update(const void *new_k, const void *new_v, const int32_t *n_new,
                        const int32_t *back, int32_t *ctx_len, void *k_ring, void *v_ring, int B,
                        int Pn, int Hkv, int D, int S, int W, int dtype, int32_t *status,
                        hipStream_t stream);

/*
 * dflash2_select - the candidate selector ("[Spec Decode] DFlash2: local convolution +
 * candidate selector - #52816", PR description, second item).
 *
 * Edge score from candidate p of slot i-1 (the anchor for slot 1) to candidate c of slot i:
 *   s_i(p, c) = cand_val[b,i-1,c] + sum_r pred_cb[p,r] * gate[b,i-1,r] * succ_cb[c,r]
 * evaluated in binary32 as fl(fl(pred*gate)*succ) summed left to right over r, then the
 * candidate's value added. Any NaN/inf score or value sets ST_NONFINITE; any index outside
 * [0, V) sets ST_BADTOKEN; such sequences get tokens = slot = -1 and q = 0.
 * Greedy (T == 0): the max-sum path (Viterbi; ties to the lower candidate slot, the last
 * slot decided first), q one-hot at the chosen slot.
 * Sampled (T > 0): for i = 1..N, with prev the previous choice: e_k = exp_c((s_k - max)/T)
 * (exp_c: a fixed binary32 exp by Cody-Waite reduction and a degree-7 Taylor polynomial),
 * Z and running sums accumulated in k order, tau = u*Z with u the walk uniform of (b, i),
 * choice = the first k whose running sum exceeds tau, q_i[k] = e_k / Z.
 *
 *   cand_idx, cand_val [B, N, 16] (from dflash2_topk16); gate [B, N, R] f32;
 *   pred_cb, succ_cb [V, R] bf16; anchor [B] int32; temperature [B] f32;
 *   tokens, slot [B, N] int32; q [B, N, 16] f32; status [B] int32 (overwritten).
 * Requires 1 <= N <= 15, 1 <= R <= 512, V >= 16, B <= 65535.
 * Workspace: dflash2_select_workspace_bytes.
 */
int dflash2_select(const int32_t *cand_idx, const float *cand_val, const float *gate,
                   const uint16_t *pred_cb, const uint16_t *succ_cb, int V, int R,
                   const int32_t *anchor, const float *temperature, uint64_t seed, uint64_t step,
                   int B, int N, int32_t *tokens, int32_t *slot, float *q, int32_t *status,
                   void *ws, size_t ws_bytes, hipStream_t stream);
size_t dflash2_select_workspace_bytes(int B, int N);

/*
 * dflash2_select_noalloc - dflash2_select for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same kernels and the same results. The
 * lattice lives in a static device array of dflash2_select_noalloc_max_bytes() bytes (4 MiB),
 * one copy per GPU, held until the process ends; its address is looked up once per device,
 * with that device current, on the device's first call (thread-safe). The call allocates
 * nothing and never synchronises. The stream must belong to the current device.
 * Requires dflash2_select_workspace_bytes(B, N) <= dflash2_select_noalloc_max_bytes()
 * (B * N <= 4096 lattice rows of 16 x 16 binary32 scores), else DFLASH2_EWORKSPACE; a failed
 * address lookup returns DFLASH2_EHIP. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other threads) race and must not be made.
 * The lattice is fully written before it is read, so nothing needs clearing between calls.
 */
int dflash2_select_noalloc(const int32_t *cand_idx, const float *cand_val, const float *gate,
                           const uint16_t *pred_cb, const uint16_t *succ_cb, int V, int R,
                           const int32_t *anchor, const float *temperature, uint64_t seed,
                           uint64_t step, int B, int N, int32_t *tokens, int32_t *slot, float *q,
                           int32_t *status, hipStream_t stream);
size_t dflash2_select_noalloc_max_bytes(void);

/*
 * dflash2_ddtree - a draft tree by best-first expansion over the selector lattice ("qwen35:
 * DSpark speculative decoding (Qwen3.8-27B drafters) - #625", the DDTree commit: candidates
 * scored as draft log-probability plus the selector's compatibility with the branch's actual
 * parent, log-softmax normalised per position, expanded best-first under a node budget).
 *   Inputs as dflash2_select (no temperature: the tree is deterministic). The edge score
 *   is the selector lattice s_i(p, k); for each parent row d_k = fl(s_k - max),
 *   Z = sum_k exp_c(d_k) (k ascending), ls_k = fl(d_k - log_c(Z)) (log_c: a fixed binary32
 *   log by exponent split and a degree-9 odd atanh series). A node's score is fl(parent
 *   score + ls), the root (the anchor) scoring 0. The frontier starts with the root's 16
 *   children (k order); each of `budget` rounds takes the entry with the largest score
 *   (ties: the earliest added), records it and, below depth N, adds its 16 children.
 *   parent, depth, slot, token [B, budget] int32 and score [B, budget] f32, in the order
 *   taken: parent is the tree index of the node's parent (-1 under the root), depth 1..N,
 *   slot the candidate index k, token cand_idx[b, depth-1, k]. Index and finiteness
 *   problems set ST_BADTOKEN / ST_NONFINITE as in dflash2_select (outputs -1, score 0);
 *   status is written. Requires 1 <= budget <= 64. Workspace: dflash2_ddtree_workspace_bytes.
 */
int dflash2_ddtree(const int32_t *cand_idx, const float *cand_val, const float *gate,
                   const uint16_t *pred_cb, const uint16_t *succ_cb, int V, int R,
                   const int32_t *anchor, int B, int N, int budget, int32_t *parent,
                   int32_t *depth, int32_t *slot, int32_t *token, float *score, int32_t *status,
                   void *ws, size_t ws_bytes, hipStream_t stream);
size_t dflash2_ddtree_workspace_bytes(int B, int N);

/*
 * dflash2_select_q8 - dflash2_select over affine-Q8 codebooks ("Geramy/LSE docs/DFLASH2.md",
 * conversion notes: selector codebooks in affine Q8 with groups of 64, BF16 scale and bias,
 * FP32 activations and accumulation).
 *   pred_codes, succ_codes [V, R] uint8; pred_scale, pred_bias, succ_scale, succ_bias
 *   [V, R/64] bf16 bits. Element r of row v is fl(fl(scale[v, r/64] * code[v, r]) +
 *   bias[v, r/64]) in binary32 (scale and bias widened from bf16); lattice, path, outputs
 *   and status are those of dflash2_select with these values in place of the bf16 codebook
 *   entries. Requires R % 64 == 0, R <= 512, 16-byte aligned codes and gate.
 *   Workspace: dflash2_select_workspace_bytes.
 */
int dflash2_select_q8(const int32_t *cand_idx, const float *cand_val, const float *gate,
                      const uint8_t *pred_codes, const uint16_t *pred_scale,
                      const uint16_t *pred_bias, const uint8_t *succ_codes,
                      const uint16_t *succ_scale, const uint16_t *succ_bias, int V, int R,
                      const int32_t *anchor, const float *temperature, uint64_t seed,
                      uint64_t step, int B, int N, int32_t *tokens, int32_t *slot, float *q,
                      int32_t *status, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * dflash2_verify - target verification of the N proposals ("Geramy/LSE docs/DFLASH2.md",
 * usage and drafter-geometry paragraphs: probability-ratio rejection with residual
 * sampling, the target consumes the anchor plus all proposals, greedy keeps the
 * deterministic chain).
 *
 * target rows r = 0..N of sequence b at target[b*seq_stride + r*row_stride + x]; row j-1
 * verifies proposal j and row N follows the last proposal.
 * Greedy (T == 0; target may be bf16 or f32 logits/probabilities): y_j = the first element
 * of row j-1 under the top-16 order; proposals are accepted while tokens[j-1] == y_j, then
 * y at the first mismatch (or the first element of row N) is emitted. A NaN chosen this
 * way sets ST_NONFINITE.
 * Sampled (T > 0; target must be f32 probabilities): proposal j is accepted iff
 * u * q[b,j-1,slot] < p_t(token), u the accept uniform of (b, j). At the first rejection
 * the token is drawn from max(0, p_t - q_j) over the whole vocabulary (q_j is zero off the
 * 16 candidates; the first of duplicated candidates counts); if all N are accepted the
 * bonus token is drawn from row N. Each weight is quantised to floor(w * 2^40); the token
 * is the first x whose running integer sum exceeds floor(word2 * Z / 2^64). Zero residual
 * mass falls back to p_t; zero p_t mass emits the row's first element (ST_ZEROMASS).
 * A proposal outside [0, V) is a rejection; one whose slot/candidate does not match sets
 * ST_BADTOKEN and is rejected with q taken as 0.
 *
 *   tokens, slot [B, N] int32; cand_idx [B, N, 16] int32; q [B, N, 16] f32;
 *   temperature [B] f32; n_accept [B] int32; out_tokens [B, N+1] int32 (accepted proposals,
 *   then the emitted token, then -1); status [B] int32 (OR-ed, not cleared).
 * Requires 1 <= N <= 15, V >= 16, strides >= 0.
 * Workspace: dflash2_verify_workspace_bytes.
 */
int dflash2_verify(const void *target, int dtype, int64_t seq_stride, int64_t row_stride, int V,
                   const int32_t *tokens, const int32_t *cand_idx, const float *q,
                   const int32_t *slot, const float *temperature, uint64_t seed, uint64_t step,
                   int B, int N, int32_t *n_accept, int32_t *out_tokens, int32_t *status,
                   void *ws, size_t ws_bytes, hipStream_t stream);
size_t dflash2_verify_workspace_bytes(int B, int N, int V, int dtype);

/*
 * dflash2_eval_fn - the library's fixed binary32 functions, evaluated elementwise, so that
 * a caller can check them against its own implementation of the same steps. The sampled
 * selector walk forms q with exp_c ("[Spec Decode] DFlash2: local convolution + candidate
 * selector - #52816", PR description: inverse-CDF walk at T > 0 returning q for the
 * lossless verify); the draft tree normalises with exp_c and log_c ("qwen35: DSpark
 * speculative decoding (Qwen3.8-27B drafters) - #625", DDTree commit).
 *   which = 0: out[i] = exp_c(x[i]) for x <= 0: 2^k P7(r) with a two-constant Cody-Waite
 *              reduction and a degree-7 Taylor polynomial in Horner form with fma, every
 *              step one correctly rounded binary32 operation; results under e^-87 are 0
 *   which = 1: out[i] = log_c(x[i]) for finite x > 0: exponent split with the mantissa in
 *              [sqrt(1/2), sqrt(2)), 2 atanh(u) by a degree-9 odd series, same rules
 *   x, out: n f32 (out may not alias x). Inputs outside a function's domain give
 *   unspecified values, not errors. No workspace.
 */
int dflash2_eval_fn(const float *x, float *out, int64_t n, int which, hipStream_t stream);

/* A short English description of a return code or of one status bit. */
const char *dflash2_status_string(int code);

/* Library version as major*10000 + minor*100 + patch. */
int dflash2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH2_H */
