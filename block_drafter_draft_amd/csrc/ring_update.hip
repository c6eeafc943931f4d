// dflash2_ring_update: keeps a drafter context ring in step with the committed sequence
// after a verify step ("Geramy/LSE docs/DFLASH2.md", native-test notes: cache rewind,
// replacement and reset). Position p of a sequence lives in ring slot p mod S, so the ring
// holds the last S committed positions and block attention reads the window from it.
//
// One workgroup per sequence: every thread reads the sequence's context length, rewind
// and count; the rewind (or reset) is applied, the new rows are copied into their slots in
// 16-byte pieces, and thread 0 writes the new context length after a barrier (so no thread
// can read the updated value). The call moves 2 * n * Hkv * D elements per sequence and is
// bound by launch latency.
#include "common.hpp"

namespace df2 {
namespace {

constexpr int kRingThreads = 256;
constexpr int kMaxNew = 16;

__global__ __launch_bounds__(kRingThreads) void ring_update_kernel(
    const u32x4_t* __restrict__ new_k, const u32x4_t* __restrict__ new_v,
    const int32_t* __restrict__ n_new, const int32_t* __restrict__ back,
    int32_t* __restrict__ ctx_len, u32x4_t* __restrict__ k_ring, u32x4_t* __restrict__ v_ring,
    int Pn, int pieces, int S, int W, int32_t* __restrict__ status) {
  const int b = blockIdx.x, t = threadIdx.x;
  const int L0 = ctx_len[b], bk = back[b], nn = n_new[b];
  int st = 0;
  const int L = L0 < 0 ? 0 : L0;
  int Lr;
  if (bk < 0) {
    Lr = 0;  // reset
  } else {
    const int r = bk < L ? bk : L;
    Lr = L - r;
    // positions the next window needs, against those the ring still holds
    const int need_lo = Lr - W + 1 > 0 ? Lr - W + 1 : 0;
    const int have_lo = L - S > 0 ? L - S : 0;
    if (need_lo < Lr && need_lo < have_lo) st |= DFLASH2_ST_RINGLOST;
  }
  int n = nn;
  if (n < 0 || n > Pn) {
    st |= DFLASH2_ST_BADCOUNT;
    n = n < 0 ? 0 : Pn;
  }
  const u32x4_t* sk = new_k + (int64_t)b * Pn * pieces;
  const u32x4_t* sv = new_v + (int64_t)b * Pn * pieces;
  u32x4_t* dk = k_ring + (int64_t)b * S * pieces;
  u32x4_t* dv = v_ring + (int64_t)b * S * pieces;
  for (int e = t; e < n * pieces; e += kRingThreads) {
    const int j = e / pieces, c = e - j * pieces;
    const int slot = (Lr + j) % S;
    const u32x4_t a = sk[(int64_t)j * pieces + c], v = sv[(int64_t)j * pieces + c];
    dk[(int64_t)slot * pieces + c] = a;
    dv[(int64_t)slot * pieces + c] = v;
  }
  __syncthreads();  // every thread has read ctx_len[b]
  if (t == 0) {
    ctx_len[b] = Lr + n;
    if (st) status[b] |= st;
  }
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" int dflash2_ring_update(const void* new_k, const void* new_v, const int32_t* n_new,
                                   const int32_t* back, int32_t* ctx_len, void* k_ring,
                                   void* v_ring, int B, int Pn, int Hkv, int D, int S, int W,
                                   int dtype, int32_t* status, hipStream_t stream) {
  if (!new_k || !new_v || !n_new || !back || !ctx_len || !k_ring || !v_ring || !status)
    return DFLASH2_EINVAL;
  if (B < 1 || Pn < 1 || Hkv < 1 || D < 1 || W < 1 || S < W - 1 || S < 1) return DFLASH2_EINVAL;
  if (dtype != DFLASH2_BF16 && dtype != DFLASH2_F32) return DFLASH2_EUNSUPPORTED;
  if (Pn > kMaxNew || S < Pn || B > 65535) return DFLASH2_EUNSUPPORTED;
  const int64_t row_bytes = (int64_t)Hkv * D * (dtype == DFLASH2_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || row_bytes / 16 > (1 << 20)) return DFLASH2_EUNSUPPORTED;
  for (const void* p : {new_k, new_v, (const void*)k_ring, (const void*)v_ring})
    if (!aligned(p, 16)) return DFLASH2_EUNSUPPORTED;
  ring_update_kernel<<<B, kRingThreads, 0, stream>>>(
      (const u32x4_t*)new_k, (const u32x4_t*)new_v, n_new, back, ctx_len, (u32x4_t*)k_ring,
      (u32x4_t*)v_ring, Pn, (int)(row_bytes / 16), S, W, status);
  return launch_status();
}
