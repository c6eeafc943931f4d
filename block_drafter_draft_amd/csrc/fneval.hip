// dflash2_eval_fn: the library's fixed binary32 exp and log, evaluated elementwise. The
// sampled selector walk turns a slot's scores into q over the 16 candidates with exp_c
// ("[Spec Decode] DFlash2: local convolution + candidate selector - #52816", PR
// description: at T > 0 the path is walked by inverse CDF and q is returned for the
// lossless verify), and the draft tree normalises each parent row with exp_c and log_c
// ("qwen35: DSpark speculative decoding (Qwen3.8-27B drafters) - #625", DDTree commit:
// per-position log-softmax). Both are defined step by step (common.hpp), so any IEEE
// implementation of the same steps agrees bit for bit; this call lets a caller check that.
#include "common.hpp"

namespace df2 {
namespace {

// grid-stride over n elements; 8 per thread per pass, all loads issued first
__global__ __launch_bounds__(256) void eval_fn_kernel(const float* __restrict__ x,
                                                      float* __restrict__ out, int64_t n,
                                                      int which) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 8;
  for (int64_t base = (int64_t)blockIdx.x * 256 * 8 + threadIdx.x; base < n; base += stride) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t e = base + 256 * u;
      v[u] = e < n ? x[e] : 1.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t e = base + 256 * u;
      if (e < n) out[e] = which == 0 ? exp_c(v[u]) : log_c(v[u]);
    }
  }
}

}  // namespace
}  // namespace df2

using namespace df2;

extern "C" int dflash2_eval_fn(const float* x, float* out, int64_t n, int which,
                               hipStream_t stream) {
  if (!x || !out || n < 0) return DFLASH2_EINVAL;
  if (which != 0 && which != 1) return DFLASH2_EUNSUPPORTED;
  if (n == 0) return DFLASH2_OK;
  const int64_t per_block = 256 * 8;
  int64_t blocks = (n + per_block - 1) / per_block;
  blocks = blocks < 4096 ? blocks : 4096;
  eval_fn_kernel<<<(unsigned)blocks, 256, 0, stream>>>(x, out, n, which);
  return launch_status();
}
