// Letter logits for the letters method ("To Classify, Try a Trie Tree", section
// 3.3).  Every label is one letter token, so the output head needs only the M
// letter rows (section 4.1, V_out = M): each document's answer-position hidden
// state is dotted with those rows and nothing else.  The label softmax and argmax
// then run on these logits as they are; the vocabulary log-sum-exp would cancel in
// the rescale over the letters, so it is never formed.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tcs_device.h"
#include "tcs_internal.h"

namespace tcs {
namespace {

// One wave per letter: child c = 1 + 4 blockIdx.x + wave of the root.  The wave
// walks documents b = blockIdx.y, blockIdx.y + gridDim.y, ... and writes
// lp[b][c] = h[b's root row] . W[token[c]] (times the row scale for fp8 W), the
// fp32 partial products summed over the wave.
template <int WK>
__global__ __launch_bounds__(256) void letter_logits_kernel(
    int B, int n_int, int n_nodes, int d, const void* __restrict__ h, const void* __restrict__ W,
    const float* __restrict__ w_scale, const int32_t* __restrict__ token, float* __restrict__ lp) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = 1 + int(blockIdx.x) * 4 + wave;
  if (c >= n_nodes) return;  // whole wave
  const int tok = token[c];
  const float sc = WK == 2 ? w_scale[tok] : 1.0f;
  const size_t es = WK == 0 ? 4 : 2;
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    // row 0 of document b is the root's
    const void* hr = static_cast<const char*>(h) + size_t(b) * n_int * d * es;
    const float acc = wave_sum(head_row_dot_lane<WK>(hr, W, tok, d, lane));
    if (lane == 0) {
      lp[size_t(b) * n_nodes + c] = acc * sc;
      if (c == 1) lp[size_t(b) * n_nodes] = 0.f;  // the root has no edge
    }
  }
}

}  // namespace

int launch_letter_logits(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                         int32_t n_int, int32_t n_nodes, int32_t d, const void* h, const void* W,
                         const float* w_scale, const int32_t* token, float* lp) {
  if (B <= 0 || n_nodes < 2) return TCS_OK;
  if (h_dtype != TCS_F32 && d % 4 != 0)
    return fail(TCS_EUNSUPPORTED, "letters: d=%d is not a multiple of 4", d);
  const dim3 grid((n_nodes - 1 + 3) / 4, std::min(B, 65535));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (h_dtype == TCS_F32 && w_dtype == TCS_F32)
    letter_logits_kernel<0><<<grid, 256, 0, s>>>(B, n_int, n_nodes, d, h, W, w_scale, token, lp);
  else if (h_dtype == TCS_BF16 && w_dtype == TCS_BF16)
    letter_logits_kernel<1><<<grid, 256, 0, s>>>(B, n_int, n_nodes, d, h, W, w_scale, token, lp);
  else if (h_dtype == TCS_BF16 && w_dtype == TCS_FP8_E4M3)
    letter_logits_kernel<2><<<grid, 256, 0, s>>>(B, n_int, n_nodes, d, h, W, w_scale, token, lp);
  else
    return fail(TCS_EUNSUPPORTED, "letters: h dtype %d with head dtype %d", int(h_dtype),
                int(w_dtype));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "letter_logits: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
