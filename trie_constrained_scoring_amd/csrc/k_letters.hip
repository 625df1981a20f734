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
// fp32 partial products summed over the wave.  bf16 hidden states: each lane takes
// 4 consecutive elements per step (d % 4 == 0, so every row is 8-byte aligned).
// WK: 0 = fp32 h and W, 1 = bf16 h and W, 2 = bf16 h and E4M3 W.
template <int WK>
__global__ __launch_bounds__(256) void letter_logits_kernel(
    int B, int n_int, int n_nodes, int d, const void* __restrict__ h, const void* __restrict__ W,
    const float* __restrict__ w_scale, const int32_t* __restrict__ token, float* __restrict__ lp) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = 1 + int(blockIdx.x) * 4 + wave;
  if (c >= n_nodes) return;  // whole wave
  const int tok = token[c];
  const float sc = WK == 2 ? w_scale[tok] : 1.0f;
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    const size_t hrow = size_t(b) * n_int * d;  // row 0 of document b is the root's
    float acc = 0.f;
    if constexpr (WK == 0) {
      const float* hr = static_cast<const float*>(h) + hrow;
      const float* wr = static_cast<const float*>(W) + size_t(tok) * d;
      for (int k = lane; k < d; k += 64) acc = fmaf(hr[k], wr[k], acc);
    } else {
      const uint2* hr = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(h) + hrow);
      for (int k4 = lane; k4 < d / 4; k4 += 64) {
        const uint2 hv = hr[k4];
        float w[4];
        if constexpr (WK == 1) {
          const uint2 wv = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) +
                                                          size_t(tok) * d)[k4];
          w[0] = bf16_to_f32(uint16_t(wv.x));
          w[1] = bf16_to_f32(uint16_t(wv.x >> 16));
          w[2] = bf16_to_f32(uint16_t(wv.y));
          w[3] = bf16_to_f32(uint16_t(wv.y >> 16));
        } else {
          // four E4M3 codes -> bf16 (hardware conversion at scale 1, exact)
          const uint32_t wv = reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(W) +
                                                                size_t(tok) * d)[k4];
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv, 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wv, 1.0f, true);
          w[0] = float(lo[0]);
          w[1] = float(lo[1]);
          w[2] = float(hi[0]);
          w[3] = float(hi[1]);
        }
        acc = fmaf(bf16_to_f32(uint16_t(hv.x)), w[0], acc);
        acc = fmaf(bf16_to_f32(uint16_t(hv.x >> 16)), w[1], acc);
        acc = fmaf(bf16_to_f32(uint16_t(hv.y)), w[2], acc);
        acc = fmaf(bf16_to_f32(uint16_t(hv.y >> 16)), w[3], acc);
      }
    }
    acc = wave_sum(acc);
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
