// Greedy decoding inside the label trie: trie_decode of "To Classify, Try a Trie
// Tree", section 3.1.  Every document starts at the root (the ANSWER: token); the
// model runs only where labels branch, one answer position per undecided document
// per step, and picks the child whose token has the highest logit; nodes with one
// child are passed without a run, and a document stops once one label remains
// below it.  These kernels keep the per-document state on the device: the steps
// of a batch run back to back on one stream with no host round trip.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "tcs_device.h"
#include "tcs_internal.h"

namespace tcs {
namespace {

// Every document starts at w0 = dec_node[root]: decided at once when one label
// remains there (label written, no run), else slot b = document b at w0.  All B
// slots get valid entries, so kernels that read slots past *n_sel see real ids.
__global__ void decode_init_kernel(int B, const int32_t* __restrict__ dec_node,
                                   const int32_t* __restrict__ sub_label,
                                   const int32_t* __restrict__ qrow, int32_t* __restrict__ cur,
                                   int32_t* __restrict__ label, int32_t* __restrict__ runs,
                                   int32_t* __restrict__ sel, int32_t* __restrict__ row_node,
                                   int32_t* __restrict__ n_sel) {
  const int w0 = dec_node[0];
  const int lab = sub_label[w0];
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b == 0) *n_sel = lab >= 0 ? 0 : B;
  if (b >= B) return;
  cur[b] = lab >= 0 ? -1 : w0;
  label[b] = lab;
  if (runs) runs[b] = 0;
  sel[2 * b] = b;
  sel[2 * b + 1] = lab >= 0 ? 0 : qrow[w0];
  row_node[b] = w0;
}

// One workgroup per slot a < *n_sel: the hidden state h[a] at node u = row_node[a]
// against the head rows of u's children (one wave per child in turn), the
// highest logit wins (lowest child index, i.e. lowest token id, on ties); then the
// document moves to dec_node[child] and is decided if one label remains there.
template <int WK>
__global__ __launch_bounds__(256) void decode_step_kernel(
    int d, const void* __restrict__ h, const void* __restrict__ W,
    const float* __restrict__ w_scale, const int32_t* __restrict__ token,
    const int32_t* __restrict__ child_begin, const int32_t* __restrict__ child_count,
    const int32_t* __restrict__ dec_node, const int32_t* __restrict__ sub_label,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ row_node,
    const int32_t* __restrict__ n_sel, int32_t* __restrict__ cur, int32_t* __restrict__ label,
    int32_t* __restrict__ runs) {
  __shared__ float bz[4];
  __shared__ int bi[4];
  const int a = blockIdx.x;
  if (a >= *n_sel) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int doc = sel[2 * a], u = row_node[a];
  const int c0 = child_begin[u], nc = child_count[u];
  const void* hr = static_cast<const char*>(h) + size_t(a) * d * (WK == 0 ? 4 : 2);
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int i = wave; i < nc; i += 4) {
    const int tok = token[c0 + i];
    float z = wave_sum(head_row_dot_lane<WK>(hr, W, tok, d, lane));
    if (WK == 2) z *= w_scale[tok];
    if (z > best || bidx == 0x7fffffff) {  // i grows, so ties keep the first
      best = z;
      bidx = i;
    }
  }
  if (lane == 0) {
    bz[wave] = best;
    bi[wave] = bidx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float z = bz[0];
    int i = bi[0];
    for (int w = 1; w < 4; ++w)
      if (bi[w] != 0x7fffffff && (bz[w] > z || (bz[w] == z && bi[w] < i) || i == 0x7fffffff)) {
        z = bz[w];
        i = bi[w];
      }
    if (i == 0x7fffffff) {  // no child: cannot happen for a node the tables mark undecided
      label[doc] = -1;
      cur[doc] = -1;
      return;
    }
    const int v = dec_node[c0 + i];
    const int lab = sub_label[v];
    if (runs) ++runs[doc];
    label[doc] = lab;
    cur[doc] = lab >= 0 ? -1 : v;
  }
}

// The next step's slots: the undecided documents in document order (one
// workgroup, blocks of 1024 documents, a ballot prefix count per wave).
__global__ __launch_bounds__(1024) void decode_compact_kernel(int B, const int32_t* __restrict__ cur,
                                                             const int32_t* __restrict__ qrow,
                                                             int32_t* __restrict__ sel,
                                                             int32_t* __restrict__ row_node,
                                                             int32_t* __restrict__ n_sel) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 1024) {
    const int b = b0 + tid;
    const int u = b < B ? cur[b] : -1;
    const bool act = u >= 0;
    const uint64_t m = __ballot(act);
    const int before = __popcll(m & ((uint64_t(1) << lane) - 1));
    if (lane == 0) wsum[wave] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    int total = 0;
    for (int w = 0; w < 16; ++w) total += wsum[w];
    if (act) {
      const int k = off + before;
      sel[2 * k] = b;
      sel[2 * k + 1] = qrow[u];
      row_node[k] = u;
    }
    base += total;
    __syncthreads();  // wsum is rewritten by the next block of documents
  }
  if (tid == 0) *n_sel = base;
}

}  // namespace

int launch_decode_init(void* stream, int32_t B, const int32_t* dec_node, const int32_t* sub_label,
                       const int32_t* qrow, int32_t* cur, int32_t* label, int32_t* runs,
                       int32_t* sel, int32_t* row_node, int32_t* n_sel) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  decode_init_kernel<<<(B + 255) / 256, 256, 0, s>>>(B, dec_node, sub_label, qrow, cur, label, runs,
                                                      sel, row_node, n_sel);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_init: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_decode_step(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t d,
                       const void* h, const void* W, const float* w_scale, const int32_t* token,
                       const int32_t* child_begin, const int32_t* child_count,
                       const int32_t* dec_node, const int32_t* sub_label, const int32_t* sel,
                       const int32_t* row_node, const int32_t* n_sel, int32_t* cur, int32_t* label,
                       int32_t* runs) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  if (h_dtype != TCS_F32 && d % 4 != 0)
    return fail(TCS_EUNSUPPORTED, "decode: d=%d is not a multiple of 4", d);
#define TCS_STEP(WK)                                                                             \
  decode_step_kernel<WK><<<B, 256, 0, s>>>(d, h, W, w_scale, token, child_begin, child_count,   \
                                           dec_node, sub_label, sel, row_node, n_sel, cur, label, \
                                           runs)
  if (h_dtype == TCS_F32 && w_dtype == TCS_F32)
    TCS_STEP(0);
  else if (h_dtype == TCS_BF16 && w_dtype == TCS_BF16)
    TCS_STEP(1);
  else if (h_dtype == TCS_BF16 && w_dtype == TCS_FP8_E4M3)
    TCS_STEP(2);
  else
    return fail(TCS_EUNSUPPORTED, "decode: h dtype %d with head dtype %d", int(h_dtype),
                int(w_dtype));
#undef TCS_STEP
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_step: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_decode_compact(void* stream, int32_t B, const int32_t* cur, const int32_t* qrow,
                          int32_t* sel, int32_t* row_node, int32_t* n_sel) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  decode_compact_kernel<<<1, 1024, 0, s>>>(B, cur, qrow, sel, row_node, n_sel);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_compact: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
