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
                                   int32_t* __restrict__ n_sel,
                                   unsigned long long* __restrict__ best_key) {
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
  best_key[b] = 0;
}

// Order-preserving key of (logit, child index): a larger logit wins, then the
// lower index (lowest token id on ties).
__device__ __forceinline__ unsigned long long pick_key(float z, int i) {
  const uint32_t u = __float_as_uint(z);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(o) << 32) | (0xFFFFFFFFu - uint32_t(i));
}

// Workgroup (a, y) for slot a < *n_sel scores children y*CH .. y*CH+CH-1 of the
// slot's node u = row_node[a] (one wave per child in turn).  It first forms the
// slot's hidden state in LDS from the projection's fp32 partials: y = their sum
// (in partial order), h = y / sqrt(mean(y^2) + eps), stored as the model dtype
// (bf16: nearest-even), as the RMSNorm of the classify pass does.  Then h against
// the children's head rows; each workgroup folds its best (logit, child) into the
// slot's key with a 64-bit atomic max, and the next launch reads the keys.
constexpr int STEP_CH = 32;  // children per workgroup: 8 per wave
template <int WK>
__global__ __launch_bounds__(256) void decode_logits_kernel(
    int B, int d, int n_part, float eps, const float* __restrict__ y, const void* __restrict__ W,
    const float* __restrict__ w_scale, const int32_t* __restrict__ token,
    const int32_t* __restrict__ child_begin, const int32_t* __restrict__ child_count,
    const int32_t* __restrict__ row_node, const int32_t* __restrict__ n_sel,
    unsigned long long* __restrict__ best_key) {
  extern __shared__ __attribute__((aligned(16))) float ys[];  // [d] fp32, then h [d]
  __shared__ unsigned long long bk[4];
  __shared__ float red[4];
  const int a = blockIdx.x;
  if (a >= *n_sel) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float ss = 0.f;
  for (int k = tid; k < d; k += 256) {
    float v = y[size_t(a) * d + k];
    for (int p = 1; p < n_part; ++p) v += y[(size_t(p) * B + a) * d + k];
    ys[k] = v;
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / float(d) + eps);
  void* hr = ys + d;
  for (int k = tid; k < d; k += 256) {
    if constexpr (WK == 0) static_cast<float*>(hr)[k] = ys[k] * rs;
    else static_cast<uint16_t*>(hr)[k] = f32_to_bf16(ys[k] * rs);
  }
  __syncthreads();
  const int u = row_node[a];
  const int c0 = child_begin[u], nc = child_count[u];
  unsigned long long key = 0;  // below every real key
  const int i_end = min(nc, int(blockIdx.y + 1) * STEP_CH);
  for (int i = int(blockIdx.y) * STEP_CH + wave; i < i_end; i += 4) {
    const int tok = token[c0 + i];
    float z = wave_sum(head_row_dot_lane<WK>(hr, W, tok, d, lane));
    if (WK == 2) z *= w_scale[tok];
    key = max(key, pick_key(z, i));
  }
  if (lane == 0) bk[wave] = key;
  __syncthreads();
  if (threadIdx.x == 0) {
    key = max(max(bk[0], bk[1]), max(bk[2], bk[3]));
    if (key) atomicMax(best_key + a, key);
  }
}

// One workgroup.  First every slot a < *n_sel takes its best child (and clears
// its key): the document moves to dec_node[child] and is decided if one label
// remains there.  Then the next step's slots are the undecided documents in
// document order (blocks of 1024 documents, a ballot prefix count per wave).
__global__ __launch_bounds__(1024) void decode_advance_kernel(
    int B, const int32_t* __restrict__ child_begin, const int32_t* __restrict__ dec_node,
    const int32_t* __restrict__ sub_label, const int32_t* __restrict__ qrow,
    unsigned long long* __restrict__ best_key, int32_t* __restrict__ cur,
    int32_t* __restrict__ label, int32_t* __restrict__ runs, int32_t* __restrict__ sel,
    int32_t* __restrict__ row_node, int32_t* __restrict__ n_sel) {
  __shared__ int wsum[16];
  const int n_old = *n_sel;
  if (n_old == 0) return;  // every document decided: nothing changes
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int a = tid; a < n_old; a += 1024) {
    const unsigned long long key = best_key[a];
    best_key[a] = 0;
    const int doc = sel[2 * a];
    if (runs) ++runs[doc];
    if (key == 0) {  // no child: cannot happen for a node the tables mark undecided
      label[doc] = -1;
      cur[doc] = -1;
      continue;
    }
    const int i = int(0xFFFFFFFFu - uint32_t(key));
    const int v = dec_node[child_begin[row_node[a]] + i];
    const int lab = sub_label[v];
    label[doc] = lab;
    cur[doc] = lab >= 0 ? -1 : v;
  }
  __syncthreads();  // the documents' new states are in before they are gathered
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
                       int32_t* sel, int32_t* row_node, int32_t* n_sel,
                       unsigned long long* best_key) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  decode_init_kernel<<<(B + 255) / 256, 256, 0, s>>>(B, dec_node, sub_label, qrow, cur, label, runs,
                                                      sel, row_node, n_sel, best_key);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_init: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_decode_logits(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                         int32_t d, int32_t n_part, float eps, const float* y, const void* W,
                         const float* w_scale,
                         const int32_t* token, const int32_t* child_begin,
                         const int32_t* child_count, const int32_t* row_node, const int32_t* n_sel,
                         int32_t max_children, unsigned long long* best_key) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  if (h_dtype != TCS_F32 && d % 4 != 0)
    return fail(TCS_EUNSUPPORTED, "decode: d=%d is not a multiple of 4", d);
  if (max_children < 1) return fail(TCS_EINVAL, "decode: max_children %d", max_children);
  const dim3 grid(B, (max_children + STEP_CH - 1) / STEP_CH);
  if (grid.y > 65535) return fail(TCS_EUNSUPPORTED, "decode: %d children", max_children);
  const size_t lds = size_t(d) * (4 + (h_dtype == TCS_F32 ? 4 : 2));
  if (lds > 64 * 1024) return fail(TCS_EUNSUPPORTED, "decode: d=%d too wide", d);
#define TCS_STEP(WK)                                                                           \
  decode_logits_kernel<WK><<<grid, 256, lds, s>>>(B, d, n_part, eps, y, W, w_scale, token,     \
                                                  child_begin, child_count, row_node, n_sel,   \
                                                  best_key)
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
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_logits: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_decode_advance(void* stream, int32_t B, const int32_t* child_begin,
                          const int32_t* dec_node, const int32_t* sub_label, const int32_t* qrow,
                          unsigned long long* best_key, int32_t* cur, int32_t* label,
                          int32_t* runs, int32_t* sel, int32_t* row_node, int32_t* n_sel) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B < 1) return TCS_OK;
  decode_advance_kernel<<<1, 1024, 0, s>>>(B, child_begin, dec_node, sub_label, qrow, best_key, cur,
                                           label, runs, sel, row_node, n_sel);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "decode_advance: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
