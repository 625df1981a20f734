// Per-label path sums, label softmax and argmax.
//
// "To Classify, Try a Trie Tree", section 3.2: a label's score is the product of
// its token probabilities, so its log score is the sum of the edge log-probs on
// its root-to-label path; a label that ends where other labels continue is also
// multiplied by the probability of not continuing; scores are divided by their
// sum over labels.  Section 2: the operator always returns one label.
#include <cfloat>
#include <climits>

#include "tcs_device.h"
#include "tcs_internal.h"

namespace tcs {

__device__ __forceinline__ double log1mexp_d(double x) {
  if (x >= 0.0) return -HUGE_VAL;
  return x > -0.6931471805599453 ? log(-expm1(x)) : log1p(-exp(x));
}

// node_qrow[v] = the query row of v's parent (v's edge), from the edge arrays.
__global__ void node_qrow_kernel(int n_edges, const int32_t* __restrict__ e_child,
                                 const int32_t* __restrict__ e_qrow, int32_t* __restrict__ node_qrow) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < n_edges) node_qrow[e_child[e]] = e_qrow[e];
}

// One workgroup per document; each thread walks the paths of its labels from the
// label node up to the root (depths are small), accumulating in fp64.  With `lse`
// set, lp holds the raw child logits and the edge log-prob of node v is
// lp[v] - lse[b n_int + node_qrow[v]] (the head's finalisation folded in).
__global__ __launch_bounds__(256) void path_sum_kernel(
    int n_nodes, int M, const float* __restrict__ lp, const float* __restrict__ lse,
    const int32_t* __restrict__ node_qrow, int n_int, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ child_begin, const int32_t* __restrict__ child_count,
    const int32_t* __restrict__ label_node, float* __restrict__ ll, float* __restrict__ prob,
    int32_t* __restrict__ label) {
  __shared__ double rv[4];
  __shared__ int ri[4];
  __shared__ double rs[4];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* lpb = lp + (size_t)b * n_nodes;
  const float* lseb = lse ? lse + (size_t)b * n_int : nullptr;
  auto edge_lp = [&](int v) -> double {
    const double x = double(lpb[v]);
    return lseb ? x - double(lseb[node_qrow[v]]) : x;
  };
  float* llb = ll + (size_t)b * M;
  double best = -HUGE_VAL;
  int best_i = INT_MAX;
  for (int m = t; m < M; m += 256) {
    const int u = label_node[m];
    double acc = 0.0;
    for (int v = u, steps = 0; v > 0 && steps < u; v = parent[v], ++steps) acc += edge_lp(v);
    const int cc = child_count[u];
    if (cc > 0) {
      const int cb = child_begin[u];
      double mx = -HUGE_VAL;
      for (int c = cb; c < cb + cc; ++c) mx = fmax(mx, edge_lp(c));
      double se = 0.0;
      for (int c = cb; c < cb + cc; ++c) se += exp(edge_lp(c) - mx);
      acc += log1mexp_d(mx + log(se));
    }
    llb[m] = float(acc);
    if (acc > best || (acc == best && m < best_i)) {
      best = acc;
      best_i = m;
    }
  }
  // argmax over the workgroup, lowest label id among equal maxima
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(best_i, o, 64);
    if (ov > best || (ov == best && oi < best_i)) {
      best = ov;
      best_i = oi;
    }
  }
  if (lane == 0) {
    rv[wave] = best;
    ri[wave] = best_i;
  }
  __syncthreads();
  best = rv[0];
  best_i = ri[0];
  for (int w = 1; w < 4; ++w)
    if (rv[w] > best || (rv[w] == best && ri[w] < best_i)) {
      best = rv[w];
      best_i = ri[w];
    }
  if (t == 0) label[b] = best_i;
  if (!prob) return;
  double s = 0.0;
  for (int m = t; m < M; m += 256) s += exp(double(llb[m]) - best);
  s = wave_sum_d(s);
  if (lane == 0) rs[wave] = s;
  __syncthreads();
  s = rs[0] + rs[1] + rs[2] + rs[3];
  const double inv = 1.0 / s;
  float* pb = prob + (size_t)b * M;
  for (int m = t; m < M; m += 256) pb[m] = float(exp(double(llb[m]) - best) * inv);
}

int launch_node_qrow(void* stream, const tcs_trie_dev* trie, int32_t* node_qrow) {
  const int n_edges = trie->n_nodes - 1;
  if (n_edges <= 0) return TCS_OK;
  node_qrow_kernel<<<(n_edges + 255) / 256, 256, 0, static_cast<hipStream_t>(stream)>>>(
      n_edges, trie->e_child, trie->e_qrow, node_qrow);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "node_qrow: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_path_sum(void* stream, int32_t B, const tcs_trie_dev* trie, const float* lp, float* ll,
                    float* prob, int32_t* label, const float* lse, const int32_t* node_qrow) {
  if (B <= 0) return TCS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  path_sum_kernel<<<B, 256, 0, s>>>(trie->n_nodes, trie->n_labels, lp, lse, node_qrow, trie->n_int,
                                    trie->parent, trie->child_begin, trie->child_count,
                                    trie->label_node, ll, prob, label);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "path_sum: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
