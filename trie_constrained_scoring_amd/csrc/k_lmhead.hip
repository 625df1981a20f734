// Full-vocabulary output head with fused log-sum-exp and child-token gather.
//
// "To Classify, Try a Trie Tree", section 4.1: turning label scores into
// probabilities needs every vocabulary row at every answer position
// (F_head = 2 d V per position).  The [rows x V] logits are never written: each
// workgroup reduces its 256-column tile to a per-row (max, sum exp) partial while
// the logits are still in the matrix-core accumulators, and the few logits that
// belong to trie edges are copied out of those registers by the lane that holds
// them.  A finalize pass merges the partials into lse and turns the gathered
// logits into token log-probabilities.
#include <cstdio>

#include "gemm_core.h"
#include "tcs_internal.h"

namespace tcs {

constexpr int HEAD_BN = 256;  // columns per tile: also the partial granularity

__device__ __forceinline__ int lower_bound_i32(const int32_t* __restrict__ a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// R rows (document b, query row q) = b * n_int + q; 256 x 256 tiles, 4 waves.
template <bool FP8>
__global__ __launch_bounds__(256, 1) void lmhead_bf16_kernel(
    int R, int V, int d, int n_int, int n_nodes, const uint16_t* __restrict__ h,
    const void* __restrict__ W, const float* __restrict__ w_scale, const int32_t* __restrict__ e_tok,
    const int32_t* __restrict__ e_qrow, const int32_t* __restrict__ e_child, int n_edges,
    float* __restrict__ raw, float2* __restrict__ part) {
  constexpr int BM = 256, BN = HEAD_BN, WM = 2, WN = 2;
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];
  const int nbm = (R + BM - 1) / BM, nbn = (V + BN - 1) / BN;
  int mt, nt;
  tile_coords<8>(nbm, nbn, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x4 acc[S::MB][S::NB];
  gemm_mainloop<BM, BN, WM, WN, FP8>(h, d, W, d, R, V, d, m0, n0, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int col_base = n0 + wn * S::TN + (lane & 15);
  const int row_base = m0 + wm * S::TM + (lane >> 4) * 4;

  // fp8 row scale, and columns past V drop out of the reduction
#pragma unroll
  for (int j = 0; j < S::NB; ++j) {
    const int col = col_base + j * 16;
    const bool ok = col < V;
    const float sc = (FP8 && ok) ? w_scale[col] : 1.0f;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = ok ? acc[i][j][r] * sc : -INFINITY;
  }

  // child-token gather: edges are sorted by token, so this tile's edges are one
  // contiguous range; the lane holding column e_tok copies the logit of every row
  // whose query row is e_qrow.
  const int e_lo = lower_bound_i32(e_tok, n_edges, n0);
  const int e_hi = lower_bound_i32(e_tok, n_edges, n0 + BN);
  if (e_lo < e_hi) {
#pragma unroll
    for (int j = 0; j < S::NB; ++j) {
      const int col = col_base + j * 16;
      for (int e = e_lo; e < e_hi; ++e) {
        if (e_tok[e] != col) continue;
        const int q = e_qrow[e], c = e_child[e];
#pragma unroll
        for (int i = 0; i < S::MB; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row_base + i * 16 + r;
            if (row < R && row % n_int == q) raw[(size_t)(row / n_int) * n_nodes + c] = acc[i][j][r];
          }
      }
    }
  }

  // per-row max and sum of exp over this wave's 128 columns (16 lanes share a row)
  float2* red = reinterpret_cast<float2*>(lds);  // [WN][BM]
#pragma unroll
  for (int i = 0; i < S::MB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float m = acc[i][0][r];
#pragma unroll
      for (int j = 1; j < S::NB; ++j) m = fmaxf(m, acc[i][j][r]);
      m = max16(m);
      float s = 0.f;
      if (m != -INFINITY) {
#pragma unroll
        for (int j = 0; j < S::NB; ++j) s += __expf(acc[i][j][r] - m);
      }
      s = sum16(s);
      if ((lane & 15) == 0) red[wn * BM + wm * S::TM + i * 16 + (lane >> 4) * 4 + r] = float2{m, s};
    }
  __syncthreads();
  {
    const int t = threadIdx.x;  // one row per thread (BM == 256 threads)
    float2 a = red[t], b = red[BM + t];
    lse_merge(a.x, a.y, b.x, b.y);
    if (m0 + t < R) part[(size_t)nt * R + m0 + t] = a;
  }
}

// fp32 head: one thread per column of a 256-column tile, 8 rows per block.
__global__ __launch_bounds__(256) void lmhead_f32_kernel(
    int R, int V, int d, int n_int, int n_nodes, const float* __restrict__ h,
    const float* __restrict__ W, const int32_t* __restrict__ e_tok,
    const int32_t* __restrict__ e_qrow, const int32_t* __restrict__ e_child, int n_edges,
    float* __restrict__ raw, float2* __restrict__ part) {
  constexpr int RB = 8, KC = 256;
  __shared__ float sh[RB][KC];
  __shared__ float2 red[4][RB];
  const int nt = blockIdx.x, n0 = nt * HEAD_BN;
  const int r0 = blockIdx.y * RB;
  const int t = threadIdx.x, col = n0 + t;
  const bool ok = col < V;
  float acc[RB] = {};
  for (int k0 = 0; k0 < d; k0 += KC) {
    for (int e = t; e < RB * KC; e += 256) {
      const int i = e / KC, k = e % KC;
      sh[i][k] = (r0 + i < R && k0 + k < d) ? h[(size_t)(r0 + i) * d + k0 + k] : 0.f;
    }
    __syncthreads();
    if (ok) {
      const int kend = min(KC, d - k0);
      for (int k = 0; k < kend; ++k) {
        const float w = W[(size_t)col * d + k0 + k];
#pragma unroll
        for (int i = 0; i < RB; ++i) acc[i] = fmaf(sh[i][k], w, acc[i]);
      }
    }
    __syncthreads();
  }
  const int e_lo = lower_bound_i32(e_tok, n_edges, n0);
  const int e_hi = lower_bound_i32(e_tok, n_edges, n0 + HEAD_BN);
  for (int e = e_lo; e < e_hi; ++e) {
    if (e_tok[e] != col) continue;
    const int q = e_qrow[e], c = e_child[e];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int row = r0 + i;
      if (row < R && row % n_int == q) raw[(size_t)(row / n_int) * n_nodes + c] = acc[i];
    }
  }
  const int lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const float v = ok ? acc[i] : -INFINITY;
    const float m = wave_max(v);
    const float s = wave_sum(m == -INFINITY ? 0.f : __expf(v - m));
    if (lane == 0) red[wave][i] = float2{m, s};
  }
  __syncthreads();
  if (t < RB && r0 + t < R) {
    float m = red[0][t].x, s = red[0][t].y;
    for (int w = 1; w < 4; ++w) lse_merge(m, s, red[w][t].x, red[w][t].y);
    part[(size_t)nt * R + r0 + t] = float2{m, s};
  }
}

__global__ void lse_finalize_kernel(int R, int n_tiles, const float2* __restrict__ part,
                                    float* __restrict__ lse) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  float m = -INFINITY, s = 0.f;
  for (int t = 0; t < n_tiles; ++t) {
    const float2 p = part[(size_t)t * R + r];
    lse_merge(m, s, p.x, p.y);
  }
  lse[r] = m + logf(s);
}

// lp[b, c] = logit - lse[row of the edge's parent]; lp[b, root] = 0.
__global__ void lp_finalize_kernel(int B, int n_int, int n_nodes, const int32_t* __restrict__ e_qrow,
                                   const int32_t* __restrict__ e_child, const float* __restrict__ lse,
                                   float* __restrict__ lp) {
  const int n_edges = n_nodes - 1;
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= long(B) * n_nodes) return;
  const int b = int(i / n_nodes), e = int(i % n_nodes);
  if (e == n_edges) {
    lp[(size_t)b * n_nodes] = 0.f;
    return;
  }
  const int c = e_child[e];
  lp[(size_t)b * n_nodes + c] -= lse[(size_t)b * n_int + e_qrow[e]];
}

int lmhead_n_tiles(tcs_dtype /*h_dtype*/, int32_t V) { return (V + HEAD_BN - 1) / HEAD_BN; }

int launch_lmhead(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                  int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                  const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                  const int32_t* e_child, int32_t n_edges, float* lse, float* lp, void* part) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = B * n_int;
  if (R <= 0) return TCS_OK;
  const int n_tiles = lmhead_n_tiles(h_dtype, V);
  float2* p = static_cast<float2*>(part);
  if (h_dtype == TCS_BF16) {
    if (d % GEMM_BK != 0) return fail(TCS_EUNSUPPORTED, "lmhead: d=%d is not a multiple of 64", d);
    const int tiles = ((R + 255) / 256) * n_tiles;
    if (w_dtype == TCS_FP8_E4M3)
      lmhead_bf16_kernel<true><<<tiles, 256, 0, s>>>(R, V, d, n_int, n_nodes,
                                                     static_cast<const uint16_t*>(h), W, w_scale,
                                                     e_tok, e_qrow, e_child, n_edges, lp, p);
    else
      lmhead_bf16_kernel<false><<<tiles, 256, 0, s>>>(R, V, d, n_int, n_nodes,
                                                      static_cast<const uint16_t*>(h), W, nullptr,
                                                      e_tok, e_qrow, e_child, n_edges, lp, p);
  } else {
    dim3 grid(n_tiles, (R + 7) / 8);
    lmhead_f32_kernel<<<grid, 256, 0, s>>>(R, V, d, n_int, n_nodes, static_cast<const float*>(h),
                                           static_cast<const float*>(W), e_tok, e_qrow, e_child,
                                           n_edges, lp, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead: %s", hipGetErrorString(e));
  lse_finalize_kernel<<<(R + 255) / 256, 256, 0, s>>>(R, n_tiles, p, lse);
  const long nlp = long(B) * n_nodes;
  lp_finalize_kernel<<<int((nlp + 255) / 256), 256, 0, s>>>(B, n_int, n_nodes, e_qrow, e_child, lse,
                                                             lp);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead finalize: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
