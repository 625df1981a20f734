// Full-vocabulary output head with fused log-sum-exp and child-token gather.
//
// "To Classify, Try a Trie Tree", section 4.1: turning label scores into
// probabilities needs every vocabulary row at every answer position
// (F_head = 2 d V per position).  The [rows x V] logits are never written: each
// workgroup reduces its 256 x 256 tile to a per-row (max, sum exp) partial while
// the logits are still in the matrix-core accumulators, and the few logits that
// belong to trie edges are copied out of those registers by the lane that holds
// them.  A finalize pass merges the partials into lse and turns the gathered
// logits into token log-probabilities.
#include <cstdio>

#include "gemm_core.h"
#include "tcs_internal.h"

namespace tcs {

constexpr int HEAD_BN = 256;  // vocabulary entries per tile: also the partial granularity
constexpr int GATHER_CHUNK = 4096;

__device__ __forceinline__ int lower_bound_i32(const int32_t* __restrict__ a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// seg[t] = first edge whose token is >= t * 256 (edges are sorted by token), so
// vocabulary tile t owns edges [seg[t], seg[t+1]).
__global__ void head_seg_kernel(int n_tiles, const int32_t* __restrict__ e_tok, int n_edges,
                                int32_t* __restrict__ seg) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t <= n_tiles) seg[t] = t == n_tiles ? n_edges : lower_bound_i32(e_tok, n_edges, t * HEAD_BN);
}

// bf16 head.  The tile is computed transposed, logits^T[v][r] = W[v] . h[r], so in
// the 32x32 MFMA result layout each lane holds one hidden row (column l%32 of a
// block) and 16 vocabulary entries per block: the row's max / sum-exp is reduced
// in-lane plus one exchange with lane l^32, then across the two vocab-side waves.
__global__ __launch_bounds__(256, 1) void lmhead_bf16_kernel(
    int R, int V, int d, int n_int, int n_nodes, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ W, const int32_t* __restrict__ seg, const int32_t* __restrict__ e_tok,
    const int32_t* __restrict__ e_qrow, const int32_t* __restrict__ e_child, float* __restrict__ raw,
    float2* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[DMA_SLOT_BYTES], st1[DMA_SLOT_BYTES],
      st2[DMA_SLOT_BYTES], st3[DMA_SLOT_BYTES], st4[DMA_SLOT_BYTES];
  const int n_rt = (R + 255) / 256, n_vt = (V + HEAD_BN - 1) / HEAD_BN;
  int rt, vt;
  if (!head_tile_coords(n_rt, n_vt, rt, vt)) return;
  const int r0 = rt * 256, v0 = vt * HEAD_BN;
  f32x16 acc[4][4];
  const DmaLds L{{st0, st1, st2, st3, st4}};
  gemm256_mainloop_dma(W, d, h, d, V, R, d, v0, r0, L, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // acc[im][jn][e]: vocabulary v0 + vlane + 32 im + 8 (e>>2) + (e&3); hidden row
  // r0 + rloc + 32 jn
  const int vlane = wm * 128 + 4 * (lane >> 5);
  const int rloc = wn * 128 + (lane & 31);

  if (v0 + HEAD_BN > V) {  // last vocabulary tile: entries past V drop out
#pragma unroll
    for (int im = 0; im < 4; ++im)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ok = v0 + vlane + im * 32 + 8 * (e >> 2) + (e & 3) < V;
#pragma unroll
        for (int jn = 0; jn < 4; ++jn) acc[im][jn][e] = ok ? acc[im][jn][e] : -INFINITY;
      }
  }

  // child-token gather: this tile's edges [e_lo, e_hi) are indexed in LDS by
  // vocabulary offset; each lane looks up its 64 vocabulary entries and copies the
  // logit of each of its hidden rows whose query row matches an edge.
  const int e_lo = seg[vt], e_hi = seg[vt + 1];
  if (e_lo < e_hi) {
    int* vmap = reinterpret_cast<int*>(st0);
    int rq[4], rb[4];
#pragma unroll
    for (int jn = 0; jn < 4; ++jn) {
      const int r = r0 + rloc + 32 * jn;
      rq[jn] = r < R ? r % n_int : -1;
      rb[jn] = r / n_int;
    }
    for (int c0 = e_lo; c0 < e_hi; c0 += GATHER_CHUNK) {
      const int c1 = min(e_hi, c0 + GATHER_CHUNK);
      vmap[threadIdx.x] = -1;
      __syncthreads();
      for (int k = c0 + threadIdx.x; k < c1; k += 256) {
        const int tok = e_tok[k];
        if (k == c0 || e_tok[k - 1] != tok) vmap[tok - v0] = k;
      }
      __syncthreads();
#pragma unroll
      for (int im = 0; im < 4; ++im)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int vo = vlane + im * 32 + 8 * (e >> 2) + (e & 3);
          int k = vmap[vo];
          if (k >= 0) {
            for (; k < c1 && e_tok[k] == v0 + vo; ++k) {
              const int q = e_qrow[k], c = e_child[k];
#pragma unroll
              for (int jn = 0; jn < 4; ++jn)
                if (rq[jn] == q) raw[(size_t)rb[jn] * n_nodes + c] = acc[im][jn][e];
            }
          }
        }
      __syncthreads();
    }
  }

  // per hidden row: max and sum of exp over this wave's 128 vocabulary entries
  float2* red = reinterpret_cast<float2*>(st1);  // [2 vocab halves][256 rows]
  constexpr float LOG2E = 1.4426950408889634f;
#pragma unroll
  for (int jn = 0; jn < 4; ++jn) {
    float m = acc[0][jn][0];
#pragma unroll
    for (int im = 0; im < 4; ++im)
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, acc[im][jn][e]);
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float s = 0.f;
    if (m != -INFINITY) {
      const float ml = m * LOG2E;
#pragma unroll
      for (int im = 0; im < 4; ++im)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += exp2f(fmaf(acc[im][jn][e], LOG2E, -ml));
    }
    s += __shfl_xor(s, 32, 64);
    if (lane < 32) red[wm * 256 + rloc + 32 * jn] = float2{m, s};
  }
  __syncthreads();
  {
    const int t = threadIdx.x;
    float2 a = red[t];
    const float2 b = red[256 + t];
    lse_merge(a.x, a.y, b.x, b.y);
    if (r0 + t < R) part[(size_t)vt * R + r0 + t] = a;
  }
}

// fp8-weight head (E4M3 codes converted to bf16 while staging; per-row fp32 scale
// applied to the dot product).  256 rows x 256 vocabulary entries per tile.
__global__ __launch_bounds__(256, 1) void lmhead_fp8_kernel(
    int R, int V, int d, int n_int, int n_nodes, const uint16_t* __restrict__ h,
    const uint8_t* __restrict__ W, const float* __restrict__ w_scale, const int32_t* __restrict__ seg,
    const int32_t* __restrict__ e_tok, const int32_t* __restrict__ e_qrow,
    const int32_t* __restrict__ e_child, float* __restrict__ raw, float2* __restrict__ part) {
  constexpr int BM = 256, BN = HEAD_BN, WM = 2, WN = 2;
  using S = GemmShape<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_ELEMS];
  const int nbm = (R + BM - 1) / BM, nbn = (V + BN - 1) / BN;
  int mt, nt;
  tile_coords<8>(nbm, nbn, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  f32x4 acc[S::MB][S::NB];
  gemm_mainloop<BM, BN, WM, WN, true>(h, d, W, d, R, V, d, m0, n0, lds, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int col_base = n0 + wn * S::TN + (lane & 15);
  const int row_base = m0 + wm * S::TM + (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < S::NB; ++j) {
    const int col = col_base + j * 16;
    const bool ok = col < V;
    const float sc = ok ? w_scale[col] : 1.0f;
#pragma unroll
    for (int i = 0; i < S::MB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = ok ? acc[i][j][r] * sc : -INFINITY;
  }
  const int e_lo = seg[nt], e_hi = seg[nt + 1];
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
    const int t = threadIdx.x;
    float2 a = red[t];
    const float2 b = red[BM + t];
    lse_merge(a.x, a.y, b.x, b.y);
    if (m0 + t < R) part[(size_t)nt * R + m0 + t] = a;
  }
}

// fp32 head: one thread per vocabulary entry of a 256-entry tile, 8 rows per block.
__global__ __launch_bounds__(256) void lmhead_f32_kernel(
    int R, int V, int d, int n_int, int n_nodes, const float* __restrict__ h,
    const float* __restrict__ W, const int32_t* __restrict__ seg, const int32_t* __restrict__ e_tok,
    const int32_t* __restrict__ e_qrow, const int32_t* __restrict__ e_child, float* __restrict__ raw,
    float2* __restrict__ part) {
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
  for (int e = seg[nt]; e < seg[nt + 1]; ++e) {
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

// Merge the per-tile (max, sum exp) partials of each row into lse.  Many rows:
// one thread per row, reads coalesced across rows.  Few rows: one wave per row,
// lanes stride over the tiles, then a shuffle merge.
__global__ void lse_finalize_kernel(int R, int n_tiles, const float2* __restrict__ part,
                                    float* __restrict__ lse) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  float m = -INFINITY, s = 0.f;
#pragma unroll 8
  for (int t = 0; t < n_tiles; ++t) {
    const float2 p = part[(size_t)t * R + r];
    lse_merge(m, s, p.x, p.y);
  }
  lse[r] = m + logf(s);
}

__global__ __launch_bounds__(256) void lse_finalize_wave_kernel(int R, int n_tiles,
                                                                const float2* __restrict__ part,
                                                                float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  float m = -INFINITY, s = 0.f;
  for (int t = lane; t < n_tiles; t += 64) {
    const float2 p = part[(size_t)t * R + r];
    lse_merge(m, s, p.x, p.y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) lse[r] = m + logf(s);
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

size_t lmhead_ws_bytes(int32_t rows, int32_t V) {
  const int n_tiles = lmhead_n_tiles(TCS_BF16, V);
  return align_up(size_t(n_tiles) * size_t(rows) * 8) + align_up(size_t(n_tiles + 1) * 4);
}

int launch_lmhead(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                  int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                  const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                  const int32_t* e_child, int32_t n_edges, float* lse, float* lp, void* ws) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = B * n_int;
  if (R <= 0) return TCS_OK;
  const int n_tiles = lmhead_n_tiles(h_dtype, V);
  Carve cv(ws);
  float2* p = cv.take<float2>(size_t(n_tiles) * R);
  int32_t* seg = cv.take<int32_t>(n_tiles + 1);
  head_seg_kernel<<<(n_tiles + 256) / 256, 256, 0, s>>>(n_tiles, e_tok, n_edges, seg);
  timer_begin(TCS_TIMER_HEAD, stream);
  if (h_dtype == TCS_BF16) {
    if (d % 64 != 0) return fail(TCS_EUNSUPPORTED, "lmhead: d=%d is not a multiple of 64", d);
    const int n_rt = (R + 255) / 256;
    if (w_dtype == TCS_FP8_E4M3)
      lmhead_fp8_kernel<<<n_rt * n_tiles, 256, 0, s>>>(R, V, d, n_int, n_nodes,
                                                        static_cast<const uint16_t*>(h),
                                                        static_cast<const uint8_t*>(W), w_scale, seg,
                                                        e_tok, e_qrow, e_child, lp, p);
    else
      lmhead_bf16_kernel<<<head_grid(n_rt, n_tiles), 256, 0, s>>>(
          R, V, d, n_int, n_nodes, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W),
          seg, e_tok, e_qrow, e_child, lp, p);
  } else {
    dim3 grid(n_tiles, (R + 7) / 8);
    lmhead_f32_kernel<<<grid, 256, 0, s>>>(R, V, d, n_int, n_nodes, static_cast<const float*>(h),
                                           static_cast<const float*>(W), seg, e_tok, e_qrow, e_child,
                                           lp, p);
  }
  timer_end(TCS_TIMER_HEAD, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead: %s", hipGetErrorString(e));
  if (R < 16384)
    lse_finalize_wave_kernel<<<(R + 3) / 4, 256, 0, s>>>(R, n_tiles, p, lse);
  else
    lse_finalize_kernel<<<(R + 255) / 256, 256, 0, s>>>(R, n_tiles, p, lse);
  const long nlp = long(B) * n_nodes;
  lp_finalize_kernel<<<int((nlp + 255) / 256), 256, 0, s>>>(B, n_int, n_nodes, e_qrow, e_child, lse,
                                                             lp);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead finalize: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
