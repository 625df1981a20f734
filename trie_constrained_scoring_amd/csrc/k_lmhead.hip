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
#include <utility>

#include "gemm_core.h"
#include "tcs_internal.h"

namespace tcs {

constexpr int HEAD_BN = 256;   // vocabulary entries per tile
constexpr int HEAD_SEG = 128;  // vocabulary entries per edge segment (and bf16 partial)
constexpr int HEAD_WGS = 256;  // persistent bf16 head: one workgroup per CU
constexpr int HEAD_LIST_ROWS = 64;  // rows per gather list (per vocabulary half-tile)
// below this many rows the matrix-core head stores its (max, sum) partials row-major
constexpr int LSE_ROWMAJOR_MAX_ROWS = 4096;

__device__ __forceinline__ int lower_bound_i32(const int32_t* __restrict__ a, int n, int key) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < key) lo = mid + 1; else hi = mid;
  }
  return lo;
}

// seg[t] = first edge whose token is >= t * 128 (edges are sorted by token), so
// vocabulary half-tile t (128 entries) owns edges [seg[t], seg[t+1]) and tile t
// (256 entries) owns [seg[2t], seg[2t+2]).
// Also clears the bf16 head's zero block (n_zero 16-byte words).
__global__ void head_prep_kernel(int n_seg, const int32_t* __restrict__ e_tok, int n_edges,
                                 int32_t* __restrict__ seg, uint4* __restrict__ zero, int n_zero) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t <= n_seg) seg[t] = t == n_seg ? n_edges : lower_bound_i32(e_tok, n_edges, t * HEAD_SEG);
  if (t < n_zero) zero[t] = uint4{0u, 0u, 0u, 0u};
}

// Gather lists of the bf16 head.  The logit of child c of query row q in document
// b sits in tile (vocabulary half-tile tok/128, row tile r/256), r = b n_int + q,
// in accumulator element t = 16 im + e of the lane whose half is hh and whose row
// is r % 256.  Each (edge, document) pair is pushed on the list of its vocabulary
// half-tile and 64-row block (the rows one wave of a 256-row tile holds), so a
// wave walks only its own rows' records: rec = {next, output index b*n_nodes + c,
// t | hh << 6 | (r % 256) << 7, 0}.
__global__ void head_list_init_kernel(int n_keys, int32_t* __restrict__ list_head) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n_keys) list_head[t] = -1;
}

__global__ void head_list_link_kernel(int B, int n_int, int n_nodes, int n_rb,
                                      const int32_t* __restrict__ e_tok,
                                      const int32_t* __restrict__ e_qrow,
                                      const int32_t* __restrict__ e_child, int n_edges,
                                      int32_t* __restrict__ list_head, int4* __restrict__ rec) {
  const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= long(n_edges) * B) return;
  const int e = int(i / B), b = int(i % B);
  const int tok = e_tok[e];
  const int r = b * n_int + e_qrow[e];
  const int off = tok & (HEAD_SEG - 1);  // 32 im + 8 (e>>2) + 4 hh + (e&3)
  const int t = (off >> 5) * 16 + (((off >> 3) & 3) << 2) + (off & 3);
  const int hh = (off >> 2) & 1;
  const int key = (tok / HEAD_SEG) * n_rb + r / HEAD_LIST_ROWS;
  const int next = atomicExch(&list_head[key], int(i));
  rec[i] = int4{next, b * n_nodes + e_child[e], t | (hh << 6) | ((r & 255) << 7), 0};
}

// ---------------------------------------------------------------------------
// Matrix-core head (bf16 or fp8 weights, bf16 hidden states).  Persistent: one
// workgroup per CU walks its own sequence of 256 x 256 tiles (head_tile_coords),
// and the LDS ring of five 32 KB operand slots runs on across tile boundaries, so
// the first k-tiles of the next tile load while the current one finishes and while
// its epilogue runs.  The workgroup has 8 waves, two per SIMD, each owning 128
// vocabulary entries x 64 rows (4 x 2 blocks of v_mfma_f32_32x32x16_bf16): while
// one wave of a SIMD waits on LDS reads, DMA issue or the step barrier, the other
// keeps the matrix core fed (measured on MI355X: 9% faster than 4 waves of
// 128 x 128 on a 97k-row head, at the cost of 1.5x the LDS reads).
//
// Global k-step g (over all tiles of this workgroup) keeps W's k-tile in slot
// 2g mod 5 and h's in slot 2g+1 mod 5; while step g is multiplied, h(g+1) and
// W(g+2) are in flight, so the streamed weight matrix gets two steps of latency
// cover.  One barrier per step.  Each operand is read by its own DMA stream that
// steps from the last k-tile of one tile to the first of the next; loads past the
// last tile go through a zero-range buffer resource and touch no memory.
//
// The tile is computed transposed, logits^T[v][r] = W[v] . h[r]: in the 32x32
// MFMA result layout each lane holds one hidden row (column l%32 of a block) and
// 16 vocabulary entries per block, so a row's max / sum-exp over the wave's 128
// entries is reduced in-lane plus one exchange with lane l^32 and written as one
// partial per (row, vocabulary half-tile).  The epilogue touches no LDS: child
// logits are picked out of the accumulators by a scalar walk over the half-tile's
// edges.
//
// fp8 weights (E4M3 codes + one fp32 scale per vocabulary row) take half the
// bytes: a W k-tile is 256 rows x 64 bytes, each lane reads 16 codes (k-steps 2m
// and 2m+1) with one 16-byte LDS read, the codes are converted to bf16 in
// registers (exact: every E4M3 value is a bf16 value) and the row scale multiplies
// the fp32 logits in the epilogue.  The k order inside a pair of k-steps is
// permuted the same way on both operands (lane half c supplies k 32m + 16c + 8s +
// 0..7 in step 2m+s), which leaves the dot products unchanged.
//
// With fp8 hidden states too (W8A8) both operands are E4M3 codes in 128-byte slot
// rows, 128 codes per k-step (the bf16 slot layout), and each 32x32 block takes two
// fp8 matrix ops per step: the steps, and so the barriers, are half as many as with
// 64-code steps, and each DMA stream has as much time to land as in the bf16 head.

// The ring kernel runs 8 waves (two per SIMD); each owns 128 vocabulary entries x
// 64 rows of the 256 x 256 tile and loads 1/8 of every operand k-tile.
constexpr int RING_WAVES = 8;
constexpr int RING_LOADS = 4;   // bf16 operand: 1 KB loads per wave per k-tile
constexpr int RING_LOADS8 = 2;  // fp8 W: 1 KB loads per wave per k-tile
// Rows per tile of the head: 256, or 128 (one 32-row block per wave).  A 128-row
// tile reads the weights once per 128 rows instead of per 256 and each wave's
// fragment reads feed 4 matrix ops instead of 8, so it costs more per product,
// but it pads fewer rows and gives the chip more tiles when the rows are few
// (the launcher's choice is head_tile_rows).

// NL bf16 loads (1 KB each) of an operand k-tile into an LDS slot: load j fills
// slot rows row0 + 8j .. +7, lane i writing 16 bytes at row i/8, position i%8;
// `vo` holds each load's lane byte offset, `k` the k-tile (scalar offset).
template <int NL>
__device__ __forceinline__ void head_issue(const void* base, int bytes, int k, uint8_t* sl, int row0,
                                           const int* vo) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
  const int so = k * DMA_BK * 2;
#pragma unroll
  for (int j = 0; j < NL; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, TCS_LDS(sl + (row0 + j * 8) * 128), 16, vo[j], so, 0, 0);
}

// fp8 W k-tile (256 rows x 64 bytes, 16 KB) of this wave: load j (0..1) fills slot
// rows wave*32 + 16j .. +15, lane i writing 16 bytes at row i/4, position i%4.
__device__ __forceinline__ void head_issue8(const void* base, int bytes, int k, uint8_t* sl,
                                            int wave, const int (&vo)[RING_LOADS8]) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
  const int so = k * DMA_BK;
#pragma unroll
  for (int j = 0; j < RING_LOADS8; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, TCS_LDS(sl + (wave * 32 + j * 16) * 64), 16, vo[j],
                                             so, 0, 0);
}
// fp8 W slot: row r (64 bytes) keeps its 16-byte chunk c at position c ^ dma8_swz(r),
// so the 16 rows read by a group of lanes fall on distinct banks.
__device__ __forceinline__ int dma8_swz(int r) { return (r >> 2) & 3; }

// Eight E4M3 codes (bytes of w0, w1, lowest first) -> eight bf16 (hardware
// conversion, scale 1: exact).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

// v[jn] = acc[t / 16][jn][t % 16] for a wave-uniform t in [0, 64): a binary
// select tree on the six bits of t (63 selects per jn, six lane masks), so the
// accumulators are only read in place.
template <int JN = 2>
__device__ __forceinline__ void head_pick(int t, const f32x16 (&acc)[4][2], float (&v)[2]) {
#pragma unroll
  for (int jn = 0; jn < JN; ++jn) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int c0 = 2 * i, c1 = 2 * i + 1;
      x[i] = (t & 1) ? acc[c1 / 16][jn][c1 % 16] : acc[c0 / 16][jn][c0 % 16];
    }
#pragma unroll
    for (int lvl = 1, n = 16; n >= 1; ++lvl, n >>= 1)
#pragma unroll
      for (int i = 0; i < n; ++i) x[i] = ((t >> lvl) & 1) ? x[2 * i + 1] : x[2 * i];
    v[jn] = x[0];
  }
}

// Max and sum of exp of each of the lane's two rows (jn) over its 64 entries
// plus the partner lane's (l ^ 32); entries at or past `vlim` are excluded when
// MASK.  One row at a time, so only that row's 64 values are live.
// exp2 is the hardware instruction: arguments are <= 0, and terms below 2^-126
// of the row maximum, which it flushes, are far below fp32 resolution of the sum.
template <bool MASK, int JN = 2>
__device__ __forceinline__ void head_rows_lse(const f32x16 (&acc)[4][2], int vlim,
                                              float2 (&out)[2]) {
  constexpr float LOG2E = 1.4426950408889634f;
#pragma unroll
  for (int jn = 0; jn < JN; ++jn) {
    float m = -INFINITY;
#pragma unroll
    for (int im = 0; im < 4; ++im)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ok = !MASK || 32 * im + 8 * (e >> 2) + (e & 3) < vlim;
        m = fmaxf(m, ok ? acc[im][jn][e] : -INFINITY);
      }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float ml = m == -INFINITY ? 0.f : m * LOG2E;
    float sum = 0.f;
#pragma unroll
    for (int im = 0; im < 4; ++im)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool ok = !MASK || 32 * im + 8 * (e >> 2) + (e & 3) < vlim;
        const float x = __builtin_amdgcn_exp2f(fmaf(acc[im][jn][e], LOG2E, -ml));
        sum += ok ? x : 0.f;
      }
    out[jn] = float2{m, sum + __shfl_xor(sum, 32, 64)};
  }
}

// acc[im][jn][e] *= scale of vocabulary entry vb + 32 im + 8 (e>>2) + (e&3) (fp8
// head); entries at or past V are left alone (the row sums exclude them).
template <int JN = 2>
__device__ __forceinline__ void head_scale_rows(f32x16 (&acc)[4][2], const float* __restrict__ w_scale,
                                                int vb, int V) {
#pragma unroll
  for (int im = 0; im < 4; ++im)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int v = vb + 32 * im + 8 * g;
      float4 sc;
      if (v + 4 <= V) {
        sc = *reinterpret_cast<const float4*>(w_scale + v);
      } else {
        sc.x = v < V ? w_scale[v] : 1.f;
        sc.y = v + 1 < V ? w_scale[v + 1] : 1.f;
        sc.z = v + 2 < V ? w_scale[v + 2] : 1.f;
        sc.w = 1.f;
      }
#pragma unroll
      for (int jn = 0; jn < JN; ++jn) {
        acc[im][jn][4 * g + 0] *= sc.x;
        acc[im][jn][4 * g + 1] *= sc.y;
        acc[im][jn][4 * g + 2] *= sc.z;
        acc[im][jn][4 * g + 3] *= sc.w;
      }
    }
}

// Plain-product mode of the ring kernel (the output projection y = x + O Wo^T of
// many rows): C[r][n] = sum_k h[r][k] W[n][k] + E[token[qnode[r % n_int]]][n], fp32.
struct RingGemmOut {
  float* C;
  int ldc;
  const uint16_t* E;
  const int32_t* token;
  const int32_t* qnode;
  int n_int;
};

// Tile order of the plain-product mode: linear tile t = 256 w + 32 xcd + slot
// (row-major over (row tile, column tile)), so each XCD takes 32 consecutive tiles
// per round and the row tiles they share stay in its L2.
__device__ __forceinline__ bool gemm_tile_coords(int bid, int n_rt, int n_vt, int& rt, int& vt) {
  const int xcd = bid & 7, slot = (bid >> 3) & 31, w = bid >> 8;
  const int t = w * 256 + xcd * 32 + slot;
  rt = t / n_vt;
  vt = t - rt * n_vt;
  return t < n_rt * n_vt;
}

template <bool W8, bool GEMM, bool A8 = false, int TR = 256>
__device__ __forceinline__ void ring_body(
    int R, int V, int d, const uint16_t* __restrict__ h, const uint8_t* __restrict__ W,
    const float* __restrict__ w_scale, const float* __restrict__ h_scale,
    const int32_t* __restrict__ list_head,
    const int4* __restrict__ rec, float* __restrict__ raw, float2* __restrict__ part,
    const uint16_t* __restrict__ zero, int rounds_per_wg, const RingGemmOut& go) {
  __shared__ __attribute__((aligned(16))) uint8_t st0[DMA_SLOT_BYTES], st1[DMA_SLOT_BYTES],
      st2[DMA_SLOT_BYTES], st3[DMA_SLOT_BYTES], st4[DMA_SLOT_BYTES];
  uint8_t* const slot[DMA_SLOTS] = {st0, st1, st2, st3, st4};
  static_assert(!A8 || (W8 && !GEMM), "fp8 activations go with fp8 weights in the head");
  static_assert(TR == 256 || (TR == 128 && !GEMM), "rows per tile: 256, or 128 in the head");
  constexpr int WRB = W8 ? 1 : 2;  // bytes per weight element
  constexpr int HRB = A8 ? 1 : 2;  // bytes per hidden-state element
  constexpr int JN = TR / 128;  // 32-row blocks per wave
  const int n_rt = (R + TR - 1) / TR, n_vt = (V + HEAD_BN - 1) / HEAD_BN;
  const int n_rbl = (R + HEAD_LIST_ROWS - 1) / HEAD_LIST_ROWS;  // row blocks of the gather lists
  // workgroup g takes rounds [w_lo, rounds) of slot g % 256: a bounded run of
  // consecutive rounds, so the workgroups that share operand tiles in an XCD's L2
  // stay within a few rounds of each other
  const int w_lo = int(blockIdx.x) / HEAD_WGS * rounds_per_wg;
  const int all_rounds = GEMM ? (n_rt * n_vt + HEAD_WGS - 1) / HEAD_WGS : head_grid(n_rt, n_vt) / HEAD_WGS;
  const int rounds = min(all_rounds, w_lo + rounds_per_wg);
  const int bslot = int(blockIdx.x) % HEAD_WGS;
  // k-step: 64 elements (128-byte bf16 rows, 64-byte fp8 W rows), or 128 fp8
  // elements (128-byte rows) when both operands are fp8
  const int nk = A8 ? d / (2 * DMA_BK) : d / DMA_BK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wr = wave >> 1;  // vocabulary half, row quarter

  auto coords = [&](int w, int& rt, int& vt) __attribute__((always_inline)) {
    if constexpr (GEMM) return gemm_tile_coords(w * HEAD_WGS + bslot, n_rt, n_vt, rt, vt);
    else return head_tile_coords(w * HEAD_WGS + bslot, n_rt, n_vt, rt, vt);
  };
  auto next_valid = [&](int w) __attribute__((always_inline)) {
    int rt, vt;
    while (w < rounds && !coords(w, rt, vt)) ++w;
    return w;
  };

  // Rows of W and h that tile w reads, as (base, bytes) of a buffer resource;
  // zero bytes past the last tile.  Rows past an operand's end lie outside the
  // resource's range, so the buffer unit drops those loads; the epilogue discards
  // those rows.  (Resources are built at each issue from these plain values, which
  // keeps them in scalar registers.)
  struct Span {
    const uint8_t* wb;
    const uint8_t* hb;
    int wn, hn;
  };
  const uint8_t* const hbytes = reinterpret_cast<const uint8_t*>(h);
  auto span = [&](int w) __attribute__((always_inline)) {
    int rt, vt;
    if (w < rounds && coords(w, rt, vt))
      return Span{W + (size_t)vt * 256 * d * WRB, hbytes + (size_t)rt * TR * d * HRB,
                  min(256, V - vt * 256) * d * WRB, min(TR, R - rt * TR) * d * HRB};
    return Span{W, hbytes, 0, 0};
  };

  // 128-byte slot rows (bf16 operands; both fp8 operands with A8).  Load j (0..3)
  // of this wave fills slot rows wave*32 + 8j .. +7 (1 KB): lane i writes row i/8,
  // position i%8, which holds global chunk (i%8) ^ swz(row % 16); row % 16 =
  // 8*(j&1) + i/8.  The k offset goes in the scalar offset.
  const int lr = lane >> 3, lp = lane & 7;
  int vo[RING_LOADS];
#pragma unroll
  for (int j = 0; j < RING_LOADS; ++j)
    vo[j] = (wave * 32 + j * 8 + lr) * (d * WRB) + (lp ^ dma_swz(lr + 8 * (j & 1))) * 16;
  // h k-tile (TR rows): the wave's TR/64 loads fill rows wave*TR/8 + 8j + i/8
  int voh[TR / 64];
#pragma unroll
  for (int j = 0; j < TR / 64; ++j)
    voh[j] = (wave * (TR / 8) + j * 8 + lr) * (d * HRB) + (lp ^ dma_swz(lr + 8 * (j & 1))) * 16;
  // fp8 W with bf16 h: load j (0..1) fills rows wave*32 + 16j + i/4, position i%4,
  // which holds chunk (i%4) ^ dma8_swz(row % 16)
  constexpr bool W8H16 = W8 && !A8;
  int vo8[RING_LOADS8];
#pragma unroll
  for (int j = 0; j < RING_LOADS8; ++j) {
    const int row = wave * 32 + j * 16 + (lane >> 2);
    vo8[j] = row * d + (((lane & 3) ^ dma8_swz(row & 15)) << 4);
  }
  constexpr int W_LOADS = W8H16 ? RING_LOADS8 : RING_LOADS;
  constexpr int H_LOADS = TR / 64;
  int w = next_valid(w_lo);
  if (w >= rounds) return;
  // A tile runs nk5 = nk rounded up to a multiple of 5 steps, so every tile starts
  // at ring position 0.  Steps past nk load both operands from `zero` (256 x d
  // bf16 zeros), so they run the same code and add nothing.  Loads run up to two
  // steps ahead, so they reach into the next tile at most.
  const int nk5 = (nk + 4) / 5 * 5;
  const int zbytes = nk5 == nk ? 0 : 256 * d * 2;
  // this tile's spans and the step to the next tile's (kept as differences, so a
  // load's operand is this tile's value plus a selected offset)
  Span s0 = span(w);
  int w1 = next_valid(w + 1);
  Span s1 = span(w1);
  long dwb = s1.wb - s0.wb, dhb = s1.hb - s0.hb;
  int dwn = s1.wn - s0.wn, dhn = s1.hn - s0.hn;
  // padded position q (steps past this tile's start) -> (operand rows, k-tile)
  auto issue_w = [&](int q, uint8_t* sl) __attribute__((always_inline)) {
    const bool nxt = q >= nk5;
    const int k = nxt ? q - nk5 : q;
    const bool pad = k >= nk;
    const uint8_t* b = s0.wb + (nxt ? dwb : 0);
    const int n = s0.wn + (nxt ? dwn : 0);
    if constexpr (W8H16)
      head_issue8(pad ? static_cast<const void*>(zero) : b, pad ? zbytes : n, pad ? 0 : k, sl, wave, vo8);
    else
      head_issue<RING_LOADS>(pad ? static_cast<const void*>(zero) : b, pad ? zbytes : n, pad ? 0 : k, sl,
                             wave * 32, vo);
  };
  auto issue_h = [&](int q, uint8_t* sl) __attribute__((always_inline)) {
    const bool nxt = q >= nk5;
    const int k = nxt ? q - nk5 : q;
    const bool pad = k >= nk;
    const uint8_t* b = s0.hb + (nxt ? dhb : 0);
    const int n = s0.hn + (nxt ? dhn : 0);
    head_issue<TR / 64>(pad ? static_cast<const void*>(zero) : b, pad ? zbytes : n, pad ? 0 : k, sl,
                        wave * (TR / 8), voh);
  };

  // h fragment of k-step ks: row base + lane%32, chunk 2 ks + lane/32 (bf16 W) or
  // 4 (ks/2) + 2 (lane/32) + ks%2 (fp8 W's k order)
  int fo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int chunk = W8 ? 4 * (ks >> 1) + 2 * (lane >> 5) + (ks & 1) : 2 * ks + (lane >> 5);
    fo[ks] = (lane & 31) * 128 + ((chunk ^ dma_swz(lane & 15)) * 16);
  }
  // fp8 W fragment pair m: row base + lane%32, chunk 2m + lane/32
  int fo8[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) fo8[m] = (lane & 31) * 64 + (((2 * m + (lane >> 5)) ^ dma8_swz(lane & 15)) << 4);
  bf16x8 fa[2][4], fb[2][JN];
  uint4 wraw[4];  // fp8 W codes of the current pair of k-steps
  f32x16 acc[4][2];
  auto read_frags = [&](const uint8_t* sa, const uint8_t* sb, int ks, bf16x8 (&xa)[4],
                        bf16x8 (&xb)[JN]) {
    if constexpr (W8) {
      if ((ks & 1) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wraw[i] = *reinterpret_cast<const uint4*>(sa + (wm * 128 + i * 32) * 64 + fo8[ks >> 1]);
      }
#pragma unroll
      for (int j = 0; j < JN; ++j)
        xb[j] = *reinterpret_cast<const bf16x8*>(sb + (wr * 32 * JN + j * 32) * 128 + fo[ks]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[i] = (ks & 1) ? e4m3x8_to_bf16(wraw[i].z, wraw[i].w) : e4m3x8_to_bf16(wraw[i].x, wraw[i].y);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[i] = *reinterpret_cast<const bf16x8*>(sa + (wm * 128 + i * 32) * 128 + fo[ks]);
#pragma unroll
      for (int j = 0; j < JN; ++j)
        xb[j] = *reinterpret_cast<const bf16x8*>(sb + (wr * 32 * JN + j * 32) * 128 + fo[ks]);
    }
  };
  auto mfma_step = [&](const bf16x8 (&xa)[4], const bf16x8 (&xb)[JN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], xb[j], acc[i][j], 0, 0, 0);
  };
  // a k-step's 4 JN matrix ops, each paired with a fragment read or conversions
  constexpr int NM = 4 * JN;
  auto interleave_ds = [&]() __attribute__((always_inline)) {
    if constexpr (W8) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1 + JN % 2 * 2, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
#pragma unroll
      for (int g = 1; g < NM / 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
#pragma unroll
      for (int g = 0; g < NM / 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x002, 8 / JN, 0);  // VALU (code conversion)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x100, 3 - JN, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
#pragma unroll
      for (int g = 1; g < 4 + JN && g < NM; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
    }
  };
  // global k-step with ring position U: W in slot 2U mod 5, h in slot 2U+1 mod 5
  // LAST: the tile's final step, which leaves the next tile's first fragments to
  // be read after the epilogue (fewer registers live across it)
  auto step = [&](auto Uc, int kt, auto Lc) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    constexpr bool LAST = decltype(Lc)::value;
    constexpr int sA = (2 * U) % 5, sB = (2 * U + 1) % 5;
    constexpr int sA1 = (2 * U + 2) % 5, sB1 = (2 * U + 3) % 5, sA2 = (2 * U + 4) % 5;
    issue_h(kt + 1, slot[sB1]);  // h(g+1)
    issue_w(kt + 2, slot[sA2]);  // W(g+2)
    {
      read_frags(slot[sA], slot[sB], 1, fa[1], fb[1]);
      mfma_step(fa[0], fb[0]);
      constexpr int VM = (H_LOADS + W_LOADS + NM - 1) / NM;  // loads per matrix op
#pragma unroll
      for (int g = 0; g < NM; ++g) {
        if (g * VM < H_LOADS + W_LOADS)
          __builtin_amdgcn_sched_group_barrier(0x020, VM, 0);  // VMEM (buffer -> LDS)
        if (W8) __builtin_amdgcn_sched_group_barrier(0x002, 4 / JN, 0);  // VALU
        else if (g == 0) __builtin_amdgcn_sched_group_barrier(0x100, 3 - JN, 0);  // DS read
        else if (g < 4 + JN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      }
      read_frags(slot[sA], slot[sB], 2, fa[0], fb[0]);
      mfma_step(fa[1], fb[1]);
      interleave_ds();
      read_frags(slot[sA], slot[sB], 3, fa[1], fb[1]);
      mfma_step(fa[0], fb[0]);
      interleave_ds();
    }
    // W(g+1) and h(g+1) of this wave have landed (only W(g+2) may be in flight),
    // and this wave's reads of the current slots are done
    wait_vmcnt<W_LOADS>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    if constexpr (!LAST) read_frags(slot[sA1], slot[sB1], 0, fa[0], fb[0]);
    mfma_step(fa[1], fb[1]);
    if constexpr (!LAST) interleave_ds();
  };

  // fp8 x fp8 (A8): a k-step is 128 codes (one 128-byte slot row per operand row),
  // two v_mfma_scale_f32_32x32x64_f8f6f4 per 32x32 block: in half s lane l supplies
  // k 64 s + 32 (l/32) .. +31 of its row on both operands (16-byte chunks
  // 4 s + 2 (l/32) and + 1); any k order shared by the two operands gives the same
  // dot products.
  int fq[2][2];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      fq[hs][t] = (lane & 31) * 128 + (((4 * hs + 2 * (lane >> 5) + t) ^ dma_swz(lane & 15)) << 4);
  // W fragments (vocabulary blocks) of the current half; h fragments of both halves
  v8i_t wf[4], hf0[JN], hf1[JN];
  auto frag8 = [&](const uint8_t* base, int hs) __attribute__((always_inline)) {
    const uint4 x = *reinterpret_cast<const uint4*>(base + fq[hs][0]);
    const uint4 y = *reinterpret_cast<const uint4*>(base + fq[hs][1]);
    return v8i_t{int(x.x), int(x.y), int(x.z), int(x.w), int(y.x), int(y.y), int(y.z), int(y.w)};
  };
  auto mfma8 = [&](int i, const v8i_t (&hf)[JN]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < JN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[i], hf[j], acc[i][j], 0, 0, 0, 127,
                                                                 0, 127);
  };
  auto wfrag = [&](const uint8_t* sl, int i, int hs) __attribute__((always_inline)) {
    wf[i] = frag8(sl + (wm * 128 + 32 * i) * 128, hs);
  };
  auto hfrag = [&](const uint8_t* sl, v8i_t (&hf)[JN], int hs) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < JN; ++j) hf[j] = frag8(sl + (wr * 32 * JN + 32 * j) * 128, hs);
  };
  // one k-step g (fragments of W blocks 0-1 and h of half 0 were read in the
  // previous step).  Each group of fragment reads is followed by four matrix ops
  // that do not need it: half 0 reads W blocks 2-3, multiplies blocks 0-1, reads
  // half 1's W blocks 0-1 and h, multiplies blocks 2-3; half 1 does the same around
  // the step's barrier, reading the next step's half-0 fragments after it.
  auto step8 = [&](auto Uc, int kt) __attribute__((always_inline)) {
    constexpr int U = decltype(Uc)::value;
    constexpr int sA = (2 * U) % 5, sB = (2 * U + 1) % 5;
    constexpr int sB1 = (2 * U + 3) % 5, sA1 = (2 * U + 2) % 5, sA2 = (2 * U + 4) % 5;
    issue_h(kt + 1, slot[sB1]);  // h(g+1)
    issue_w(kt + 2, slot[sA2]);  // W(g+2)
    wfrag(slot[sA], 2, 0);
    wfrag(slot[sA], 3, 0);
    mfma8(0, hf0);
    mfma8(1, hf0);
    __builtin_amdgcn_sched_barrier(0);
    wfrag(slot[sA], 0, 1);
    wfrag(slot[sA], 1, 1);
    hfrag(slot[sB], hf1, 1);
    mfma8(2, hf0);
    mfma8(3, hf0);
    __builtin_amdgcn_sched_barrier(0);
    wfrag(slot[sA], 2, 1);
    wfrag(slot[sA], 3, 1);
    mfma8(0, hf1);
    mfma8(1, hf1);
    wait_vmcnt<W_LOADS>();
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    wfrag(slot[sA1], 0, 0);
    wfrag(slot[sA1], 1, 0);
    hfrag(slot[sB1], hf0, 0);
    mfma8(2, hf1);
    mfma8(3, hf1);
    __builtin_amdgcn_sched_barrier(0);
  };
  // fragments of a tile's first step: W(0) blocks 0-1 in slot 0, h(0) in slot 1
  auto first_frags8 = [&]() __attribute__((always_inline)) {
    wfrag(slot[0], 0, 0);
    wfrag(slot[0], 1, 0);
    hfrag(slot[1], hf0, 0);
  };

  // prologue: W(0), h(0), W(1)
  issue_w(0, slot[0]);
  issue_h(0, slot[1]);
  issue_w(1, slot[2]);
  wait_vmcnt<W_LOADS>();
  __builtin_amdgcn_s_barrier();
  if constexpr (A8) first_frags8();
  else read_frags(slot[0], slot[1], 0, fa[0], fb[0]);

  const int vhalf = wm * 128 + 4 * (lane >> 5);  // + 32 im + 8 (e>>2) + (e&3)
  const int rloc = wr * 32 * JN + (lane & 31);   // + 32 jn
  for (; w < rounds;) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    using F = std::false_type;
    int kt = 0;
    if constexpr (A8) {
      // The whole tile is one branch-free loop (its final step also reads the next
      // tile's first fragments, which are read again after the epilogue).  A
      // straight-line final group of steps would let the compiler move its matrix
      // ops past the step barriers.
#pragma unroll 1
      for (; kt < nk5; kt += 5) {
        step8(std::integral_constant<int, 0>{}, kt);
        step8(std::integral_constant<int, 1>{}, kt + 1);
        step8(std::integral_constant<int, 2>{}, kt + 2);
        step8(std::integral_constant<int, 3>{}, kt + 3);
        step8(std::integral_constant<int, 4>{}, kt + 4);
      }
    } else {
      for (; kt + 5 < nk5; kt += 5) {
        step(std::integral_constant<int, 0>{}, kt, F{});
        step(std::integral_constant<int, 1>{}, kt + 1, F{});
        step(std::integral_constant<int, 2>{}, kt + 2, F{});
        step(std::integral_constant<int, 3>{}, kt + 3, F{});
        step(std::integral_constant<int, 4>{}, kt + 4, F{});
      }
      step(std::integral_constant<int, 0>{}, kt, F{});
      step(std::integral_constant<int, 1>{}, kt + 1, F{});
      step(std::integral_constant<int, 2>{}, kt + 2, F{});
      step(std::integral_constant<int, 3>{}, kt + 3, F{});
      step(std::integral_constant<int, 4>{}, kt + 4, std::true_type{});
    }

    // ---- epilogue of tile w (no LDS: the ring keeps loading the next tile) ----
    int rt, vt;
    coords(w, rt, vt);
    const int r0 = rt * TR, v0 = vt * HEAD_BN;
    // acc[im][jn][e]: vocabulary v0 + vhalf + 32 im + 8 (e>>2) + (e&3); hidden row
    // r0 + rloc + 32 jn
    if constexpr (GEMM) {
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int r = r0 + rloc + 32 * jn;
        if (r >= R) continue;
        const uint16_t* x = go.E + (size_t)go.token[go.qnode[r % go.n_int]] * V;
        float* c = go.C + (size_t)r * go.ldc;
#pragma unroll
        for (int im = 0; im < 4; ++im)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = v0 + vhalf + 32 * im + 8 * g;
            if (n + 4 <= V) {
              const uint2 xr = *reinterpret_cast<const uint2*>(x + n);
              *reinterpret_cast<float4*>(c + n) = float4{
                  acc[im][jn][4 * g + 0] + __uint_as_float(xr.x << 16),
                  acc[im][jn][4 * g + 1] + __uint_as_float(xr.x & 0xFFFF0000u),
                  acc[im][jn][4 * g + 2] + __uint_as_float(xr.y << 16),
                  acc[im][jn][4 * g + 3] + __uint_as_float(xr.y & 0xFFFF0000u)};
            } else {
#pragma unroll
              for (int t = 0; t < 4; ++t)
                if (n + t < V) c[n + t] = acc[im][jn][4 * g + t] + bf16_to_f32(x[n + t]);
            }
          }
      }
    } else {
    if constexpr (W8) head_scale_rows<JN>(acc, w_scale, v0 + vhalf, V);
    if constexpr (A8) {  // each hidden row's own activation scale
#pragma unroll
      for (int jn = 0; jn < JN; ++jn) {
        const float hs = h_scale[min(r0 + rloc + 32 * jn, R - 1)];
#pragma unroll
        for (int im = 0; im < 4; ++im)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[im][jn][e] *= hs;
      }
    }
    // entries at or past V (last vocabulary tile) drop out of the row sums; the
    // accumulators are only read from here on
    const int vlim = V - v0 - vhalf;  // entry (im, e) is valid iff 32 im + 8 (e>>2) + (e&3) < vlim
    // child-token gather: walk the list of this half-tile and this wave's 64-row block
    // (scalar; rit is the row within the 256-row tile).  The wave's rows are block
    // 4 rt + wr of a 256-row tile; rows 32 wr .. of a 128-row tile fall in block
    // 2 rt + wr / 2, whose other half the filter below skips.  A block past the
    // last row has no list.
    const int lblk = TR == 128 ? 2 * rt + (wr >> 1) : 4 * rt + wr;
    for (int k = lblk < n_rbl ? list_head[(2 * vt + wm) * n_rbl + lblk] : -1; k >= 0;) {
      const int4 q = rec[k];
      const int t = q.z & 63, hh = (q.z >> 6) & 1, rit = q.z >> 7;
      // row r0 + (rit mod TR) is in this wave's share of the tile's rows
      const bool mine = TR == 128 ? ((rit >> 7) == (rt & 1) && ((rit >> 5) & 3) == wr) : (rit >> 6) == wr;
      if (mine) {
        float v[2];
        head_pick<JN>(t, acc, v);
        const float x = (JN == 2 && ((rit >> 5) & 1)) ? v[1] : v[0];
        if (lane == (rit & 31) + 32 * hh) raw[q.y] = x;
      }
      k = q.x;
    }
    // per hidden row: max and sum of exp over this wave's 128 vocabulary entries
    // (only the last vocabulary tile has entries at or past V)
    float2 ms[2];
    if (v0 + HEAD_BN <= V) head_rows_lse<false, JN>(acc, vlim, ms);
    else head_rows_lse<true, JN>(acc, vlim, ms);
#pragma unroll
    for (int jn = 0; jn < JN; ++jn) {
      const int r = r0 + rloc + 32 * jn;
      // few rows: partials [row][half-tile], so each row's are contiguous for the
      // finalisation; else [half-tile][row]
      const size_t pi = R < LSE_ROWMAJOR_MAX_ROWS ? (size_t)r * (2 * n_vt) + 2 * vt + wm
                                                  : (size_t)(2 * vt + wm) * R + r;
      if (lane < 32 && r < R) part[pi] = ms[jn];
    }
    }
    // the next tile's W(0) and h(0) are in slots 0 and 1 (landed at the last
    // barrier, and no load targets those slots until its first step).  The fp8 x fp8
    // loop's final step read them too, but those values are not kept across the
    // epilogue: reading them again here leaves the epilogue 32 more registers.
    if constexpr (A8) first_frags8();
    else read_frags(slot[0], slot[1], 0, fa[0], fb[0]);
    w = w1;
    w1 = next_valid(w1 + 1);
    s0 = s1;
    s1 = span(w1);
    dwb = s1.wb - s0.wb;
    dhb = s1.hb - s0.hb;
    dwn = s1.wn - s0.wn;
    dhn = s1.hn - s0.hn;
  }
  wait_vmcnt<0>();  // loads past the last tile: nothing may still target LDS at exit
}

// The output head (bf16 or fp8 weights; A8: fp8 hidden states with row scales).
template <bool W8, bool A8 = false, int TR = 256>
__global__ __launch_bounds__(64 * RING_WAVES, 1) void lmhead_ring_kernel(
    int R, int V, int d, const uint16_t* __restrict__ h, const uint8_t* __restrict__ W,
    const float* __restrict__ w_scale, const float* __restrict__ h_scale,
    const int32_t* __restrict__ list_head, const int4* __restrict__ rec, float* __restrict__ raw,
    float2* __restrict__ part, const uint16_t* __restrict__ zero, int rounds_per_wg) {
  ring_body<W8, false, A8, TR>(R, V, d, h, W, w_scale, h_scale, list_head, rec, raw, part, zero,
                           rounds_per_wg, RingGemmOut{});
}

// The output projection of many rows (plain products plus the embedding residual).
__global__ __launch_bounds__(64 * RING_WAVES, 1) void proj_ring_kernel(int M, int N, int K,
                                                           const uint16_t* __restrict__ A,
                                                           const uint8_t* __restrict__ B,
                                                           const uint16_t* __restrict__ zero,
                                                           int rounds_per_wg, RingGemmOut go) {
  ring_body<false, true>(M, N, K, A, B, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, zero,
                         rounds_per_wg, go);
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
  for (int e = seg[2 * nt]; e < seg[2 * nt + 2]; ++e) {
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

// Merge the (max, sum exp) partials of each row (one per vocabulary tile, or per
// half-tile for the bf16 head) into lse.  Many rows:
// one thread per row, reads coalesced across rows.  Few rows: one wave per row,
// lanes stride over the tiles, then a shuffle merge.
__global__ void lse_finalize_kernel(int R, int n_parts, const float2* __restrict__ part,
                                    float* __restrict__ lse) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= R) return;
  float m = -INFINITY, s = 0.f;
#pragma unroll 8
  for (int t = 0; t < n_parts; ++t) {
    const float2 p = part[(size_t)t * R + r];
    lse_merge(m, s, p.x, p.y);
  }
  lse[r] = m + logf(s);
}

__global__ __launch_bounds__(256) void lse_finalize_wave_kernel(int R, int n_parts,
                                                                const float2* __restrict__ part,
                                                                float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  float m = -INFINITY, s = 0.f;
  // eight loads in flight per lane before they are merged
  for (int t0 = lane; t0 < n_parts; t0 += 64 * 8) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = t0 + 64 * u;
      p[u] = t < n_parts ? part[(size_t)t * R + r] : float2{-INFINITY, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) lse_merge(m, s, p[u].x, p[u].y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) lse[r] = m + logf(s);
}

// Few rows (partials stored row-major by the matrix-core head): one workgroup per
// row, every thread with its own strided share of the row's partials (all loads
// issued before the merges), then a workgroup merge.
__global__ __launch_bounds__(256) void lse_finalize_block_kernel(int R, int n_parts,
                                                                 const float2* __restrict__ part,
                                                                 float* __restrict__ lse) {
  __shared__ float2 red[4];
  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  float m = -INFINITY, s = 0.f;
  const float2* pr = part + (size_t)r * n_parts;  // this row's partials, contiguous
  for (int t0 = t; t0 < n_parts; t0 += 256 * 8) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = t0 + 256 * u;
      p[u] = k < n_parts ? pr[k] : float2{-INFINITY, 0.f};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) lse_merge(m, s, p[u].x, p[u].y);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
    lse_merge(m, s, m2, s2);
  }
  if (lane == 0) red[wave] = float2{m, s};
  __syncthreads();
  if (t == 0) {
    for (int w = 1; w < 4; ++w) lse_merge(m, s, red[w].x, red[w].y);
    lse[r] = m + logf(s);
  }
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

// Rounds of 256 tiles per bf16-head workgroup: long enough to amortise the
// prologue and launch, short enough that the workgroups sharing operand tiles in
// an XCD's L2 stay within a few rounds of each other (measured on MI355X: 8 is
// 9% faster than a fully persistent grid on a 97k-row head, 2% faster than 1).
static int head_rounds_per_wg(int /*rounds*/) { return 8; }

// 256 x d zeros for the padding steps of the bf16 head when d / 64 is not a
// multiple of 5 (else none).  The W8A8 head's steps are 128 codes: when d / 128
// is not a multiple of 5, d / 64 = 2 d / 128 is not either, so the zeros exist.
static size_t head_zero_bytes(int32_t d) {
  const int nk = d / DMA_BK;
  return nk % 5 == 0 ? 0 : size_t(256) * d * 2;
}

// Per-label-set part of the head's workspace: the edge segment table (fp32 head),
// the zero block and the gather lists (matrix-core head), for batches of B documents.
struct HeadPrep {
  int32_t* seg;
  uint4* zero;
  int32_t* list_head;
  int4* rec;
};
static HeadPrep head_prep_layout(Carve& cv, tcs_dtype h_dtype, int32_t B, int32_t n_int,
                                 int32_t n_nodes, int32_t d, int32_t V) {
  const size_t R = size_t(B) * n_int;
  const size_t n_tiles = size_t(lmhead_n_tiles(h_dtype, V));
  const bool mfma_head = h_dtype == TCS_BF16;
  const size_t n_rbl = (R + HEAD_LIST_ROWS - 1) / HEAD_LIST_ROWS;
  HeadPrep P;
  P.seg = cv.take<int32_t>(2 * n_tiles + 1);
  P.zero = cv.take<uint4>(mfma_head ? head_zero_bytes(d) / 16 : 0);
  P.list_head = cv.take<int32_t>(mfma_head ? 2 * n_tiles * n_rbl : 0);
  P.rec = cv.take<int4>(mfma_head ? size_t(n_nodes - 1) * B : 0);
  return P;
}

// Rows per tile of the matrix-core head: the size whose busiest workgroup (tiles
// dealt over HEAD_WGS slots) finishes first, a 128-row tile taking 0.56 of a
// 256-row tile's time.  Measured on MI355X, long-document head (V = 151,936, d =
// 2,560, fp8 W), ms per launch with 256- / 128-row tiles: 256 rows 0.260 / 0.254,
// 384 rows 0.367 / 0.345, 512 rows 0.395 / 0.447, 640 rows 0.514 / 0.517, 1,024
// rows 0.704 / 0.785 (the ratio 0.56 is the last pair's per tile); 128 rows take
// 0.145 with 128-row tiles.
static int head_tile_rows(int R, int n_vt) {
  const long busiest256 = ((R + 255) / 256 * long(n_vt) + HEAD_WGS - 1) / HEAD_WGS;
  const long busiest128 = ((R + 127) / 128 * long(n_vt) + HEAD_WGS - 1) / HEAD_WGS;
  return busiest128 * 56 < busiest256 * 100 ? 128 : 256;
}

template <bool W8, bool A8>
static void launch_ring_head(int TR, int grid, hipStream_t s, int R, int V, int d, const uint16_t* h,
                             const uint8_t* W, const float* w_scale, const float* h_scale,
                             const HeadPrep& P, float* lp, float2* part, const uint16_t* zero,
                             int per) {
  if (TR == 128)
    lmhead_ring_kernel<W8, A8, 128><<<grid, 64 * RING_WAVES, 0, s>>>(
        R, V, d, h, W, w_scale, h_scale, P.list_head, P.rec, lp, part, zero, per);
  else
    lmhead_ring_kernel<W8, A8, 256><<<grid, 64 * RING_WAVES, 0, s>>>(
        R, V, d, h, W, w_scale, h_scale, P.list_head, P.rec, lp, part, zero, per);
}

size_t lmhead_prep_bytes(tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t n_nodes, int32_t d,
                         int32_t V) {
  Carve cv(nullptr);
  head_prep_layout(cv, h_dtype, B, n_int, n_nodes, d, V);
  return cv.used;
}

size_t lmhead_part_bytes(tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t V) {
  const size_t parts = size_t(lmhead_n_tiles(h_dtype, V)) * (h_dtype == TCS_BF16 ? 2 : 1);
  return align_up(parts * size_t(B) * n_int * 8);
}

size_t lmhead_ws_bytes(tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                       int32_t n_nodes, int32_t d, int32_t V) {
  return lmhead_prep_bytes(h_dtype, B, n_int, n_nodes, d, V) + lmhead_part_bytes(h_dtype, B, n_int, V) +
         lmhead_act8_bytes(w_dtype, B * n_int, d);
}

int launch_lmhead_prep(void* stream, tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t n_nodes,
                       int32_t d, int32_t V, const int32_t* e_tok, const int32_t* e_qrow,
                       const int32_t* e_child, int32_t n_edges, void* prep) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = B * n_int;
  if (R <= 0) return TCS_OK;
  const int n_tiles = lmhead_n_tiles(h_dtype, V);
  Carve cv(prep);
  const HeadPrep P = head_prep_layout(cv, h_dtype, B, n_int, n_nodes, d, V);
  const bool mfma_head = h_dtype == TCS_BF16;
  const size_t zbytes = mfma_head ? head_zero_bytes(d) : 0;
  const int n_rbl = (R + HEAD_LIST_ROWS - 1) / HEAD_LIST_ROWS;
  const int n_keys = mfma_head ? 2 * n_tiles * n_rbl : 0;
  const long n_pairs = mfma_head ? long(n_edges) * B : 0;
  const int n_prep = max(2 * n_tiles + 1, int(zbytes / 16));
  head_prep_kernel<<<(n_prep + 255) / 256, 256, 0, s>>>(2 * n_tiles, e_tok, n_edges, P.seg, P.zero,
                                                        int(zbytes / 16));
  if (mfma_head) {
    head_list_init_kernel<<<(n_keys + 255) / 256, 256, 0, s>>>(n_keys, P.list_head);
    if (n_pairs > 0)
      head_list_link_kernel<<<int((n_pairs + 255) / 256), 256, 0, s>>>(
          B, n_int, n_nodes, n_rbl, e_tok, e_qrow, e_child, n_edges, P.list_head, P.rec);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead prep: %s", hipGetErrorString(e));
  return TCS_OK;
}

// E4M3FN code of a finite fp32 value: the nearest E4M3 value, ties to the even
// code (rintf rounds half to even), magnitudes from 448 up saturating to 448.
__device__ __forceinline__ uint32_t e4m3_rne(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 31) << 7;
  const float a = fabsf(q);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7E;
  } else if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (8 steps is the smallest normal)
    code = uint32_t(rintf(a * 512.0f));
  } else {  // a in [2^E, 2^(E+1)), E in [-6, 8]: mantissa steps of 2^(E-3)
    const int E = int((__float_as_uint(a) >> 23) & 0xFF) - 127;
    const float m = rintf(a * __uint_as_float(uint32_t(127 - E) << 23) * 8.0f) - 8.0f;  // 0..8
    code = uint32_t((E + 7) * 8 + int(m));  // m = 8 carries into the exponent
  }
  return code | sign;
}

// One wave per hidden row: s = max|h| / 448 and codes E4M3(h / s), both divisions
// correctly rounded; an all-zero row gets s = 0 and zero codes.  d % 4 == 0.
__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(int R, int d, const uint16_t* __restrict__ h,
                                                              uint32_t* __restrict__ q,
                                                              float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= R) return;
  const uint2* hr = reinterpret_cast<const uint2*>(h + (size_t)row * d);
  float amax = 0.f;
  for (int k4 = lane; k4 < d / 4; k4 += 64) {
    const uint2 v = hr[k4];
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_to_f32(uint16_t(v.x))), fabsf(bf16_to_f32(uint16_t(v.x >> 16)))),
                             fmaxf(fabsf(bf16_to_f32(uint16_t(v.y))), fabsf(bf16_to_f32(uint16_t(v.y >> 16))))));
  }
  amax = wave_max(amax);
  const float s = __fdiv_rn(amax, 448.0f);
  if (lane == 0) scale[row] = s;
  uint32_t* qr = q + (size_t)row * (d / 4);
  for (int k4 = lane; k4 < d / 4; k4 += 64) {
    const uint2 v = hr[k4];
    const float x[4] = {bf16_to_f32(uint16_t(v.x)), bf16_to_f32(uint16_t(v.x >> 16)),
                        bf16_to_f32(uint16_t(v.y)), bf16_to_f32(uint16_t(v.y >> 16))};
    uint32_t packed = 0;
    if (s > 0.f) {
#pragma unroll
      for (int t = 0; t < 4; ++t) packed |= e4m3_rne(__fdiv_rn(x[t], s)) << (8 * t);
    }
    qr[k4] = packed;
  }
}

size_t lmhead_act8_bytes(tcs_dtype w_dtype, int32_t R, int32_t d) {
  return w_dtype == TCS_FP8_E4M3_A8 ? align_up(size_t(R) * d) + align_up(size_t(R) * 4) : 0;
}

int launch_lmhead_run(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                      int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                      const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                      const int32_t* e_child, float* lse, float* lp, const void* prep, void* part,
                      bool finalize_lp, void* act8) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int R = B * n_int;
  if (R <= 0) return TCS_OK;
  const int n_tiles = lmhead_n_tiles(h_dtype, V);
  Carve cv(const_cast<void*>(prep));
  const HeadPrep P = head_prep_layout(cv, h_dtype, B, n_int, n_nodes, d, V);
  float2* p = static_cast<float2*>(part);
  int n_parts = n_tiles;
  timer_begin(TCS_TIMER_HEAD, stream);
  if (h_dtype == TCS_BF16) {
    if (d % 64 != 0) return fail(TCS_EUNSUPPORTED, "lmhead: d=%d is not a multiple of 64", d);
    const int TR = head_tile_rows(R, n_tiles);
    const int n_rt_k = (R + TR - 1) / TR;
    const int rounds = head_grid(n_rt_k, n_tiles) / HEAD_WGS;
    const int per = head_rounds_per_wg(rounds);
    const int grid = (rounds + per - 1) / per * HEAD_WGS;
    auto hp = static_cast<const uint16_t*>(h);
    auto wp = static_cast<const uint8_t*>(W);
    auto zp = reinterpret_cast<const uint16_t*>(P.zero);
    if (w_dtype == TCS_FP8_E4M3_A8) {
      if (!act8) return fail(TCS_EINVAL, "lmhead: W8A8 head without its activation buffer");
      if (d % 128 != 0) return fail(TCS_EUNSUPPORTED, "lmhead: W8A8 head needs d %% 128 == 0 (d=%d)", d);
      auto codes = static_cast<uint32_t*>(act8);
      auto hs = reinterpret_cast<float*>(static_cast<char*>(act8) + align_up(size_t(R) * d));
      quant_rows_e4m3_kernel<<<(R + 3) / 4, 256, 0, s>>>(R, d, hp, codes, hs);
      launch_ring_head<true, true>(TR, grid, s, R, V, d, reinterpret_cast<const uint16_t*>(codes), wp,
                                   w_scale, hs, P, lp, p, zp, per);
    } else if (w_dtype == TCS_FP8_E4M3) {
      launch_ring_head<true, false>(TR, grid, s, R, V, d, hp, wp, w_scale, nullptr, P, lp, p, zp, per);
    } else {
      launch_ring_head<false, false>(TR, grid, s, R, V, d, hp, wp, nullptr, nullptr, P, lp, p, zp, per);
    }
    n_parts = 2 * n_tiles;
  } else {
    dim3 grid(n_tiles, (R + 7) / 8);
    lmhead_f32_kernel<<<grid, 256, 0, s>>>(R, V, d, n_int, n_nodes, static_cast<const float*>(h),
                                           static_cast<const float*>(W), P.seg, e_tok, e_qrow, e_child,
                                           lp, p);
  }
  timer_end(TCS_TIMER_HEAD, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead: %s", hipGetErrorString(e));
  if (h_dtype == TCS_BF16 && R < LSE_ROWMAJOR_MAX_ROWS)
    lse_finalize_block_kernel<<<R, 256, 0, s>>>(R, n_parts, p, lse);
  else if (R < 16384)
    lse_finalize_wave_kernel<<<(R + 3) / 4, 256, 0, s>>>(R, n_parts, p, lse);
  else
    lse_finalize_kernel<<<(R + 255) / 256, 256, 0, s>>>(R, n_parts, p, lse);
  if (finalize_lp) {
    const long nlp = long(B) * n_nodes;
    lp_finalize_kernel<<<int((nlp + 255) / 256), 256, 0, s>>>(B, n_int, n_nodes, e_qrow, e_child,
                                                               lse, lp);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "lmhead finalize: %s", hipGetErrorString(e));
  return TCS_OK;
}

size_t gemm_ring_zero_bytes(int32_t K) {
  const int nk = K / DMA_BK;
  return nk % 5 == 0 ? 0 : size_t(256) * K * 2;
}

bool gemm_ring_ok(int32_t M, int32_t N, int32_t K) {
  return K % DMA_BK == 0 && K <= 65536 && N % 4 == 0 &&
         long((M + 255) / 256) * ((N + 255) / 256) >= 512;
}

int launch_gemm_ring_resid(void* stream, int32_t M, int32_t N, int32_t K, const void* A,
                           const void* B, float* C, int32_t ldc, const GemmResid& res,
                           const void* zero) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int n_rt = (M + 255) / 256, n_vt = (N + 255) / 256;
  const int rounds = (n_rt * n_vt + HEAD_WGS - 1) / HEAD_WGS;
  const int per = head_rounds_per_wg(rounds);
  const int grid = (rounds + per - 1) / per * HEAD_WGS;
  const RingGemmOut go{C, ldc, static_cast<const uint16_t*>(res.E), res.token, res.qnode, res.n_int};
  proj_ring_kernel<<<grid, 64 * RING_WAVES, 0, s>>>(M, N, K, static_cast<const uint16_t*>(A),
                                        static_cast<const uint8_t*>(B),
                                        static_cast<const uint16_t*>(zero), per, go);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "gemm ring: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_lmhead(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                  int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                  const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                  const int32_t* e_child, int32_t n_edges, float* lse, float* lp, void* ws) {
  // workspace: [prepared gather lists | partials | fp8 codes and scales of h (W8A8)]
  const size_t pb = lmhead_prep_bytes(h_dtype, B, n_int, n_nodes, d, V);
  const size_t qb = lmhead_part_bytes(h_dtype, B, n_int, V);
  if (int rc = launch_lmhead_prep(stream, h_dtype, B, n_int, n_nodes, d, V, e_tok, e_qrow, e_child,
                                  n_edges, ws))
    return rc;
  void* act8 = w_dtype == TCS_FP8_E4M3_A8 ? static_cast<char*>(ws) + pb + qb : nullptr;
  return launch_lmhead_run(stream, h_dtype, w_dtype, B, n_int, n_nodes, d, V, h, W, w_scale, e_tok,
                           e_qrow, e_child, lse, lp, ws, static_cast<char*>(ws) + pb, true, act8);
}

}  // namespace tcs
