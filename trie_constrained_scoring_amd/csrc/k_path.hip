// Per-label path sums, label softmax and argmax.
//
// "To Classify, Try a Trie Tree", section 3.2: a label's score is the product of
// its token probabilities, so its log score is the sum of the edge log-probs on
// its root-to-label path; a label that ends where other labels continue is also
// multiplied by the probability of not continuing; scores are divided by their
// sum over labels.  Section 2: the operator always returns one label.
#include <algorithm>
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

// Entry i of an fp32 array of n entries, 0 when i is outside [0, n) (the buffer
// unit drops the load), with no branch around it.
__device__ __forceinline__ float gather_load(const float* base, int n, int i) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, n * 4, 0x00020000);
  const uint32_t off = uint32_t(i) < uint32_t(n) ? uint32_t(i) * 4u : 0x80000000u;
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
__device__ __forceinline__ int gather_load_i32(const int32_t* base, int n, int i) {
  return int(__float_as_uint(gather_load(reinterpret_cast<const float*>(base), n, i)));
}

// Deep tries (depth >= PATH_STAGE_DEPTH, up to PATH_STAGE_NODES nodes) take the
// staged walk below; shallow ones walk the global arrays directly.
constexpr int PATH_STAGE_DEPTH = 8;
constexpr int PATH_STAGE_NODES = 8192;  // 4 bytes of LDS each
constexpr int PATH_WALK_BATCH = 8;      // path nodes whose log-probs are requested together

// One workgroup per document; each thread walks the paths of its labels from the
// label node up to the root, accumulating in fp64.  With `lse` set, lp holds the
// raw child logits and the edge log-prob of node v is lp[v] - lse[b n_int +
// node_qrow[v]] (the head's finalisation folded in).
// STAGED: the parent and parent-row arrays are first copied to LDS (uint16), so
// the chain of parent reads runs in LDS, and the log-probs of PATH_WALK_BATCH path
// nodes at a time are requested together: a depth-40 path costs five rounds of
// global loads instead of forty dependent ones.  The sum runs in the same order
// either way, so both forms give the same bits.
template <bool STAGED>
__global__ __launch_bounds__(256) void path_sum_kernel(
    int n_nodes, int M, const float* __restrict__ lp, const float* __restrict__ lse,
    const int32_t* __restrict__ node_qrow, int n_int, const int32_t* __restrict__ parent,
    const int32_t* __restrict__ child_begin, const int32_t* __restrict__ child_count,
    const int32_t* __restrict__ label_node, float* __restrict__ ll, float* __restrict__ prob,
    int32_t* __restrict__ label) {
  __shared__ double rv[4];
  __shared__ int ri[4];
  __shared__ double rs[4];
  extern __shared__ uint16_t walk_lds[];  // STAGED: parent [n_nodes] | parent's row [n_nodes]
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* lpb = lp + (size_t)b * n_nodes;
  const float* lseb = lse ? lse + (size_t)b * n_int : nullptr;
  auto edge_lp = [&](int v) -> double {
    const double x = double(lpb[v]);
    return lseb ? x - double(lseb[node_qrow[v]]) : x;
  };
  uint16_t* const spn = walk_lds;
  uint16_t* const sqr = walk_lds + n_nodes;
  if constexpr (STAGED) {
    constexpr int CH = 8;  // loads in flight per thread and array
    for (int v0 = 0; v0 < n_nodes; v0 += CH * 256) {
      int pv[CH], qv[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) pv[i] = gather_load_i32(parent, n_nodes, v0 + t + 256 * i);
      if (lseb) {
#pragma unroll
        for (int i = 0; i < CH; ++i) qv[i] = gather_load_i32(node_qrow, n_nodes, v0 + t + 256 * i);
      } else {
#pragma unroll
        for (int i = 0; i < CH; ++i) qv[i] = 0;
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int v = v0 + t + 256 * i;
        if (v < n_nodes) {
          spn[v] = uint16_t(v == 0 ? 0 : pv[i]);
          sqr[v] = uint16_t(v == 0 ? 0 : qv[i]);
        }
      }
    }
    __syncthreads();
  }
  float* llb = ll + (size_t)b * M;
  double best = -HUGE_VAL;
  int best_i = INT_MAX;
  for (int m = t; m < M; m += 256) {
    const int u = label_node[m];
    double acc = 0.0;
    if constexpr (STAGED) {
      int v = u, steps = 0;
      while (v > 0 && steps < u) {
        // the next nodes of the path and their parents' rows (-1 past the root)
        int vs[PATH_WALK_BATCH], qs[PATH_WALK_BATCH];
#pragma unroll
        for (int i = 0; i < PATH_WALK_BATCH; ++i) {
          const bool on = v > 0 && steps < u;
          vs[i] = on ? v : -1;
          qs[i] = -1;
          if (on) {
            qs[i] = sqr[v];
            v = spn[v];
            ++steps;
          }
        }
        float x[PATH_WALK_BATCH], ls[PATH_WALK_BATCH];
#pragma unroll
        for (int i = 0; i < PATH_WALK_BATCH; ++i) x[i] = gather_load(lpb, n_nodes, vs[i]);
        if (lseb) {
#pragma unroll
          for (int i = 0; i < PATH_WALK_BATCH; ++i) ls[i] = gather_load(lseb, n_int, qs[i]);
#pragma unroll
          for (int i = 0; i < PATH_WALK_BATCH; ++i)
            if (vs[i] >= 0) acc += double(x[i]) - double(ls[i]);
        } else {
#pragma unroll
          for (int i = 0; i < PATH_WALK_BATCH; ++i)
            if (vs[i] >= 0) acc += double(x[i]);
        }
      }
    } else {
      for (int v = u, steps = 0; v > 0 && steps < u; v = parent[v], ++steps) acc += edge_lp(v);
    }
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

// ---------------------------------------------------------------- by levels
//
// The same sums for tries of up to PATH_MAX_ROWS query rows, organised so that a
// document's lp row is read once, coalesced, and nothing waits on a chain of
// dependent loads.  Every internal node's prefix sum S(v) = S(parent v) + lp(v) is
// shared by the labels below it; query rows follow node order, so the rows of one
// depth are contiguous and their parents lie one depth up.  A persistent
// workgroup of 512 threads takes documents blockIdx.x, blockIdx.x + gridDim.x, ...:
//   1. each internal node's edge log-prob goes to LDS at its row (thread t holds lp
//      of nodes t + 512 k in registers, loaded while the previous document was
//      scored);
//   2. depth by depth, S(row) += S(parent row) (parent rows kept in LDS);
//   3. each label reads the prefix sum of its row and adds its own edge (leaf) or
//      the prefix term (internal node), then argmax and softmax as above.
// A prefix sum is kept as an fp32 value plus its bf16 remainder (about 2^-33 of
// the value), so with the uint16 parent row a row costs 8 bytes of LDS; a label's
// score and prefix term are formed in fp64 from it.
constexpr int PATH_THREADS = 512;
constexpr int PATH_KREG = 48;         // lp entries per thread held in registers
constexpr int PATH_LREG = 16;         // labels per thread (so at most 8192 labels)
constexpr int PATH_MAX_ROWS = 19968;  // 8 bytes each
constexpr int PATH_MAX_LEVELS = 256;
constexpr int PATH_PROWS = (PATH_MAX_ROWS + PATH_THREADS - 1) / PATH_THREADS;  // parent rows per thread
// Up to this many labels the per-label walk is faster (measured on MI355X per
// launch, walk vs levels: 10 labels 7 vs 20 us, 255 labels 22 vs 36 us, 5,000
// labels 151 vs 50 us; since then the staged walk takes 13 us at 255 labels and
// the batched set-up loads bring the levels kernel to 35 us at 5,000): it has
// no level barriers, and each thread walks about one label.
constexpr int PATH_WALK_MAX_LABELS = 512;

// A sum held as an unevaluated pair hi + lo of fp32 values (lo stored as bf16),
// added with error-free fp32 transformations (Knuth's TwoSum, then a fast
// renormalisation): about 2^-33 relative error per addition.
struct F2 {
  float h, l;
};
__device__ __forceinline__ F2 two_sum(float a, float b) {
  const float s = a + b, bb = s - a;
  return F2{s, (a - (s - bb)) + (b - bb)};
}
__device__ __forceinline__ F2 f2_add(F2 a, F2 b) {
  const F2 s = two_sum(a.h, b.h);
  const float t = s.l + (a.l + b.l);
  const float h = s.h + t;
  return F2{h, t - (h - s.h)};
}
__device__ __forceinline__ F2 sum_get(const float* hi, const uint16_t* lo, int r) {
  return F2{hi[r], __uint_as_float(uint32_t(lo[r]) << 16)};
}
__device__ __forceinline__ void sum_put(float* hi, uint16_t* lo, int r, F2 s) {
  hi[r] = s.h;
  lo[r] = f32_to_bf16(s.l);
}
// Dword k (0 <= k < PATH_KREG) of this thread's share of an int32/fp32 row of n
// entries: entry t + 512 k, 0 past the end (outside the buffer's range).
__device__ __forceinline__ uint32_t row_load(const void* base, int n, int t, int k) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n * 4, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b32(rs, t * 4, k * PATH_THREADS * 4, 0);
}

// LDS writes before, LDS reads after; outstanding global loads stay in flight
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ __launch_bounds__(PATH_THREADS) void path_levels_kernel(
    int B, int n_nodes, int n_int, int M, int max_depth, const float* __restrict__ lp,
    const float* __restrict__ lse, const int32_t* __restrict__ qrow,
    const int32_t* __restrict__ qparent, const int32_t* __restrict__ row_level_offsets,
    const int32_t* __restrict__ label_node, const int32_t* __restrict__ label_row,
    const int32_t* __restrict__ child_begin, const int32_t* __restrict__ child_count,
    float* __restrict__ ll, float* __restrict__ prob, int32_t* __restrict__ label) {
  extern __shared__ __attribute__((aligned(16))) uint8_t path_lds[];
  float* shi = reinterpret_cast<float*>(path_lds);          // [n_int]
  uint16_t* slo = reinterpret_cast<uint16_t*>(shi + n_int);  // [n_int]
  uint16_t* spar = slo + n_int;                              // [n_int]
  __shared__ int slev[PATH_MAX_LEVELS];
  __shared__ float rv[PATH_THREADS / 64];
  __shared__ double rs[PATH_THREADS / 64];
  __shared__ int ri[PATH_THREADS / 64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Set-up.  Every load that does not depend on another is requested before any
  // is used (a loop of one load and one LDS write per row waits for each load in
  // turn): the parent rows (into LDS), the level offsets, this thread's node rows
  // t + 512 k (0 past the end) and label nodes and rows t + 512 j; then, with the
  // nodes, whether each label node is a leaf.  Node rows are packed two to a
  // register (0xFFFF for a leaf), a label as node | row << 16 | leaf << 31 (nodes
  // and rows are below 2^15 here).
  int pv[PATH_PROWS];
#pragma unroll
  for (int i = 0; i < PATH_PROWS; ++i) pv[i] = gather_load_i32(qparent, n_int, t + i * PATH_THREADS);
  const int lvo = gather_load_i32(row_level_offsets, max_depth + 2, t);
  uint32_t qr2[PATH_KREG / 2];
#pragma unroll
  for (int k = 0; k < PATH_KREG; k += 2)
    qr2[k / 2] = (row_load(qrow, n_nodes, t, k) & 0xFFFFu) | (row_load(qrow, n_nodes, t, k + 1) << 16);
  int lnode[PATH_LREG], lrow[PATH_LREG];
#pragma unroll
  for (int j = 0; j < PATH_LREG; ++j) {
    lnode[j] = gather_load_i32(label_node, M, t + PATH_THREADS * j);
    lrow[j] = gather_load_i32(label_row, M, t + PATH_THREADS * j);
  }
#pragma unroll
  for (int i = 0; i < PATH_PROWS; ++i) {
    const int r = t + i * PATH_THREADS;
    if (r < n_int) spar[r] = uint16_t(r == 0 ? 0 : pv[i]);
  }
  if (t < max_depth + 2) slev[t] = lvo;
  uint32_t lab[PATH_LREG];
  {
    int cc[PATH_LREG];
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j)
      cc[j] = gather_load_i32(child_count, n_nodes, t + PATH_THREADS * j < M ? lnode[j] : -1);
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      const bool lf = t + PATH_THREADS * j >= M || cc[j] == 0;
      lab[j] = uint32_t(lnode[j]) | (uint32_t(lrow[j]) << 16) | (lf ? 0x80000000u : 0u);
    }
  }
  const bool any_internal = __syncthreads_or(int(
      [&] {
        bool a = false;
#pragma unroll
        for (int j = 0; j < PATH_LREG; ++j) a |= (lab[j] >> 31) == 0;
        return a;
      }()));
  auto lab_u = [&](int j) { return int(lab[j] & 0xFFFFu); };
  auto lab_r = [&](int j) { return int((lab[j] >> 16) & 0x7FFFu); };
  auto lab_leaf = [&](int j) { return (lab[j] >> 31) != 0; };

  float cur[PATH_KREG];
  auto load_row = [&](int bb) __attribute__((always_inline)) {
    const float* p = lp + (size_t)bb * n_nodes;
#pragma unroll
    for (int k = 0; k < PATH_KREG; ++k) cur[k] = __uint_as_float(row_load(p, n_nodes, t, k));
  };
  int b = blockIdx.x;
  if (b < B) load_row(b);
  for (; b < B; b += gridDim.x) {
    const float* lpb = lp + (size_t)b * n_nodes;
    const float* lseb = lse ? lse + (size_t)b * n_int : nullptr;
    // keep the packed values opaque across documents, so that the compiler does
    // not hold every address derived from them live through the loop
#pragma unroll
    for (int k = 0; k < PATH_KREG / 2; ++k) asm volatile("" : "+v"(qr2[k]));
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) asm volatile("" : "+v"(lab[j]));
    lds_barrier();  // parent rows in place; the previous document's reads are done
    // 1. edge log-probs of the internal nodes, by row (the root's row holds 0);
    //    with lse, the parent rows' lse are all requested before any is used
    const int n_lse = lseb ? n_int : 0;
    auto row_of = [&](int k) { return int((qr2[k / 2] >> (16 * (k & 1))) & 0xFFFFu); };
    if (lseb) {
      constexpr int CH = 16;
#pragma unroll
      for (int k0 = 0; k0 < PATH_KREG; k0 += CH) {
        float lsv[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int r = row_of(k0 + i);
          lsv[i] = gather_load(lseb, n_lse, r > 0 && r < 0xFFFF ? int(spar[r]) : -1);
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int r = row_of(k0 + i);
          if (r > 0 && r < 0xFFFF) sum_put(shi, slo, r, two_sum(cur[k0 + i], -lsv[i]));
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < PATH_KREG; ++k) {
        const int r = row_of(k);
        if (r > 0 && r < 0xFFFF) sum_put(shi, slo, r, F2{cur[k], 0.f});
      }
    }
    for (int v = t + PATH_THREADS * PATH_KREG; v < n_nodes; v += PATH_THREADS) {
      const int r = qrow[v];
      if (r > 0) sum_put(shi, slo, r, two_sum(lpb[v], -gather_load(lseb, n_lse, spar[r])));
    }
    if (t == 0) {
      shi[0] = 0.f;
      slo[0] = 0;
    }
    // the labels' own edges and the next document's row are in flight through step 2
    float lpu[PATH_LREG], lsr[PATH_LREG];
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      const bool in = t + PATH_THREADS * j < M;
      lpu[j] = gather_load(lpb, n_nodes, lab_leaf(j) && in ? lab_u(j) : -1);
      lsr[j] = gather_load(lseb, n_lse, in ? lab_r(j) : -1);
    }
    if (b + int(gridDim.x) < B) load_row(b + gridDim.x);
    lds_barrier();
    // 2. prefix sums, one depth at a time (depth 0 is the root)
    // (rows of one depth never read each other, so four at a time, reads first)
    for (int d = 1; d <= max_depth; ++d) {
      const int r1 = slev[d + 1];
      for (int r = slev[d] + t; r < r1; r += 4 * PATH_THREADS) {
        int p[4];
        F2 x[4], y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = r + i * PATH_THREADS < r1 ? spar[r + i * PATH_THREADS] : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = sum_get(shi, slo, p[i]);
          y[i] = r + i * PATH_THREADS < r1 ? sum_get(shi, slo, r + i * PATH_THREADS) : F2{0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r + i * PATH_THREADS < r1) sum_put(shi, slo, r + i * PATH_THREADS, f2_add(x[i], y[i]));
      }
      lds_barrier();
    }
    // 3. labels: a leaf adds its own edge; a label that ends at an internal node
    //    adds the prefix term, in a pass of its own (rare: none in prefix-free sets)
    float* llb = ll + (size_t)b * M;
    float llv[PATH_LREG];
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      const int m = t + PATH_THREADS * j;
      const F2 pre = sum_get(shi, slo, lab_r(j));
      llv[j] = m < M ? float(double(pre.h) + double(pre.l) + (double(lpu[j]) - double(lsr[j])))
                     : -INFINITY;
      if (m < M && lab_leaf(j)) llb[m] = llv[j];
    }
    if (any_internal) {
      for (int m = t; m < M; m += PATH_THREADS) {
        const int u = label_node[m], cc = child_count[u];
        if (cc == 0) continue;
        const int r = label_row[m], cb = child_begin[u];
        const double lsr1 = lseb ? double(lseb[r]) : 0.0;
        double mx = -HUGE_VAL;
        for (int c = cb; c < cb + cc; ++c) mx = fmax(mx, double(lpb[c]) - lsr1);
        double se = 0.0;
        for (int c = cb; c < cb + cc; ++c) se += exp(double(lpb[c]) - lsr1 - mx);
        const F2 pre = sum_get(shi, slo, r);
        llb[m] = float(double(pre.h) + double(pre.l) + log1mexp_d(mx + log(se)));
      }
      // this thread wrote the labels it reads back
#pragma unroll
      for (int j = 0; j < PATH_LREG; ++j) {
        const int m = t + PATH_THREADS * j;
        if (m < M && !lab_leaf(j)) llv[j] = llb[m];
      }
    }
    // argmax of the stored scores over the workgroup, lowest label id among equal
    // maxima (labels increase with j, so a strict > keeps the first)
    float best = -INFINITY;
    int best_i = INT_MAX;
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      const int m = t + PATH_THREADS * j;
      if (m < M && (llv[j] > best || best_i == INT_MAX)) {
        best = llv[j];
        best_i = m;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
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
    lds_barrier();
    best = rv[0];
    best_i = ri[0];
    for (int w = 1; w < PATH_THREADS / 64; ++w)
      if (rv[w] > best || (rv[w] == best && ri[w] < best_i)) {
        best = rv[w];
        best_i = ri[w];
      }
    if (t == 0) label[b] = best_i;
    if (!prob) continue;
    // softmax of the stored (fp32) scores against their maximum, in fp32 with the
    // hardware exp2 (arguments <= 0, -inf past M); the sum in fp64
    constexpr float LOG2E = 1.4426950408889634f;
    const float bf = best;
    double sm = 0.0;
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      llv[j] = __builtin_amdgcn_exp2f((llv[j] - bf) * LOG2E);
      sm += llv[j];
    }
    sm = wave_sum_d(sm);
    if (lane == 0) rs[wave] = sm;
    lds_barrier();
    sm = 0.0;
    for (int w = 0; w < PATH_THREADS / 64; ++w) sm += rs[w];
    const float inv = float(1.0 / sm);
    float* pb = prob + (size_t)b * M;
#pragma unroll
    for (int j = 0; j < PATH_LREG; ++j) {
      const int m = t + PATH_THREADS * j;
      if (m < M) pb[m] = llv[j] * inv;
    }
  }
}

static bool path_levels_ok(const tcs_trie_dev* trie) {
  return trie->qrow && trie->qparent && trie->row_level_offsets && trie->label_row &&
         trie->n_int <= PATH_MAX_ROWS &&
         trie->max_depth + 2 <= PATH_MAX_LEVELS && trie->n_labels <= PATH_LREG * PATH_THREADS &&
         trie->n_nodes <= 32768;
}

static int launch_path_levels(hipStream_t s, int32_t B, const tcs_trie_dev* trie, const float* lp,
                              float* ll, float* prob, int32_t* label, const float* lse) {
  const size_t lds = size_t(trie->n_int) * 8;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(path_levels_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             PATH_MAX_ROWS * 8);
    if (e != hipSuccess) return fail(TCS_EHIP, "path_sum: %s", hipGetErrorString(e));
    attr_set = true;
  }
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(TCS_EHIP, "path_sum: device query failed");
  // workgroups per CU: by LDS (static part ~1 KB each), at most 4 (32 waves)
  const int per_cu = int(std::max<size_t>(1, std::min<size_t>(4, (160 * 1024) / (lds + 1024))));
  const int grid = int(std::min<long>(B, long(n_cu) * per_cu));
  path_levels_kernel<<<grid, PATH_THREADS, lds, s>>>(
      B, trie->n_nodes, trie->n_int, trie->n_labels, trie->max_depth, lp, lse, trie->qrow,
      trie->qparent, trie->row_level_offsets, trie->label_node, trie->label_row, trie->child_begin,
      trie->child_count, ll, prob, label);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "path_sum: %s", hipGetErrorString(e));
  return TCS_OK;
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
  if (trie->n_labels > PATH_WALK_MAX_LABELS && path_levels_ok(trie))
    return launch_path_levels(s, B, trie, lp, ll, prob, label, lse);
  if (trie->max_depth >= PATH_STAGE_DEPTH && trie->n_nodes <= PATH_STAGE_NODES)
    path_sum_kernel<true><<<B, 256, size_t(trie->n_nodes) * 4, s>>>(
        trie->n_nodes, trie->n_labels, lp, lse, node_qrow, trie->n_int, trie->parent,
        trie->child_begin, trie->child_count, trie->label_node, ll, prob, label);
  else
    path_sum_kernel<false><<<B, 256, 0, s>>>(trie->n_nodes, trie->n_labels, lp, lse, node_qrow,
                                             trie->n_int, trie->parent, trie->child_begin,
                                             trie->child_count, trie->label_node, ll, prob, label);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "path_sum: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
