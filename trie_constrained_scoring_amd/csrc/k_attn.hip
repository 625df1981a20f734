// Ancestor-masked tree attention.
//
// "To Classify, Try a Trie Tree", section 3.2 ("Custom attention kernel"): one
// request carries every answer node of a document, and a node's keys are the
// document's plus those of its ancestors and itself, never a sibling branch's.  The
// scores of a node against its ancestor chain do not depend on the document, so
// they are reduced once per trie to a softmax partial (max, sum, weighted value
// sum) per (node, head).  The document
// part is a dense attention of every node query against the document's keys; its
// online-softmax state is merged with the path partial by log-sum-exp at the end,
// the same combine that "Building an Ultra-High Throughput AI-SQL Engine"
// (section 3.2.4) applies to its two attention calls for joins.
#include <algorithm>
#include <type_traits>
#include <cstdio>

#include "tcs_device.h"
#include "tcs_internal.h"

namespace tcs {

constexpr float LOG2E = 1.4426950408889634f;

// Two floats -> packed bf16 (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- fp32 path
// One wave per (document, query row, head): keys are the document's keys, then
// the path from the row up to the root.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_simt_kernel(
    int B, int n_int, int Hq, int Hkv, const T* __restrict__ Qn, const T* __restrict__ Kn,
    const T* __restrict__ Vn, const T* __restrict__ Kd, const T* __restrict__ Vd,
    const int32_t* __restrict__ doc_offsets, const int32_t* __restrict__ qparent, float scale,
    T* __restrict__ O, const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel) {
  constexpr int E = HD / 64;
  const int lane = threadIdx.x & 63;
  const long gw = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gw >= long(B) * n_int * Hq) return;
  const int h = int(gw % Hq);
  const int r = int((gw / Hq) % n_int);
  const int b = int(gw / (long(Hq) * n_int));
  const int g = h / (Hq / Hkv);
  // with sel: slot b scores document sel[2b] at query row sel[2b+1] (n_int is 1)
  int doc = b, rr = r;
  if (sel) {
    if (b >= *n_sel) return;
    doc = sel[2 * b];
    rr = sel[2 * b + 1];
  }
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = to_f32(Qn[((size_t)rr * Hq + h) * HD + lane * E + e]);
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const T* k, const T* v) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(q[e], to_f32(k[lane * E + e]), s);
    s = wave_sum(s) * scale;
    const float mn = fmaxf(m, s);
    const float c = __expf(m - mn), p = __expf(s - mn);
    l = l * c + p;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * c + p * to_f32(v[lane * E + e]);
    m = mn;
  };
  for (int j = doc_offsets[doc]; j < doc_offsets[doc + 1]; ++j)
    visit(Kd + ((size_t)j * Hkv + g) * HD, Vd + ((size_t)j * Hkv + g) * HD);
  for (int w = rr, steps = 0; w >= 0 && steps <= rr; w = qparent[w], ++steps)
    visit(Kn + ((size_t)w * Hkv + g) * HD, Vn + ((size_t)w * Hkv + g) * HD);
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < E; ++e)
    O[(((size_t)b * n_int + r) * Hq + h) * HD + lane * E + e] = from_f32<T>(o[e] * inv);
}

// ---------------------------------------------------------------- path partial
// One wave per (query row, head): softmax partial over the row's own path.
// anc_ml[(r*Hq + h)] = (max score, sum exp), anc_o = unnormalised value sum (fp32).
template <typename T, int HD>
__global__ __launch_bounds__(256) void anc_attn_kernel(int n_int, int Hq, int Hkv,
                                                       const T* __restrict__ Qn,
                                                       const T* __restrict__ Kn,
                                                       const T* __restrict__ Vn,
                                                       const int32_t* __restrict__ qparent,
                                                       float scale, float2* __restrict__ anc_ml,
                                                       float* __restrict__ anc_o) {
  constexpr int E = HD / 64;
  const int lane = threadIdx.x & 63;
  const long gw = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (gw >= long(n_int) * Hq) return;
  const int h = int(gw % Hq), r = int(gw / Hq);
  const int g = h / (Hq / Hkv);
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = to_f32(Qn[((size_t)r * Hq + h) * HD + lane * E + e]);
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int w = r, steps = 0; w >= 0 && steps <= r; w = qparent[w], ++steps) {
    const T* k = Kn + ((size_t)w * Hkv + g) * HD;
    const T* v = Vn + ((size_t)w * Hkv + g) * HD;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s = fmaf(q[e], to_f32(k[lane * E + e]), s);
    s = wave_sum(s) * scale;
    const float mn = fmaxf(m, s);
    const float c = __expf(m - mn), p = __expf(s - mn);
    l = l * c + p;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * c + p * to_f32(v[lane * E + e]);
    m = mn;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) anc_o[(size_t)gw * HD + lane * E + e] = o[e];
  if (lane == 0) anc_ml[gw] = float2{m, l};
}

// ---------------------------------------------------------------- document part (MFMA)
//
// Workgroup: one document b, one KV head g, and 32*WR query rows of that head
// (row j = node * G + hh, G = Hq/Hkv query heads per KV head).  4 waves laid out
// WR (row blocks of 32) x WK (key tiles of 32).  Each iteration stages WK*32 keys
// into LDS: keys in their natural [key][hd] layout, values transposed to
// [hd][key] so both MFMA operands read 8 consecutive contraction elements.
//
// Per wave, with v_mfma_f32_32x32x16_bf16:
//   S^T[key][row] = K . Q^T  (A = K from LDS, B = Q^T from registers)
//     -> lane l holds row l%32 and keys 8j + 4(l/32) + i, so the softmax row
//        statistics stay in the lane (plus its partner lane l^32);
//   O^T[hd][row] += V^T . P^T (A = V^T from LDS, B = P^T straight from the S^T
//     registers, with the same key order on both operands).
template <int HD, int WR, int WK>
__global__ __launch_bounds__(256) void doc_attn_mfma_kernel(
    int n_int, int Hq, int Hkv, const uint16_t* __restrict__ Qn, const uint16_t* __restrict__ Kd,
    const uint16_t* __restrict__ Vd, const int32_t* __restrict__ doc_offsets,
    const float2* __restrict__ anc_ml, const float* __restrict__ anc_o, float scale,
    uint16_t* __restrict__ O) {
  static_assert(WR * WK == 4, "4 waves");
  constexpr int KT = 32 * WK;        // keys per stage
  constexpr int LDK = HD + 8;        // sK row (bf16)
  constexpr int LDV = KT + 8;        // sVt row (bf16)
  constexpr int STAGE = KT * LDK + HD * LDV;
  constexpr int K_CH = KT * (HD / 8) / 256;              // K chunks per thread
  constexpr int V_GROUPS = (KT / 4) * (HD / 8);          // 4 keys x 8 hd groups
  constexpr int V_GR = (V_GROUPS + 255) / 256;
  constexpr int NBLK = HD / 32;      // O^T blocks
  constexpr int KSTEPS = HD / 16;
  static_assert(K_CH * 256 == KT * (HD / 8), "K staging");
  constexpr int MERGE_FLOATS = WR * WK * 32 * (HD + 1) + WR * WK * 32 * 2;
  constexpr int LDS_BYTES = (2 * STAGE * 2 > MERGE_FLOATS * 4) ? 2 * STAGE * 2 : MERGE_FLOATS * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LDS_BYTES];
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);

  const int G = Hq / Hkv;
  const int rows_total = n_int * G;
  const int n_rb = (rows_total + 32 * WR - 1) / (32 * WR);
  const int rb = blockIdx.x % n_rb;
  const int g = (blockIdx.x / n_rb) % Hkv;
  const int b = blockIdx.x / (n_rb * Hkv);
  const int j0 = rb * 32 * WR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave / WK, wk = wave % WK;
  const int doc0 = doc_offsets[b];
  const int L = doc_offsets[b + 1] - doc0;

  // Q^T fragments for this wave's 32 rows (lane: row l%32, hd 16*ks + 8*(l/32) ..)
  bf16x8 qf[KSTEPS];
  {
    const int j = j0 + wr * 32 + (lane & 31);
    const bool ok = j < rows_total;
    const int r = ok ? j / G : 0, h = g * G + (ok ? j % G : 0);
    const uint16_t* qp = Qn + ((size_t)r * Hq + h) * HD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : uint4{0, 0, 0, 0};
      qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  uint4 rk[K_CH];
  uint4 rv[V_GR][4];
  auto load_stage = [&](int key0) {
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int kk = c / (HD / 8), hc = c % (HD / 8);
      const int key = key0 + kk;
      rk[i] = key < L ? *reinterpret_cast<const uint4*>(Kd + ((size_t)(doc0 + key) * Hkv + g) * HD + hc * 8)
                      : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < V_GR; ++i) {
      const int gi = tid + i * 256;
      const int kg = gi / (HD / 8), hc = gi % (HD / 8);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int key = key0 + kg * 4 + t;
        rv[i][t] = (gi < V_GROUPS && key < L)
                       ? *reinterpret_cast<const uint4*>(Vd + ((size_t)(doc0 + key) * Hkv + g) * HD + hc * 8)
                       : uint4{0, 0, 0, 0};
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* sK = lds + buf * STAGE;
    uint16_t* sV = sK + KT * LDK;
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int kk = c / (HD / 8), hc = c % (HD / 8);
      *reinterpret_cast<uint4*>(sK + kk * LDK + hc * 8) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_GR; ++i) {
      const int gi = tid + i * 256;
      if (gi >= V_GROUPS) continue;
      const int kg = gi / (HD / 8), hc = gi % (HD / 8);
      const uint32_t w[4][4] = {{rv[i][0].x, rv[i][0].y, rv[i][0].z, rv[i][0].w},
                                {rv[i][1].x, rv[i][1].y, rv[i][1].z, rv[i][1].w},
                                {rv[i][2].x, rv[i][2].y, rv[i][2].z, rv[i][2].w},
                                {rv[i][3].x, rv[i][3].y, rv[i][3].z, rv[i][3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t k0 = (w[0][e >> 1] >> sh) & 0xFFFFu, k1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t k2 = (w[2][e >> 1] >> sh) & 0xFFFFu, k3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2*>(sV + (hc * 8 + e) * LDV + kg * 4) = uint2{k0 | (k1 << 16), k2 | (k3 << 16)};
      }
    }
  };

  f32x16 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;   // base-2 running max; this lane's share of the sum
  const float qk = scale * LOG2E;

  const int n_it = (L + KT - 1) / KT;
  if (n_it > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int cur = it & 1;
    if (it + 1 < n_it) load_stage((it + 1) * KT);
    const uint16_t* sK = lds + cur * STAGE;
    const uint16_t* sV = sK + KT * LDK;
    // S^T = K Q^T for this wave's 32 keys
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    const uint16_t* kp = sK + (wk * 32 + (lane & 31)) * LDK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp + ks * 16);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
    }
    // online softmax (base 2); keys past the document end are masked
    const int kbase = it * KT + wk * 32;
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      s[e] = key < L ? s[e] * qk : -INFINITY;
      tmax = fmaxf(tmax, s[e]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float c = mn == -INFINITY ? 1.f : exp2f(m - mn);
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = mn == -INFINITY ? 0.f : exp2f(s[e] - mn);
      lsum = lsum * (e == 0 ? c : 1.f) + p[e];
    }
    m = mn;
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] *= c;
    // P^T fragments: keys {8j + 4(l/32) + i}; step 0 takes j = 0,1, step 1 j = 2,3.
    // P is split into a bf16 high part and a bf16 remainder (two MFMAs), which
    // keeps the weights to ~2^-17 relative error instead of bf16's 2^-9.
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float a = p[8 * st + 2 * q2], c2 = p[8 * st + 2 * q2 + 1];
        wh[q2] = pack_bf16(a, c2);
        wl[q2] = pack_bf16(a - __uint_as_float(wh[q2] << 16), c2 - __uint_as_float(wh[q2] & 0xFFFF0000u));
      }
      uint4 uh{wh[0], wh[1], wh[2], wh[3]}, ul{wl[0], wl[1], wl[2], wl[3]};
      ph[st] = *reinterpret_cast<bf16x8*>(&uh);
      pl[st] = *reinterpret_cast<bf16x8*>(&ul);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const uint16_t* vp = sV + (blk * 32 + (lane & 31)) * LDV + wk * 32 + 4 * (lane >> 5);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint2 lo = *reinterpret_cast<const uint2*>(vp + 16 * st);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16 * st + 8);
        uint4 u{lo.x, lo.y, hi.x, hi.y};
        const bf16x8 vf = *reinterpret_cast<bf16x8*>(&u);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph[st], acc[blk], 0, 0, 0);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[st], acc[blk], 0, 0, 0);
      }
    }
    if (it + 1 < n_it) store_stage(cur ^ 1);
    __syncthreads();
  }

  // merge the WK key slices of each row block and the row's path partial
  float* so = reinterpret_cast<float*>(lds_raw);            // [WR*WK][32][HD+1]
  float* sml = so + WR * WK * 32 * (HD + 1);                 // [WR*WK][32][2]
  lsum += __shfl_xor(lsum, 32, 64);
  {
    float* base = so + (size_t)wave * 32 * (HD + 1);
    const int row = lane & 31;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int hd = blk * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        base[row * (HD + 1) + hd] = acc[blk][e];
      }
    if (lane < 32) {
      sml[(wave * 32 + row) * 2 + 0] = m;
      sml[(wave * 32 + row) * 2 + 1] = lsum;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < WR * 32 * HD; idx += 256) {
    const int rw = idx / HD, hd = idx % HD;      // rw: row within the workgroup
    const int wrr = rw / 32, row = rw % 32;
    const int j = j0 + rw;
    if (j >= rows_total) continue;
    const int r = j / G, h = g * G + j % G;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < WK; ++k) M = fmaxf(M, sml[((wrr * WK + k) * 32 + row) * 2]);
    float Ls = 0.f, Os = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int k = 0; k < WK; ++k) {
        const int wv = wrr * WK + k;
        const float f = exp2f(sml[(wv * 32 + row) * 2] - M);
        Ls += f * sml[(wv * 32 + row) * 2 + 1];
        Os += f * so[((size_t)wv * 32 + row) * (HD + 1) + hd];
      }
    }
    const float2 a = anc_ml[(size_t)r * Hq + h];
    const float ma = a.x * LOG2E;
    const float Mt = fmaxf(M, ma);
    const float fd = M == -INFINITY ? 0.f : exp2f(M - Mt);
    const float fa = exp2f(ma - Mt);
    const float num = Os * fd + anc_o[((size_t)r * Hq + h) * HD + hd] * fa;
    const float den = Ls * fd + a.y * fa;
    O[(((size_t)b * n_int + r) * Hq + h) * HD + hd] = f32_to_bf16(num / den);
  }
}

// ---------------------------------------------------------------- document part, few rows
//
// When a trie's query rows for one (document, KV head) fill one or two 32-row
// blocks, the document part is a stream over the document's keys at ~48 FLOP per
// byte of K and V, far below the matrix cores' ridge: the kernel is built to keep
// HBM busy.  One workgroup takes one (document, KV head, 32-row block); each of its
// four waves streams its own 32-key stages (keys [32 t, 32 t + 32) for
// t = wave, wave + 4, ...) through a private LDS ring of NS slots filled by direct
// buffer-to-LDS loads, so the key loop has no workgroup barrier.  With NS = 1 two
// workgroups share a CU and each covers the other's load waits (measured on MI355X:
// 12% faster than NS = 2 with one workgroup per CU on 512-key documents, equal on
// 4096-key ones); the next stage's K is loaded as soon as the scores have read the
// current one, so it is in flight during the softmax and PV.
//
// K and V stay in their natural [key][hd] layout.  In a slot, the 16-byte chunk c
// of key row r sits at position c ^ kv_swz(r mod 16), which puts both the K
// fragment reads (16 key rows per LDS phase) and the transposing reads of V (4 keys
// x 64 bytes per half-wave) on distinct banks.
//   S^T[key][row] = K Q^T   (A = K rows from LDS, B = Q^T in registers): each lane
//     holds one query row and 16 of the 32 keys;
//   O^T[hd][row] += V^T P^T (A = V^T read with ds_read_tr16_b64 straight from the
//     natural V tile, B = P^T from the S^T registers, P split into a bf16 high
//     part and a bf16 remainder, which keeps the weights to ~2^-17 relative error).
// The four waves' key slices and the row's path partial are merged by log-sum-exp
// in the epilogue.

// Online-softmax update of a wave's rows for a new block of keys whose scaled
// row maximum (base 2) is `smax`.  The running maximum m is raised only when some
// row of the wave would exceed it by more than 8 (a factor 256): the block's
// weights exp2(s - m) then stay at most 256, which fp32 sums and the bf16
// high/low split of the weights carry without loss, and the accumulators are
// rescaled a few times per document instead of at every block.  Every quantity
// is relative to the same m, so the normalised result does not depend on when m
// was raised.  m = -inf before the first block (which always raises it).
template <int NB>
__device__ __forceinline__ void lazy_rescale(float& m, float smax, float& lsum, f32x16 (&acc)[NB]) {
  if (__builtin_amdgcn_ballot_w64(smax > m + 8.f) == 0) return;  // wave-uniform
  const float mn = fmaxf(m, smax);
  const float cf = __builtin_amdgcn_exp2f(m - mn);  // 0 while m = -inf, 1 where m stays
  m = mn;
  lsum *= cf;
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] *= cf;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int kv_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Two transposing 8-byte LDS reads (ds_read_tr16_b64) joined into one MFMA operand:
// within each group of 16 lanes, lane i receives element i%4 of the 4-element
// pieces that lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12 point at.
__device__ __forceinline__ bf16x8 lds_read_tr_x2(const uint8_t* p0, const uint8_t* p1) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)TCS_LDS(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)TCS_LDS(p1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  return __builtin_bit_cast(bf16x8, v8i16{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}


// NLD 1 KB buffer-to-LDS loads of one operand stage: load j writes dst + 1 KB j,
// lane i at 16 i, from byte vo[j] of a buffer resource over [base, base + bytes).
template <int NLD>
__device__ __forceinline__ void kv_issue(const uint16_t* base, int bytes, uint8_t* dst,
                                         const int (&vo)[NLD]) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NLD; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, TCS_LDS(dst + j * 1024), 16, vo[j], 0, 0, 0);
}

template <int HD, int NS>
__global__ __launch_bounds__(256, 3 - NS) void doc_attn_stream_kernel(
    int n_int, int Hq, int Hkv, const uint16_t* __restrict__ Qn, const uint16_t* __restrict__ Kd,
    const uint16_t* __restrict__ Vd, const int32_t* __restrict__ doc_offsets,
    const float2* __restrict__ anc_ml, const float* __restrict__ anc_o, float scale,
    uint16_t* __restrict__ O, const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    int S, float2* __restrict__ pml, float* __restrict__ po) {
  static_assert(HD == 128, "256-byte key rows: 16 chunks, one per swizzle position");
  constexpr int KB = 32;                 // keys per stage
  constexpr int ROW = HD * 2;            // bytes per key row
  constexpr int OPB = KB * ROW;          // bytes per operand per stage (8 KB)
  constexpr int NLD = OPB / 1024;        // 1 KB loads per operand per stage
  constexpr int NBLK = HD / 32, KSTEPS = HD / 16;
  // K and V stages live in two distinct arrays, so the compiler can tell that a
  // buffer-to-LDS load into one does not write what is being read from the other
  // (with one array it waits for every such load before the next LDS read).  The
  // merge at the end reuses them: hd 0..63 of the 4 x 32 rows in the K array and hd
  // 64..127 in the V array ([4][32][65] fp32 each), then each (wave, row)'s max
  // and sum after them.
  constexpr int HALF = HD / 2, OUT_LD2 = HALF + 1;
  constexpr int EPI_HALF = 4 * 32 * OUT_LD2 * 4, SML_BYTES = 4 * 32 * 4;
  constexpr int OPS_BYTES = 4 * NS * OPB;
  constexpr int ARR_BYTES = OPS_BYTES > EPI_HALF + SML_BYTES ? OPS_BYTES : EPI_HALF + SML_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t sk_arr[ARR_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sv_arr[ARR_BYTES];

  const int G = Hq / Hkv;
  const int rows_total = n_int * G;
  const int n_rb = (rows_total + 31) / 32;
  // block i -> document i mod B: block i runs on XCD i mod 8, so each XCD reads whole
  // key rows (all KV heads) of its documents
  // S > 1: the S workgroups z of a (document, row block, KV head) take every S-th
  // group of four key stages each and leave (max, sum, unnormalised output)
  // partials for doc_attn_merge_kernel
  const int Bn = int(gridDim.x) / (n_rb * Hkv * S);
  const int b = blockIdx.x % Bn, rest = blockIdx.x / Bn;
  const int rb = rest % n_rb, g = (rest / n_rb) % Hkv, z = rest / (n_rb * Hkv);
  const int vw = z * 4 + __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6), NW = 4 * S;
  // with sel: slot b scores document sel[2b] with the queries and path partials of
  // row sel[2b+1] (n_int is 1); slots from *n_sel on have nothing to do
  int doc = b, rq = 0;
  if (sel) {
    if (b >= *n_sel) return;
    doc = sel[2 * b];
    rq = sel[2 * b + 1];
  }
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = rb * 32;
  const int doc0 = doc_offsets[doc];
  const int L = doc_offsets[doc + 1] - doc0;
  const int RS = Hkv * HD * 2;           // bytes between consecutive keys of one head
  uint8_t* const kring = sk_arr + wave * NS * OPB;  // this wave's K slots
  uint8_t* const vring = sv_arr + wave * NS * OPB;  // and V slots

  // this wave's slots start as zeros, so a key past the document end that no load
  // writes still holds finite values (its weight is 0)
#pragma unroll
  for (int i = 0; i < NS * OPB / (64 * 16); ++i) {
    *reinterpret_cast<uint4*>(kring + (i * 64 + lane) * 16) = uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(vring + (i * 64 + lane) * 16) = uint4{0u, 0u, 0u, 0u};
  }

  // Q^T fragments: lane holds row l%32, hd 16 ks + 8 (l/32) ..
  bf16x8 qf[KSTEPS];
  {
    const int j = j0 + (lane & 31);
    const bool ok = j < rows_total;
    const int r = ok ? j / G : 0, h = g * G + (ok ? j % G : 0);
    const uint16_t* qp = Qn + ((size_t)(rq + r) * Hq + h) * HD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : uint4{0, 0, 0, 0};
      qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  // DMA: load j of an operand fills slot rows 4j .. 4j+3 (1 KB); lane i writes row
  // 4j + i/16 at position i%16, which holds chunk (i%16) ^ kv_swz(row).
  int vo[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int row = 4 * j + (lane >> 4);
    vo[j] = row * RS + (((lane & 15) ^ kv_swz(row & 15)) << 4);
  }
  const uint16_t* const kbase = Kd + ((size_t)doc0 * Hkv + g) * HD;
  const uint16_t* const vbase = Vd + ((size_t)doc0 * Hkv + g) * HD;
  // Stage t into slot s: one buffer resource per stage over its valid keys, so keys
  // past the document end fall outside the range and read nothing.
  // (operand 0: K, 1: V)
  auto issue_op = [&](int t, int s, int op) __attribute__((always_inline)) {
    const int nkeys = min(KB, L - t * KB);
    const int bytes = (nkeys - 1) * RS + ROW;
    const size_t off = (size_t)t * KB * Hkv * HD;
    if (op) kv_issue<NLD>(vbase + off, bytes, vring + s * OPB, vo);
    else kv_issue<NLD>(kbase + off, bytes, kring + s * OPB, vo);
  };
  auto issue = [&](int t, int s) __attribute__((always_inline)) {
    issue_op(t, s, 0);
    issue_op(t, s, 1);
  };

  // fragment offsets inside a slot
  const int kr = lane & 31, c = lane >> 5;
  int ko[KSTEPS];  // K: row kr, chunk 2 ks + c
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) ko[ks] = kr * ROW + (((2 * ks + c) ^ kv_swz(kr & 15)) << 4);
  // V^T by transposing reads: for step st and half q, the 16 lanes of group
  // gq = lane/16 read keys 16 st + 8 q + 4 c + 0..3 at hd 32 blk + 16 (gq%2) + 0..15;
  // as a source lane, lane s of the group points at key (.. + s/4), hd (.. + 4 (s%4)).
  int vof[2][2][NBLK];
  {
    const int s = lane & 15, hsel = (lane >> 4) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int key = 16 * st + 8 * q + 4 * c + (s >> 2);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
          const int chunk = 4 * blk + 2 * hsel + ((s & 3) >> 1);
          vof[st][q][blk] = key * ROW + ((chunk ^ kv_swz(key & 15)) << 4) + 8 * (s & 1);
        }
      }
  }

  f32x16 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // base-2 running max; this lane's share of the sum
  const float qk = scale * LOG2E;

  // after_s runs once the stage's K fragments have all been read (the one-slot
  // loop refills the K half there)
  auto compute = [&](const uint8_t* sl, const uint8_t* vl, int t, auto&& after_s) __attribute__((always_inline)) {
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sl + ko[ks]);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc, 0, 0, 0);
    }
    after_s();
    // online softmax (base 2); only the document's last stage has keys past its
    // end, which are masked (the empty asm keeps this a branch)
    if (t * KB + KB > L) {
      asm volatile("");
      const int kb0 = t * KB + 4 * c;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (kb0 + 8 * (e >> 2) + (e & 3) >= L) sc[e] = -INFINITY;
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sc[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * qk;  // finite: every stage has a valid key
    lazy_rescale(m, tmax, lsum, acc);
    float p[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      p[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], qk, -m));
      lsum += p[e];
    }
    // P^T fragments: step st takes keys {16 st + 4c + 0..3, 16 st + 8 + 4c + 0..3}
    bf16x8 ph[2], pl[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const float a = p[8 * st + 2 * q2], a2 = p[8 * st + 2 * q2 + 1];
        wh[q2] = pack_bf16(a, a2);
        wl[q2] = pack_bf16(a - __uint_as_float(wh[q2] << 16), a2 - __uint_as_float(wh[q2] & 0xFFFF0000u));
      }
      uint4 uh{wh[0], wh[1], wh[2], wh[3]}, ul{wl[0], wl[1], wl[2], wl[3]};
      ph[st] = *reinterpret_cast<bf16x8*>(&uh);
      pl[st] = *reinterpret_cast<bf16x8*>(&ul);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 vf = lds_read_tr_x2(vl + vof[st][0][blk], vl + vof[st][1][blk]);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph[st], acc[blk], 0, 0, 0);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[st], acc[blk], 0, 0, 0);
      }
  };

  const int n_st = (L + KB - 1) / KB;
  // stages vw, vw + NW, ...
  const int cnt = n_st > vw ? (n_st - vw + NW - 1) / NW : 0;
  wait_lgkmcnt0();  // the zero fill is in LDS before any load can land on it
  if constexpr (NS == 2) {
    if (cnt > 0) issue(vw, 0);
    if (cnt > 1) issue(vw + NW, 1);
    for (int i = 0; i < cnt; ++i) {
      if (i + 1 < cnt) wait_vmcnt<2 * NLD>(); else wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      compute(kring + (i & 1) * OPB, vring + (i & 1) * OPB, vw + NW * i, [] {});
      if (i + 2 < cnt) {
        wait_lgkmcnt0();  // this slot's reads are done before it is refilled
        __builtin_amdgcn_sched_barrier(0);
        issue(vw + NW * (i + 2), i & 1);
      }
    }
  } else {
    // one slot: the other workgroup on the CU covers each wave's load wait.  The
    // next stage's K goes into the slot as soon as this stage's scores have read
    // it, so it is in flight during the softmax and PV; its V once PV is done.
    if (cnt > 0) issue(vw, 0);
    for (int i = 0; i < cnt; ++i) {
      const bool more = i + 1 < cnt;
      const int tn = vw + NW * (i + 1);
      wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      compute(kring, vring, vw + NW * i, [&]() __attribute__((always_inline)) {
        if (more) {
          wait_lgkmcnt0();  // K's reads are done before it is refilled
          __builtin_amdgcn_sched_barrier(0);
          issue_op(tn, 0, 0);
        }
      });
      wait_lgkmcnt0();  // V's reads are done before it is refilled
      __builtin_amdgcn_sched_barrier(0);
      if (more) issue_op(tn, 0, 1);
    }
  }
  __syncthreads();

  // merge the four key slices of each row and the row's path partial
  float* const so_lo = reinterpret_cast<float*>(sk_arr);  // [4][32][65]: hd 0..63
  float* const so_hi = reinterpret_cast<float*>(sv_arr);  // hd 64..127
  float* const sm = reinterpret_cast<float*>(sk_arr + EPI_HALF);  // [4][32] max
  float* const ss = reinterpret_cast<float*>(sv_arr + EPI_HALF);  // [4][32] sum
  lsum += __shfl_xor(lsum, 32, 64);
  {
    const int wr = (wave * 32 + kr) * OUT_LD2;
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int hd = blk * 32 + 8 * (e >> 2) + 4 * c + (e & 3);
        if (blk < NBLK / 2) so_lo[wr + hd] = acc[blk][e];
        else so_hi[wr + hd - HALF] = acc[blk][e];
      }
    if (lane < 32) {
      sm[wave * 32 + kr] = m;
      ss[wave * 32 + kr] = lsum;
    }
  }
  __syncthreads();
  {
    // thread t writes row t/8, hd [16 (t%8), +16): its path-partial loads are all
    // issued before any is used
    constexpr int SEG = HD / 8;
    const int row = tid >> 3, h0 = (tid & 7) * SEG;
    // this thread's 16 hd of the merge tile
    const float* const so = (h0 < HALF ? so_lo : so_hi) + (h0 < HALF ? h0 : h0 - HALF);
    const int j = j0 + row;
    if (j < rows_total) {
      const int r = j / G, h = g * G + j % G;
      if (S > 1) {  // this workgroup's share of the keys: (max, sum, unnormalised output)
        float M = -INFINITY;
#pragma unroll
        for (int k = 0; k < 4; ++k) M = fmaxf(M, sm[k * 32 + row]);
        float f[4], Ls = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          f[k] = M == -INFINITY ? 0.f : exp2f(sm[k * 32 + row] - M);
          Ls += f[k] * ss[k * 32 + row];
        }
        const size_t pi = (size_t)z * Bn * n_int * Hq + ((size_t)b * n_int + r) * Hq + h;
        if ((tid & 7) == 0) pml[pi] = float2{M, Ls};
        float4* pp = reinterpret_cast<float4*>(po + pi * HD + h0);
#pragma unroll
        for (int i = 0; i < SEG / 4; ++i) {
          float w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w[e] = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[e] += f[k] * so[(k * 32 + row) * OUT_LD2 + 4 * i + e];
          }
          pp[i] = float4{w[0], w[1], w[2], w[3]};
        }
        return;
      }
      const float4* ao = reinterpret_cast<const float4*>(anc_o + ((size_t)(rq + r) * Hq + h) * HD + h0);
      float4 av[SEG / 4];
#pragma unroll
      for (int i = 0; i < SEG / 4; ++i) av[i] = ao[i];
      const float2 a = anc_ml[(size_t)(rq + r) * Hq + h];
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k) M = fmaxf(M, sm[k * 32 + row]);
      float f[4], Ls = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[k] = M == -INFINITY ? 0.f : exp2f(sm[k * 32 + row] - M);
        Ls += f[k] * ss[k * 32 + row];
      }
      const float ma = a.x * LOG2E;
      const float Mt = fmaxf(M, ma);
      const float fd = M == -INFINITY ? 0.f : exp2f(M - Mt);
      const float fa = exp2f(ma - Mt);
      const float inv = 1.0f / (Ls * fd + a.y * fa);
      float v[SEG];
#pragma unroll
      for (int e = 0; e < SEG; ++e) {
        float Os = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) Os += f[k] * so[(k * 32 + row) * OUT_LD2 + e];
        const float an = (&av[e / 4].x)[e % 4];
        v[e] = (Os * fd + an * fa) * inv;
      }
      uint4* op = reinterpret_cast<uint4*>(O + (((size_t)b * n_int + r) * Hq + h) * HD + h0);
#pragma unroll
      for (int i = 0; i < SEG / 8; ++i)
        op[i] = uint4{pack_bf16(v[8 * i], v[8 * i + 1]), pack_bf16(v[8 * i + 2], v[8 * i + 3]),
                      pack_bf16(v[8 * i + 4], v[8 * i + 5]), pack_bf16(v[8 * i + 6], v[8 * i + 7])};
    }
  }
}

// Output of a key-split document attention: per (document row, query head) x, the
// S workgroup partials (base-2 max, sum, unnormalised output) of its document keys
// and the path partial of its trie row merge into one softmax; 4 output values per
// thread.  NRH = B n_int Hq, NH = n_int Hq (path partials are per trie row).
__global__ __launch_bounds__(256) void doc_attn_merge_kernel(int NRH, int NH, int HD, int S,
                                                             const float2* __restrict__ anc_ml,
                                                             const float* __restrict__ anc_o,
                                                             const float2* __restrict__ pml,
                                                             const float* __restrict__ po,
                                                             uint16_t* __restrict__ O) {
  const long t = long(blockIdx.x) * 256 + threadIdx.x;
  const int nq = HD / 4;
  if (t >= long(NRH) * nq) return;
  const int x = int(t / nq), q4 = int(t % nq) * 4;
  const float2 a = anc_ml[x % NH];
  const float ma = a.x * LOG2E;
  float Mt = ma;
  for (int z = 0; z < S; ++z) Mt = fmaxf(Mt, pml[(size_t)z * NRH + x].x);
  const float fa = exp2f(ma - Mt);
  float den = a.y * fa;
  const float4 an = *reinterpret_cast<const float4*>(anc_o + (size_t)(x % NH) * HD + q4);
  float4 num{an.x * fa, an.y * fa, an.z * fa, an.w * fa};
  for (int z = 0; z < S; ++z) {
    const float2 p = pml[(size_t)z * NRH + x];
    const float fz = p.x == -INFINITY ? 0.f : exp2f(p.x - Mt);
    den += fz * p.y;
    const float4 o = *reinterpret_cast<const float4*>(po + ((size_t)z * NRH + x) * HD + q4);
    num.x += fz * o.x;
    num.y += fz * o.y;
    num.z += fz * o.z;
    num.w += fz * o.w;
  }
  const float inv = 1.0f / den;
  *reinterpret_cast<uint2*>(O + (size_t)x * HD + q4) =
      uint2{pack_bf16(num.x * inv, num.y * inv), pack_bf16(num.z * inv, num.w * inv)};
}

// Key split of the document attention with few rows per (document, KV head): the
// (document, row block, KV head) workgroups alone would leave CUs idle (fewer
// than 256), so each is split S ways over its keys (S <= 4, up to ~512
// workgroups).  Not with a row selection.
static int doc_attn_splits(int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv, int32_t hd) {
  const long rows = long(n_int) * (Hq / Hkv);
  if (hd != 128 || rows > 64 || B <= 0) return 1;
  const long blocks = long(B) * Hkv * ((rows + 31) / 32);
  return blocks >= 256 ? 1 : int(std::min(4L, std::max(1L, 512 / blocks)));
}

size_t doc_attn_split_bytes(int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv, int32_t hd) {
  const int S = doc_attn_splits(B, n_int, Hq, Hkv, hd);
  if (S == 1) return 0;
  const size_t nrh = size_t(B) * n_int * Hq;
  return align_up(S * nrh * 8) + S * nrh * hd * 4;
}

// ---------------------------------------------------------------- launchers

int launch_anc_attn(void* stream, tcs_dtype dt, int32_t n_int, int32_t Hq, int32_t Hkv, int32_t hd,
                    const void* Qn, const void* Kn, const void* Vn, const int32_t* qparent,
                    float scale, float* anc_ml, float* anc_o) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const long waves = long(n_int) * Hq;
  if (waves == 0) return TCS_OK;
  const int grid = int((waves + 3) / 4);
  float2* ml = reinterpret_cast<float2*>(anc_ml);
#define TCS_ANC(T, HDV)                                                                            \
  anc_attn_kernel<T, HDV><<<grid, 256, 0, s>>>(n_int, Hq, Hkv, static_cast<const T*>(Qn),        \
                                               static_cast<const T*>(Kn), static_cast<const T*>(Vn), \
                                               qparent, scale, ml, anc_o)
  if (dt == TCS_BF16) {
    if (hd == 128) TCS_ANC(bf16_t, 128); else TCS_ANC(bf16_t, 64);
  } else {
    if (hd == 128) TCS_ANC(float, 128); else TCS_ANC(float, 64);
  }
#undef TCS_ANC
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "anc_attn: %s", hipGetErrorString(e));
  return TCS_OK;
}

// Document part for tries with many query rows per (document, KV head): each wave
// owns 32 query rows (j -> node j / G, head g G + j % G) and all four waves share
// one 64-key stage of K (row-major) and V^T in LDS, loaded through registers one
// stage ahead.  The stage is processed in two 32-key blocks with the same MFMA
// formulation as doc_attn_mfma_kernel (S^T = K Q^T with a lane per row; O^T +=
// V^T P^T with P split into bf16 high and low parts).  Two workgroups fit on a CU
// (at most 256 registers per lane, ~70 KB of LDS), so one's loads and barriers
// overlap the other's MFMAs.  The epilogue merges each row with its path partial
// and writes whole rows through a per-wave LDS tile.
template <int HD>
__global__ __launch_bounds__(256, 2) void doc_attn_rows_kernel(
    int B, int dpw, int n_int, int Hq, int Hkv, const uint16_t* __restrict__ Qn,
    const uint16_t* __restrict__ Kd, const uint16_t* __restrict__ Vd,
    const int32_t* __restrict__ doc_offsets, const float2* __restrict__ anc_ml,
    const float* __restrict__ anc_o, float scale, uint16_t* __restrict__ O) {
  constexpr int KT = 64;                       // keys per stage
  constexpr int LDK = HD + 8;                  // sK row (bf16): conflict-free 16-byte reads
  constexpr int LDV = KT + 4;                  // sVt row (bf16): conflict-free 8-byte reads
  constexpr int STAGE = KT * LDK + HD * LDV;   // bf16 elements
  constexpr int K_CH = KT * (HD / 8) / 256;    // 16-byte K chunks per thread
  constexpr int V_GROUPS = (KT / 4) * (HD / 8);  // 4 keys x 8 hd per group
  constexpr int NBLK = HD / 32, KSTEPS = HD / 16;
  constexpr int OUT_LD = HD + 1;               // epilogue fp32 row
  constexpr int EPI_BYTES = 4 * 32 * OUT_LD * 4 + 4 * 32 * 2 * 4;
  constexpr int LDS_BYTES = 2 * STAGE * 2 > EPI_BYTES ? 2 * STAGE * 2 : EPI_BYTES;
  static_assert(K_CH * 256 == KT * (HD / 8) && V_GROUPS <= 256, "staging");
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[LDS_BYTES];
  uint16_t* lds = reinterpret_cast<uint16_t*>(lds_raw);

  const int G = Hq / Hkv;
  const int rows_total = n_int * G;
  const int n_rb = (rows_total + 127) / 128;
  const int rb = blockIdx.x % n_rb;
  const int g = (blockIdx.x / n_rb) % Hkv;
  const int b_lo = blockIdx.x / (n_rb * Hkv) * dpw;
  const int b_hi = min(B, b_lo + dpw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j0 = rb * 128 + wave * 32;  // this wave's first row

  // Q^T fragments (lane: row l%32, hd 16 ks + 8 (l/32) ..)
  bf16x8 qf[KSTEPS];
  {
    const int j = j0 + (lane & 31);
    const bool ok = j < rows_total;
    const int r = ok ? j / G : 0, h = g * G + (ok ? j % G : 0);
    const uint16_t* qp = Qn + ((size_t)r * Hq + h) * HD + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : uint4{0, 0, 0, 0};
      qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  uint4 rk[K_CH];
  uint4 rv[4];
  int doc0 = 0, L = 0;
  auto load_stage = [&](int key0) {
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int kk = c / (HD / 8), hc = c % (HD / 8);
      const int key = key0 + kk;
      rk[i] = key < L ? *reinterpret_cast<const uint4*>(Kd + ((size_t)(doc0 + key) * Hkv + g) * HD + hc * 8)
                      : uint4{0, 0, 0, 0};
    }
    const int kg = tid / (HD / 8), hc = tid % (HD / 8);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = key0 + kg * 4 + t;
      rv[t] = (tid < V_GROUPS && key < L)
                  ? *reinterpret_cast<const uint4*>(Vd + ((size_t)(doc0 + key) * Hkv + g) * HD + hc * 8)
                  : uint4{0, 0, 0, 0};
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* sK = lds + buf * STAGE;
    uint16_t* sV = sK + KT * LDK;
#pragma unroll
    for (int i = 0; i < K_CH; ++i) {
      const int c = tid + i * 256;
      const int kk = c / (HD / 8), hc = c % (HD / 8);
      *reinterpret_cast<uint4*>(sK + kk * LDK + hc * 8) = rk[i];
    }
    if (tid < V_GROUPS) {
      const int kg = tid / (HD / 8), hc = tid % (HD / 8);
      const uint32_t w[4][4] = {{rv[0].x, rv[0].y, rv[0].z, rv[0].w},
                                {rv[1].x, rv[1].y, rv[1].z, rv[1].w},
                                {rv[2].x, rv[2].y, rv[2].z, rv[2].w},
                                {rv[3].x, rv[3].y, rv[3].z, rv[3].w}};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t k0 = (w[0][e >> 1] >> sh) & 0xFFFFu, k1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t k2 = (w[2][e >> 1] >> sh) & 0xFFFFu, k3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2*>(sV + (hc * 8 + e) * LDV + kg * 4) = uint2{k0 | (k1 << 16), k2 | (k3 << 16)};
      }
    }
  };

  const float qk = scale * LOG2E;
  // the documents of this workgroup one after another: the query fragments stay in
  // registers and the rows' path partials stay in cache across them
  for (int b = b_lo; b < b_hi; ++b) {
  doc0 = doc_offsets[b];
  L = doc_offsets[b + 1] - doc0;
  f32x16 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  float m = -INFINITY, lsum = 0.f;  // base-2 running max; this lane's share of the sum

  const int n_it = (L + KT - 1) / KT;
  if (n_it > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int cur = it & 1;
    if (it + 1 < n_it) load_stage((it + 1) * KT);
    const uint16_t* sK = lds + cur * STAGE;
    const uint16_t* sV = sK + KT * LDK;
    // S^T for the stage's two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
      const uint16_t* kp = sK + (kb * 32 + (lane & 31)) * LDK + 8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kp + ks * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
      }
    }
    // online softmax (base 2) over the 64 keys; keys past the document end are masked
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = it * KT + kb * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        s[kb][e] = key < L ? s[kb][e] * qk : -INFINITY;
        tmax = fmaxf(tmax, s[kb][e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float c = mn == -INFINITY ? 1.f : exp2f(m - mn);
    lsum *= c;
    m = mn;
#pragma unroll
    for (int i = 0; i < NBLK; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] *= c;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = mn == -INFINITY ? 0.f : exp2f(s[kb][e] - mn);
        lsum += p[e];
      }
      // P^T fragments: keys {8j + 4(l/32) + i}; step 0 takes j = 0,1, step 1 j = 2,3.
      bf16x8 ph[2], pl[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const float a = p[8 * st + 2 * q2], c2 = p[8 * st + 2 * q2 + 1];
          wh[q2] = pack_bf16(a, c2);
          wl[q2] = pack_bf16(a - __uint_as_float(wh[q2] << 16), c2 - __uint_as_float(wh[q2] & 0xFFFF0000u));
        }
        uint4 uh{wh[0], wh[1], wh[2], wh[3]}, ul{wl[0], wl[1], wl[2], wl[3]};
        ph[st] = *reinterpret_cast<bf16x8*>(&uh);
        pl[st] = *reinterpret_cast<bf16x8*>(&ul);
      }
      // O^T += V^T P^T
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk) {
        const uint16_t* vp = sV + (blk * 32 + (lane & 31)) * LDV + kb * 32 + 4 * (lane >> 5);
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const uint2 lo = *reinterpret_cast<const uint2*>(vp + 16 * st);
          const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16 * st + 8);
          uint4 u{lo.x, lo.y, hi.x, hi.y};
          const bf16x8 vf = *reinterpret_cast<bf16x8*>(&u);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, ph[st], acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[st], acc[blk], 0, 0, 0);
        }
      }
    }
    if (it + 1 < n_it) store_stage(cur ^ 1);
    __syncthreads();
  }

  // epilogue: this wave's 32 rows through its own LDS tile (the stages are free)
  lsum += __shfl_xor(lsum, 32, 64);
  float* so = reinterpret_cast<float*>(lds_raw) + (size_t)wave * 32 * OUT_LD;
  float* sf = reinterpret_cast<float*>(lds_raw) + 4 * 32 * OUT_LD + wave * 64;  // [32][2]
  const int rw = lane & 31;
  {
    const int j = j0 + rw;
    float s_doc = 0.f, s_anc = 0.f;
    if (j < rows_total) {
      const int r = j / G, h = g * G + j % G;
      const float2 a = anc_ml[(size_t)r * Hq + h];
      const float ma = a.x * LOG2E;
      const float Mt = fmaxf(m, ma);
      const float fd = m == -INFINITY ? 0.f : exp2f(m - Mt);
      const float fa = exp2f(ma - Mt);
      const float inv = 1.0f / (lsum * fd + a.y * fa);
      s_doc = fd * inv;
      s_anc = fa * inv;
    }
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int hd = blk * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        so[rw * OUT_LD + hd] = acc[blk][e];
      }
    if (lane < 32) {
      sf[rw * 2 + 0] = s_doc;
      sf[rw * 2 + 1] = s_anc;
    }
  }
  __syncthreads();
  {
    // lane pair (2 rr, 2 rr + 1) writes row rr, one half of hd each: all of the
    // half-row's path-partial loads are issued before any is used
    constexpr int HH = HD / 2;
    const int rr = lane >> 1, half = lane & 1;
    const int j = j0 + rr;
    if (j < rows_total) {
      const int r = j / G, h = g * G + j % G;
      const float4* ao = reinterpret_cast<const float4*>(anc_o + ((size_t)r * Hq + h) * HD + half * HH);
      float4 av[HH / 4];
#pragma unroll
      for (int i = 0; i < HH / 4; ++i) av[i] = ao[i];
      const float sd = sf[rr * 2], sa = sf[rr * 2 + 1];
      const float* sr = so + rr * OUT_LD + half * HH;
      uint4* op = reinterpret_cast<uint4*>(O + (((size_t)b * n_int + r) * Hq + h) * HD + half * HH);
#pragma unroll
      for (int i = 0; i < HH / 8; ++i) {
        const float4 a0 = av[2 * i], a1 = av[2 * i + 1];
        const float* x = sr + 8 * i;
        op[i] = uint4{pack_bf16(x[0] * sd + a0.x * sa, x[1] * sd + a0.y * sa),
                      pack_bf16(x[2] * sd + a0.z * sa, x[3] * sd + a0.w * sa),
                      pack_bf16(x[4] * sd + a1.x * sa, x[5] * sd + a1.y * sa),
                      pack_bf16(x[6] * sd + a1.z * sa, x[7] * sd + a1.w * sa)};
      }
    }
  }
  __syncthreads();  // the epilogue's LDS tile is the next document's stage buffer
  }
}

// Document part for tries with many query rows per (document, KV head), hd 128:
// 128 query rows (32 per wave) of one KV head against the documents
// [b_lo, b_hi) one after another.  64-key stages of K and V go through a two-slot
// LDS ring filled by buffer-to-LDS loads (natural [key][hd] layout, chunk-swizzled
// like the key-streaming kernel), shared by the four waves; the ring runs on
// across documents.  Per stage each wave computes S^T = K Q^T for two 32-key
// blocks, one online-softmax update, and O^T += V^T P^T with V^T from transposing
// LDS reads and P split into bf16 high and low parts.  Each row's softmax state
// starts from its path partial at the document's first stage; at the document's
// end each lane normalises its half of the row and writes it straight from the
// accumulators, so the ring keeps loading meanwhile.  Two workgroups fit on a CU
// (64 KB of LDS each), and each wave raises its priority over its matrix ops, so
// the SIMD's other wave (of the other workgroup) runs its softmax under them.
constexpr int ROWS_DMA_MAX_DPW = 64;  // documents per workgroup of the kernel below, at most
__global__ __launch_bounds__(256, 2) void doc_attn_rows_dma_kernel(
    int B, int dpw, int n_int, int Hq, int Hkv, const uint16_t* __restrict__ Qn,
    const uint16_t* __restrict__ Kd, const uint16_t* __restrict__ Vd,
    const int32_t* __restrict__ doc_offsets, const float2* __restrict__ anc_ml,
    const float* __restrict__ anc_o, float scale, uint16_t* __restrict__ O) {
  constexpr int HD = 128;
  constexpr int KT = 64;                 // keys per stage
  constexpr int ROW = HD * 2;            // bytes per key row
  constexpr int OPB = KT * ROW;          // bytes per operand per stage (16 KB)
  constexpr int SLOT = 2 * OPB;          // K then V
  constexpr int NBLK = HD / 32, KSTEPS = HD / 16;
  // the two ring slots are distinct arrays, and every stage below is compiled for
  // one slot parity, so the compiler can tell that a stage's fragment reads and the
  // next stage's buffer-to-LDS loads touch different memory (with one array and a
  // computed slot offset it must wait for those loads before the first read)
  __shared__ __attribute__((aligned(16))) uint8_t slot0[SLOT];
  __shared__ __attribute__((aligned(16))) uint8_t slot1[SLOT];
  // offsets of the workgroup's documents: the prefetch cursor reads them from LDS,
  // so stepping into the next document waits on no vector-memory load (a global
  // read there would also wait for the stage loads just issued)
  __shared__ int s_doc[ROWS_DMA_MAX_DPW + 1];

  const int G = Hq / Hkv;
  const int rows_total = n_int * G;
  const int n_rb = (rows_total + 127) / 128;
  const int rb = blockIdx.x % n_rb;
  const int g = (blockIdx.x / n_rb) % Hkv;
  const int b_lo = blockIdx.x / (n_rb * Hkv) * dpw;
  const int b_hi = min(B, b_lo + dpw);
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid <= b_hi - b_lo) s_doc[tid] = doc_offsets[b_lo + tid];
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j0 = rb * 128 + wave * 32;   // this wave's first row
  const int RS = Hkv * HD * 2;           // bytes between consecutive keys of one head

  // slots start as zeros, so a key past a document's end that no load writes
  // still holds finite values (its weight is 0)
#pragma unroll
  for (int i = 0; i < SLOT / (256 * 16); ++i) {
    *reinterpret_cast<uint4*>(slot0 + (i * 256 + tid) * 16) = uint4{0u, 0u, 0u, 0u};
    *reinterpret_cast<uint4*>(slot1 + (i * 256 + tid) * 16) = uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();  // every wave's zeros are in place before any load can land

  // Q^T fragments: lane holds row l%32, hd 16 ks + 8 (l/32) ..
  const int kr = lane & 31, c = lane >> 5;
  const int jrow = j0 + kr;
  const bool row_ok = jrow < rows_total;
  const int r = row_ok ? jrow / G : 0, h = g * G + (row_ok ? jrow % G : 0);
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = Qn + ((size_t)r * Hq + h) * HD + 8 * c;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint4 v = row_ok ? *reinterpret_cast<const uint4*>(qp + ks * 16) : uint4{0, 0, 0, 0};
      qf[ks] = *reinterpret_cast<bf16x8*>(&v);
    }
  }

  // DMA: load j (0..15) of an operand fills stage rows 4j .. 4j+3; this wave issues
  // loads 4 wave .. 4 wave + 3 of K and of V.  Lane i writes row 4j + i/16 at
  // position i%16, which holds chunk (i%16) ^ kv_swz(row).
  int vo[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int row = 4 * (4 * wave + jj) + (lane >> 4);
    vo[jj] = row * RS + (((lane & 15) ^ kv_swz(row & 15)) << 4);
  }
  auto doc_at = [&](int b) { return __builtin_amdgcn_readfirstlane(s_doc[b - b_lo]); };
  auto n_stages = [&](int b) { return (doc_at(b + 1) - doc_at(b) + KT - 1) / KT; };
  // stage t of document b into ring slot `slot`; past the last document (b = b_hi)
  // the loads go through a zero-range buffer resource and touch no memory, so every
  // stage issues the same loads and no branch decides whether a slot is being filled
  auto issue = [&](int b, int t, uint8_t* slot) __attribute__((always_inline)) {
    const bool ok = b < b_hi;
    const int bb = ok ? b : b_lo;
    const int doc0 = doc_at(bb), L = doc_at(bb + 1) - doc0;
    const int nkeys = min(KT, L - t * KT);
    const int bytes = ok ? (nkeys - 1) * RS + ROW : 0;
    const size_t off = ((size_t)(doc0 + t * KT) * Hkv + g) * HD;
    uint8_t* dst = slot + wave * 4 * 1024;
    kv_issue<4>(Kd + off, bytes, dst, vo);
    kv_issue<4>(Vd + off, bytes, dst + OPB, vo);
  };

  // fragment offsets inside a slot (key block kb adds kb * 32 rows)
  int ko[KSTEPS];  // K: row kr, chunk 2 ks + c
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) ko[ks] = kr * ROW + (((2 * ks + c) ^ kv_swz(kr & 15)) << 4);
  int vof[2][2][NBLK];  // V^T, as in the key-streaming kernel
  {
    const int sidx = lane & 15, hsel = (lane >> 4) & 1;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int key = 16 * st + 8 * q + 4 * c + (sidx >> 2);
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) {
          const int chunk = 4 * blk + 2 * hsel + ((sidx & 3) >> 1);
          vof[st][q][blk] = OPB + key * ROW + ((chunk ^ kv_swz(key & 15)) << 4) + 8 * (sidx & 1);
        }
      }
  }
  const float qk = scale * LOG2E;

  // prefetch cursor: the next stage to load (documents without keys are skipped)
  int pb = b_lo, pt = 0;
  while (pb < b_hi && n_stages(pb) == 0) ++pb;
  int kc = 0;  // stages computed so far (slot kc & 1)
  if (pb < b_hi) issue(pb, 0, slot0);
  auto advance = [&]() __attribute__((always_inline)) {
    if (++pt >= n_stages(pb)) {
      pt = 0;
      do ++pb; while (pb < b_hi && n_stages(pb) == 0);
    }
  };
  advance();

  // P^T fragments of one 32-key block, built one pair of keys at a time: pair q
  // (keys 2q, 2q+1 of the lane's 16) gives word q % 4 of fragment q / 4, as the
  // weights exp2(s - m) split into a bf16 high part and the bf16 remainder; the
  // pair's weights are added to ls.
  auto weight_pair = [&](const f32x16& scb, float mrow, float& ls, int q, uint32_t (&wh)[2][4],
                         uint32_t (&wl)[2][4]) __attribute__((always_inline)) {
    const float a = __builtin_amdgcn_exp2f(fmaf(scb[2 * q], qk, -mrow));
    const float a2 = __builtin_amdgcn_exp2f(fmaf(scb[2 * q + 1], qk, -mrow));
    ls += a;
    ls += a2;
    const uint32_t h2 = pack_bf16(a, a2);
    wh[q >> 2][q & 3] = h2;
    wl[q >> 2][q & 3] = pack_bf16(a - __uint_as_float(h2 << 16), a2 - __uint_as_float(h2 & 0xFFFF0000u));
  };
  auto frags = [&](const uint32_t (&w)[2][4], int st) __attribute__((always_inline)) {
    uint4 u{w[st][0], w[st][1], w[st][2], w[st][3]};
    return *reinterpret_cast<bf16x8*>(&u);
  };

  for (int b = b_lo; b < b_hi; ++b) {
    const int L = doc_at(b + 1) - doc_at(b);
    const int nst = (L + KT - 1) / KT;
    // The row's softmax state starts from its path partial (the keys of its own
    // ancestors and itself): acc = their unnormalised value sum, m = their maximum
    // score (base 2), and lsum = their weight sum, held by one lane of the row's two.
    // The document's keys then extend the same online softmax, and the end of the
    // document only normalises.  The partial is loaded at the document's first stage,
    // before that stage's buffer-to-LDS loads are issued, so its first use waits for
    // these loads alone while the stage's QK products run.
    f32x16 acc[NBLK];
    float m = 0.f, lsum = 0.f;  // base-2 running max; this lane's share of the sum
    auto seed = [&]() __attribute__((always_inline)) {
      const float* ao = anc_o + ((size_t)r * Hq + h) * HD + 4 * c;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float4 v = *reinterpret_cast<const float4*>(ao + blk * 32 + 8 * e4);
          acc[blk][4 * e4 + 0] = v.x;
          acc[blk][4 * e4 + 1] = v.y;
          acc[blk][4 * e4 + 2] = v.z;
          acc[blk][4 * e4 + 3] = v.w;
        }
      const float2 a = anc_ml[(size_t)r * Hq + h];
      m = a.x * LOG2E;
      lsum = c == 0 ? a.y : 0.f;
    };
    // (an empty document's row is its path partial alone)
    if (nst == 0) seed();
    // one stage; Par = kc & 1 picks the slot it reads and the slot it refills, and
    // First (the document's first stage) loads the path partial; both are compile-time
    // so the loads and the slots need no branch
    auto stage = [&](auto Par, auto First, int t) __attribute__((always_inline)) {
      constexpr int P = decltype(Par)::value;
      uint8_t* const cur = P ? slot1 : slot0;
      uint8_t* const nxt = P ? slot0 : slot1;
      wait_vmcnt<0>();       // this wave's part of stage kc has landed
      wait_lgkmcnt0();       // and its reads of stage kc - 1 are done
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(First)::value) seed();
      __builtin_amdgcn_sched_barrier(0);
      issue(pb, pt, nxt);    // stage kc + 1 into the slot stage kc - 1 used
      if (pb < b_hi) advance();
      const uint8_t* sl = cur;
      f32x16 sc[2];
      // the matrix ops of this stage's scores run at raised wave priority, so the
      // SIMD's other wave (another workgroup, in its vector phase) yields to them
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[kb][e] = 0.f;
      // the two key blocks' products alternate, so consecutive matrix ops do not
      // depend on each other; K fragments are read four matrix ops ahead, so their
      // LDS latency is not waited out one fragment at a time
      {
        constexpr int NF = 2 * KSTEPS, AHEAD = 4;
        auto kfrag = [&](int i) __attribute__((always_inline)) {
          return *reinterpret_cast<const bf16x8*>(sl + (i & 1) * 32 * ROW + ko[i >> 1]);
        };
        bf16x8 kq[AHEAD];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) kq[i] = kfrag(i);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
          sc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[i % AHEAD], qf[i >> 1], sc[i & 1], 0, 0, 0);
          if (i + AHEAD < NF) kq[i % AHEAD] = kfrag(i + AHEAD);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS read
#pragma unroll
        for (int i = 0; i < NF - AHEAD; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);  // MFMA
      }
      __builtin_amdgcn_s_setprio(0);
      // online softmax (base 2) over the 64 keys; only a document's last stage has
      // keys past its end, which are masked (the empty asm keeps this a branch
      // rather than selects on every stage)
      if (L - t * KT < KT) {
        asm volatile("");
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = t * KT + kb * 32 + 8 * (e >> 2) + 4 * c + (e & 3);
            sc[kb][e] = key < L ? sc[kb][e] : -INFINITY;
          }
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sc[kb][e]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * qk;
      lazy_rescale(m, tmax, lsum, acc);
      // weights of block 0; then block 0's PV products, each pair of matrix ops
      // followed by one pair of block 1's weights (the matrix cores and the vector
      // ALU work at once); then block 1's products
      uint32_t w0h[2][4], w0l[2][4], w1h[2][4], w1l[2][4];
#pragma unroll
      for (int q = 0; q < 8; ++q) weight_pair(sc[0], m, lsum, q, w0h, w0l);
      __builtin_amdgcn_s_setprio(1);  // the PV matrix ops, as the scores'
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 vf = lds_read_tr_x2(sl + vof[st][0][blk], sl + vof[st][1][blk]);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, frags(w0h, st), acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, frags(w0l, st), acc[blk], 0, 0, 0);
          weight_pair(sc[1], m, lsum, 2 * blk + st, w1h, w1l);
        }
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 vf = lds_read_tr_x2(sl + 32 * ROW + vof[st][0][blk], sl + 32 * ROW + vof[st][1][blk]);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, frags(w1h, st), acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, frags(w1l, st), acc[blk], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      // the schedule of that block (after lazy_rescale's branch): block 0's weights
      // (12 vector instructions per pair of keys), then per V^T fragment two DS reads,
      // a matrix op, six vector instructions, a matrix op, six more
      __builtin_amdgcn_sched_group_barrier(0x002, 96, 0);  // VALU: block 0's weights
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read (V^T)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      }
    };
    using Odd = std::integral_constant<int, 1>;
    using Even = std::integral_constant<int, 0>;
    if (nst > 0) {
      if (kc & 1) stage(Odd{}, std::true_type{}, 0);
      else stage(Even{}, std::true_type{}, 0);
      ++kc;
    }
    // the rest in (even slot, odd slot) pairs, so that the loop body is straight-line
    // code and the accumulators stay in the same registers from stage to stage (a
    // branch on the parity at every stage made the compiler copy them out and back)
    using F = std::false_type;
    int t = 1;
    if (t < nst && (kc & 1)) {
      stage(Odd{}, F{}, t);
      ++t;
      ++kc;
    }
    for (; t + 1 < nst; t += 2, kc += 2) {
      stage(Even{}, F{}, t);
      stage(Odd{}, F{}, t + 1);
    }
    if (t < nst) {
      stage(Even{}, F{}, t);
      ++kc;
    }
    // normalise; lane writes hd blk*32 + 8 e4 + 4 c + 0..3
    lsum += __shfl_xor(lsum, 32, 64);
    if (row_ok) {
      const float inv = 1.0f / lsum;
      uint16_t* op = O + (((size_t)b * n_int + r) * Hq + h) * HD + 4 * c;
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
          *reinterpret_cast<uint2*>(op + blk * 32 + 8 * e4) =
              uint2{pack_bf16(acc[blk][4 * e4] * inv, acc[blk][4 * e4 + 1] * inv),
                    pack_bf16(acc[blk][4 * e4 + 2] * inv, acc[blk][4 * e4 + 3] * inv)};
    }
  }
  wait_vmcnt<0>();  // nothing may still target LDS at exit
}

int launch_doc_attn(void* stream, tcs_dtype dt, int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv,
                    int32_t hd, const void* Qn, const void* Kd, const void* Vd,
                    const int32_t* doc_offsets, const float* anc_ml, const float* anc_o,
                    float scale, void* O, const int32_t* sel, const int32_t* n_sel, void* split) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (B == 0 || n_int == 0) return TCS_OK;
  if (dt != TCS_BF16) return fail(TCS_EUNSUPPORTED, "doc_attn: MFMA path is bf16 only");
  if (sel && (n_int != 1 || hd != 128 || Hq / Hkv > 64))
    return fail(TCS_EUNSUPPORTED, "doc_attn: row selection needs one row, head_dim 128, <= 64 rows");
  const int G = Hq / Hkv;
  const long rows = long(n_int) * G;
  const float2* ml = reinterpret_cast<const float2*>(anc_ml);
  auto q = static_cast<const uint16_t*>(Qn);
  auto kd = static_cast<const uint16_t*>(Kd);
  auto vd = static_cast<const uint16_t*>(Vd);
  auto o = static_cast<uint16_t*>(O);
  timer_begin(TCS_TIMER_DOC_ATTN, stream);
  if (rows <= 64) {
    const long grid = long(B) * Hkv * ((rows + 31) / 32);
    const int S = split && !sel ? doc_attn_splits(B, n_int, Hq, Hkv, hd) : 1;
    if (hd == 128 && S > 1) {
      const size_t nrh = size_t(B) * n_int * Hq;
      auto pml = static_cast<float2*>(split);
      auto po = reinterpret_cast<float*>(static_cast<char*>(split) + align_up(S * nrh * 8));
      doc_attn_stream_kernel<128, 1><<<grid * S, 256, 0, s>>>(n_int, Hq, Hkv, q, kd, vd, doc_offsets, ml, anc_o, scale, o,
                                                              nullptr, nullptr, S, pml, po);
      const long threads = long(nrh) * (hd / 4);
      doc_attn_merge_kernel<<<int((threads + 255) / 256), 256, 0, s>>>(int(nrh), n_int * Hq, hd, S, ml, anc_o, pml, po, o);
    } else if (hd == 128)
      doc_attn_stream_kernel<128, 1><<<grid, 256, 0, s>>>(n_int, Hq, Hkv, q, kd, vd, doc_offsets, ml, anc_o, scale, o, sel, n_sel,
                                                          1, nullptr, nullptr);
    else
      doc_attn_mfma_kernel<64, 1, 4><<<grid, 256, 0, s>>>(n_int, Hq, Hkv, q, kd, vd, doc_offsets, ml, anc_o, scale, o);
  } else {
    // documents per workgroup: as many as keep >= 4096 workgroups (8 rounds of two
    // per CU, so the last round's tail stays small); the queries and path partials
    // are then read once per dpw documents
    const long blocks = long(Hkv) * ((rows + 127) / 128);
    const long chunks = std::min(long(B), (4096 + blocks - 1) / blocks);
    const int dpw = int(std::min(long(ROWS_DMA_MAX_DPW), std::max(1L, B / chunks)));
    const long grid = blocks * ((B + dpw - 1) / dpw);
    if (hd == 128)
      doc_attn_rows_dma_kernel<<<grid, 256, 0, s>>>(B, dpw, n_int, Hq, Hkv, q, kd, vd, doc_offsets, ml, anc_o, scale, o);
    else
      doc_attn_rows_kernel<64><<<grid, 256, 0, s>>>(B, dpw, n_int, Hq, Hkv, q, kd, vd, doc_offsets, ml, anc_o, scale, o);
  }
  timer_end(TCS_TIMER_DOC_ATTN, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "doc_attn: %s", hipGetErrorString(e));
  return TCS_OK;
}

int launch_attn_simt(void* stream, tcs_dtype dt, int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv,
                     int32_t hd, const void* Qn, const void* Kn, const void* Vn, const void* Kd,
                     const void* Vd, const int32_t* doc_offsets, const int32_t* qparent, float scale,
                     void* O, const int32_t* sel, const int32_t* n_sel) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sel && n_int != 1) return fail(TCS_EUNSUPPORTED, "attn_simt: row selection needs n_int = 1");
  const long waves = long(B) * n_int * Hq;
  if (waves == 0) return TCS_OK;
  const int grid = int((waves + 3) / 4);
#define TCS_SIMT(T, HDV)                                                                           \
  attn_simt_kernel<T, HDV><<<grid, 256, 0, s>>>(                                                   \
      B, n_int, Hq, Hkv, static_cast<const T*>(Qn), static_cast<const T*>(Kn),                     \
      static_cast<const T*>(Vn), static_cast<const T*>(Kd), static_cast<const T*>(Vd), doc_offsets, \
      qparent, scale, static_cast<T*>(O), sel, n_sel)
  if (dt == TCS_BF16) {
    if (hd == 128) TCS_SIMT(bf16_t, 128); else TCS_SIMT(bf16_t, 64);
  } else {
    if (hd == 128) TCS_SIMT(float, 128); else TCS_SIMT(float, 64);
  }
#undef TCS_SIMT
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TCS_EHIP, "attn_simt: %s", hipGetErrorString(e));
  return TCS_OK;
}

}  // namespace tcs
