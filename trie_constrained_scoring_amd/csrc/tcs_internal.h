// Internal declarations shared by the libtcs translation units.
#pragma once

#include <cstddef>
#include <cstdint>

#include "tcs.h"

namespace tcs {

// Thread-local error message; returns `code` so callers can `return fail(...)`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Sub-allocator over a caller workspace: hands out 256-byte aligned slices.
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t count) {
    size_t off = used;
    used = align_up(used + count * sizeof(T));
    return base ? reinterpret_cast<T*>(base + off) : nullptr;
  }
};

inline size_t dtype_bytes(tcs_dtype t) { return t == TCS_F32 ? 4 : t == TCS_BF16 ? 2 : 1; }

// Kernel timing (tcs_timing_enable): both calls are no-ops while timing is off.
void timer_begin(int timer, void* stream);
void timer_end(int timer, void* stream);

// ---- kernel launchers (each returns TCS_OK or TCS_EHIP) ------------------

// a[r] = RMSNorm(E[tok(r)]), tok(r) = idx2 ? idx2[idx[r]] : idx[r]; a row whose
// token is outside [0, V) is written as NaN.
int launch_embed_rmsnorm(void* stream, tcs_dtype dt, const void* E, const int32_t* idx,
                         const int32_t* idx2, int32_t n, int32_t d, int32_t V, float eps, void* out);

// h[r] = RMSNorm(y[r]) for fp32 y = sum of n_part partials [n_part][n][d], written in
// dtype dt.
// live (optional, device): when it holds 0 the launch does nothing.
int launch_rownorm(void* stream, tcs_dtype dt, const float* y, int32_t n, int32_t d, int32_t n_part,
                   float eps, void* out, const int32_t* live = nullptr);

// C[m, n] = sum_k A[m, k] * B[n, k].  Epilogues:
//   STORE: C stored in dtype dt (rounded) with leading dimension ldc.
//   RESID: C + E[tok(row)] stored as fp32, tok(row) = token[qnode[row % n_int]]; may
//          be split over K into gemm_resid_splits(...) fp32 partials [splits][M][ldc]
//          (the residual in the first), to be summed by launch_rownorm.  lda and ldb
//          must then be multiples of 8.
enum GemmEpi { GEMM_STORE = 0, GEMM_RESID = 1 };
int gemm_resid_splits(tcs_dtype dt, int32_t M, int32_t N, int32_t K);
struct GemmResid {
  const void* E;
  const int32_t* token;
  const int32_t* qnode;
  int32_t n_int;
  const int32_t* live;  // optional (device): when it holds 0 the launch does nothing
};
int launch_gemm_nt(void* stream, tcs_dtype dt, GemmEpi epi, int32_t M, int32_t N, int32_t K,
                   const void* A, int32_t lda, const void* B, int32_t ldb, void* C, int32_t ldc,
                   const GemmResid* resid);

// Output projection of many rows on the output head's LDS-DMA ring:
// C[r][n] = sum_k A[r][k] B[n][k] + E[tok(r)][n] (bf16 operands, fp32 C), for shapes
// with gemm_ring_ok; `zero` holds gemm_ring_zero_bytes(K) zero bytes (none needed
// when K / 64 is a multiple of 5).
bool gemm_ring_ok(int32_t M, int32_t N, int32_t K);
size_t gemm_ring_zero_bytes(int32_t K);
int launch_gemm_ring_resid(void* stream, int32_t M, int32_t N, int32_t K, const void* A,
                           const void* B, float* C, int32_t ldc, const GemmResid& res,
                           const void* zero);
// Zero `bytes` (a multiple of 16) of device memory with a fill kernel.
int launch_zero_fill(void* stream, void* p, size_t bytes);

// Output head, see tcs_lmhead_lse_gather.  Its workspace is a per-label-set part
// (lmhead_prep_bytes: edge segments, zero block, gather lists for batches of B
// documents; written by launch_lmhead_prep) followed by the per-batch (max, sum exp)
// partials (lmhead_part_bytes), then for a W8A8 head the hidden rows' codes and
// scales (lmhead_act8_bytes).  launch_lmhead does all of it on one workspace.
int lmhead_n_tiles(tcs_dtype h_dtype, int32_t V);
size_t lmhead_prep_bytes(tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t n_nodes, int32_t d,
                         int32_t V);
size_t lmhead_part_bytes(tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t V);
size_t lmhead_ws_bytes(tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                       int32_t n_nodes, int32_t d, int32_t V);
int launch_lmhead_prep(void* stream, tcs_dtype h_dtype, int32_t B, int32_t n_int, int32_t n_nodes,
                       int32_t d, int32_t V, const int32_t* e_tok, const int32_t* e_qrow,
                       const int32_t* e_child, int32_t n_edges, void* prep);
// finalize_lp = false leaves the raw child logits in lp (for a fused path sum).
int launch_lmhead_run(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                      int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                      const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                      const int32_t* e_child, float* lse, float* lp, const void* prep, void* part,
                      bool finalize_lp = true, void* act8 = nullptr);
// Scratch of a W8A8 head (w_dtype TCS_FP8_E4M3_A8): the hidden rows' E4M3 codes and
// scales; 0 for other heads.
size_t lmhead_act8_bytes(tcs_dtype w_dtype, int32_t R, int32_t d);
int launch_lmhead(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                  int32_t n_nodes, int32_t d, int32_t V, const void* h, const void* W,
                  const float* w_scale, const int32_t* e_tok, const int32_t* e_qrow,
                  const int32_t* e_child, int32_t n_edges, float* lse, float* lp, void* ws);

// letters: lp[b][c] = h[b n_int] . W[token[c]] (x row scale for fp8 W) for the
// root's children c = 1 .. n_nodes-1, lp[b][0] = 0.
int launch_letter_logits(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                         int32_t n_int, int32_t n_nodes, int32_t d, const void* h, const void* W,
                         const float* w_scale, const int32_t* token, float* lp);

// Greedy decoding in the trie (per-document state on the device).
int launch_decode_init(void* stream, int32_t B, const int32_t* dec_node, const int32_t* sub_label,
                       const int32_t* qrow, int32_t* cur, int32_t* label, int32_t* runs,
                       int32_t* sel, int32_t* row_node, int32_t* n_sel,
                       unsigned long long* best_key);
// y: the projection's fp32 partials [n_part][B][d] (RMSNorm applied in the kernel).
int launch_decode_logits(void* stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                         int32_t d, int32_t n_part, float eps, const float* y, const void* W,
                         const float* w_scale,
                         const int32_t* token, const int32_t* child_begin,
                         const int32_t* child_count, const int32_t* row_node, const int32_t* n_sel,
                         int32_t max_children, unsigned long long* best_key);
int launch_decode_advance(void* stream, int32_t B, const int32_t* child_begin,
                          const int32_t* dec_node, const int32_t* sub_label, const int32_t* qrow,
                          unsigned long long* best_key, int32_t* cur, int32_t* label,
                          int32_t* runs, int32_t* sel, int32_t* row_node, int32_t* n_sel);

// Tree attention pieces.
int launch_anc_attn(void* stream, tcs_dtype dt, int32_t n_int, int32_t Hq, int32_t Hkv,
                    int32_t hd, const void* Qn, const void* Kn, const void* Vn,
                    const int32_t* qparent, float scale, float* anc_ml, float* anc_o);
int launch_doc_attn(void* stream, tcs_dtype dt, int32_t B, int32_t n_int, int32_t Hq,
                    int32_t Hkv, int32_t hd, const void* Qn, const void* Kd, const void* Vd,
                    const int32_t* doc_offsets, const float* anc_ml, const float* anc_o,
                    float scale, void* O, const int32_t* sel = nullptr,
                    const int32_t* n_sel = nullptr, void* split = nullptr);
// Scratch of a key-split document attention (partials per row, head and split;
// 0 when that shape runs unsplit); `split` of launch_doc_attn, or null (unsplit).
size_t doc_attn_split_bytes(int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv, int32_t hd);

// Path sums, label softmax and argmax.  lp: edge log-probs [B, n_nodes]; or, with
// lse and node_qrow set, the raw child logits, each edge's log-prob being
// lp - lse[b n_int + node_qrow[node]].
int launch_path_sum(void* stream, int32_t B, const tcs_trie_dev* trie, const float* lp,
                    float* ll, float* prob, int32_t* label, const float* lse = nullptr,
                    const int32_t* node_qrow = nullptr);
// node_qrow[v] = query row of v's parent, for every non-root node v.
int launch_node_qrow(void* stream, const tcs_trie_dev* trie, int32_t* node_qrow);

}  // namespace tcs
