// C-ABI entry points of libtcs: argument checks, workspace layout, and the
// classify chain on one stream.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include <hip/hip_runtime.h>

#include "tcs_internal.h"

namespace tcs {

int launch_attn_simt(void* stream, tcs_dtype dt, int32_t B, int32_t n_int, int32_t Hq, int32_t Hkv,
                     int32_t hd, const void* Qn, const void* Kn, const void* Vn, const void* Kd,
                     const void* Vd, const int32_t* doc_offsets, const int32_t* qparent, float scale,
                     void* O, const int32_t* sel = nullptr, const int32_t* n_sel = nullptr);

static int check_attn_dims(tcs_dtype dt, int32_t Hq, int32_t Hkv, int32_t hd) {
  if (dt != TCS_F32 && dt != TCS_BF16) return fail(TCS_EUNSUPPORTED, "dtype %d not supported", int(dt));
  if (hd != 64 && hd != 128) return fail(TCS_EUNSUPPORTED, "head_dim %d (need 64 or 128)", hd);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(TCS_EINVAL, "heads Hq=%d Hkv=%d (Hq must be a multiple of Hkv)", Hq, Hkv);
  return TCS_OK;
}

static size_t anc_bytes(int32_t n_int, int32_t Hq, int32_t hd) {
  return align_up(size_t(n_int) * Hq * 8) + align_up(size_t(n_int) * Hq * hd * 4);
}

// Tree attention on a workspace laid out as [anc_ml | anc_o].
static int tree_attn_impl(void* stream, tcs_dtype dt, int32_t B, int32_t n_int, int32_t Hq,
                          int32_t Hkv, int32_t hd, const void* Qn, const void* Kn, const void* Vn,
                          const void* Kd, const void* Vd, const int32_t* doc_offsets,
                          const int32_t* qparent, float scale, void* O, void* ws) {
  if (dt == TCS_F32)
    return launch_attn_simt(stream, dt, B, n_int, Hq, Hkv, hd, Qn, Kn, Vn, Kd, Vd, doc_offsets,
                            qparent, scale, O);
  Carve c(ws);
  float* ml = c.take<float>(size_t(n_int) * Hq * 2);
  float* ao = c.take<float>(size_t(n_int) * Hq * hd);
  int rc = launch_anc_attn(stream, dt, n_int, Hq, Hkv, hd, Qn, Kn, Vn, qparent, scale, ml, ao);
  if (rc) return rc;
  return launch_doc_attn(stream, dt, B, n_int, Hq, Hkv, hd, Qn, Kd, Vd, doc_offsets, ml, ao, scale, O);
}


// Scratch of tcs_tree_attn_noalloc: the path partials live in this file-scope
// device array instead of a caller workspace.  Every GPU the library runs on holds
// its own copy until the process ends.  In host code the array's name is only a
// stand-in: its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[TCS_NOALLOC_SCRATCH_BYTES];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call
// for that device, with the device current).
static int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TCS_EHIP, "tree_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(TCS_EUNSUPPORTED, "tree_attn_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(TCS_EHIP, "tree_attn_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TCS_OK;
}

}  // namespace tcs

using namespace tcs;

extern "C" {

size_t tcs_tree_attn_workspace_bytes(int32_t n_int, int32_t Hq, int32_t hd) {
  return anc_bytes(n_int, Hq, hd);
}

int tcs_tree_attn(tcs_stream stream, tcs_dtype dtype, int32_t B, int32_t n_int, int32_t Hq,
                  int32_t Hkv, int32_t hd, const void* Qn, const void* Kn, const void* Vn,
                  const void* Kd, const void* Vd, const int32_t* doc_offsets,
                  const int32_t* qparent, float scale, void* O, void* ws, size_t ws_bytes) {
  clear_error();
  if (int rc = check_attn_dims(dtype, Hq, Hkv, hd)) return rc;
  if (B < 0 || n_int < 0) return fail(TCS_EINVAL, "tree_attn: B=%d n_int=%d", B, n_int);
  if (B == 0 || n_int == 0) return TCS_OK;
  if (!Qn || !Kn || !Vn || !Kd || !Vd || !doc_offsets || !qparent || !O)
    return fail(TCS_EINVAL, "tree_attn: null pointer");
  if (dtype == TCS_BF16 && (!ws || ws_bytes < anc_bytes(n_int, Hq, hd)))
    return fail(TCS_ECAPACITY, "tree_attn: workspace %zu < %zu bytes", ws_bytes, anc_bytes(n_int, Hq, hd));
  return tree_attn_impl(stream, dtype, B, n_int, Hq, Hkv, hd, Qn, Kn, Vn, Kd, Vd, doc_offsets,
                        qparent, scale, O, ws);
}

static bool head_dtypes_ok(tcs_dtype h_dtype, tcs_dtype w_dtype) {
  if (h_dtype != TCS_F32 && h_dtype != TCS_BF16) return false;
  return w_dtype == h_dtype ||
         (h_dtype == TCS_BF16 && (w_dtype == TCS_FP8_E4M3 || w_dtype == TCS_FP8_E4M3_A8));
}

int tcs_tree_attn_noalloc(tcs_stream stream, tcs_dtype dtype, int32_t B, int32_t n_int, int32_t Hq,
                          int32_t Hkv, int32_t hd, const void* Qn, const void* Kn, const void* Vn,
                          const void* Kd, const void* Vd, const int32_t* doc_offsets,
                          const int32_t* qparent, float scale, void* O) {
  clear_error();
  if (int rc = check_attn_dims(dtype, Hq, Hkv, hd)) return rc;
  if (B < 0 || n_int < 0) return fail(TCS_EINVAL, "tree_attn_noalloc: B=%d n_int=%d", B, n_int);
  if (B == 0 || n_int == 0) return TCS_OK;
  if (!Qn || !Kn || !Vn || !Kd || !Vd || !doc_offsets || !qparent || !O)
    return fail(TCS_EINVAL, "tree_attn_noalloc: null pointer");
  const size_t need = dtype == TCS_BF16 ? anc_bytes(n_int, Hq, hd) : 0;
  if (need > TCS_NOALLOC_SCRATCH_BYTES)
    return fail(TCS_ECAPACITY,
                "tree_attn_noalloc: %d rows x %d heads need %zu bytes of scratch, more than the "
                "built-in %zu (use tcs_tree_attn with a workspace)",
                n_int, Hq, need, size_t(TCS_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0)
    if (int rc = noalloc_scratch(&ws)) return rc;
  return tree_attn_impl(stream, dtype, B, n_int, Hq, Hkv, hd, Qn, Kn, Vn, Kd, Vd, doc_offsets,
                        qparent, scale, O, ws);
}

size_t tcs_lmhead_workspace_bytes(tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                                  int32_t n_nodes, int32_t d, int32_t V) {
  if (!head_dtypes_ok(h_dtype, w_dtype)) return 0;
  if (B < 0 || n_int < 1 || n_nodes < 2 || d < 1 || V < 1 || int64_t(B) * n_int > INT32_MAX) return 0;
  return lmhead_ws_bytes(h_dtype, w_dtype, B, n_int, n_nodes, d, V);
}

int tcs_lmhead_lse_gather(tcs_stream stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                          int32_t n_int, int32_t n_nodes, int32_t d, int32_t V, const void* h,
                          const void* W, const float* w_scale, const int32_t* e_tok,
                          const int32_t* e_qrow, const int32_t* e_child, float* lse, float* lp,
                          void* ws, size_t ws_bytes) {
  clear_error();
  if (!head_dtypes_ok(h_dtype, w_dtype))
    return fail(TCS_EUNSUPPORTED, "lmhead: weight dtype %d with h dtype %d", int(w_dtype), int(h_dtype));
  if (B < 0 || n_int < 1 || n_nodes < 2 || d < 1 || V < 1)
    return fail(TCS_EINVAL, "lmhead: B=%d n_int=%d n_nodes=%d d=%d V=%d", B, n_int, n_nodes, d, V);
  if (h_dtype == TCS_BF16 && d % 64 != 0)
    return fail(TCS_EUNSUPPORTED, "lmhead: bf16 head needs d %% 64 == 0 (d=%d)", d);
  if (w_dtype == TCS_FP8_E4M3_A8 && d % 128 != 0)
    return fail(TCS_EUNSUPPORTED, "lmhead: W8A8 head needs d %% 128 == 0 (d=%d)", d);
  if (B == 0) return TCS_OK;
  const bool fp8_w = w_dtype == TCS_FP8_E4M3 || w_dtype == TCS_FP8_E4M3_A8;
  if (!h || !W || !e_tok || !e_qrow || !e_child || !lse || !lp || (fp8_w && !w_scale))
    return fail(TCS_EINVAL, "lmhead: null pointer");
  const int64_t rows = int64_t(B) * n_int;
  if (rows > INT32_MAX) return fail(TCS_EINVAL, "lmhead: %lld rows", (long long)rows);
  const size_t need = lmhead_ws_bytes(h_dtype, w_dtype, B, n_int, n_nodes, d, V);
  if (!ws || ws_bytes < need) return fail(TCS_ECAPACITY, "lmhead: workspace %zu < %zu bytes", ws_bytes, need);
  return launch_lmhead(stream, h_dtype, w_dtype, B, n_int, n_nodes, d, V, h, W, w_scale, e_tok,
                       e_qrow, e_child, n_nodes - 1, lse, lp, ws);
}

int tcs_path_sum_softmax(tcs_stream stream, int32_t B, const tcs_trie_dev* trie, const float* lp,
                         float* ll, float* prob, int32_t* label) {
  clear_error();
  if (!trie) return fail(TCS_EINVAL, "path_sum: null trie");
  if (B < 0 || trie->n_labels < 1 || trie->n_nodes < 2)
    return fail(TCS_EINVAL, "path_sum: B=%d M=%d n_nodes=%d", B, trie->n_labels, trie->n_nodes);
  if (B == 0) return TCS_OK;
  if (!lp || !ll || !label || !trie->parent || !trie->child_begin || !trie->child_count ||
      !trie->label_node || !trie->qparent)
    return fail(TCS_EINVAL, "path_sum: null pointer");
  return launch_path_sum(stream, B, trie, lp, ll, prob, label);
}

// ---------------------------------------------------------------- classify

// Per-label-set state (tcs_classify_prepare): node input rows, node q/k/v, the path
// partials (bf16 models) and the head's gather lists for B documents.
struct PrepLayout {
  size_t total;
  void *a_nodes, *Qn, *Kn, *Vn, *anc, *head, *gemm_zero;
  int32_t* node_qrow;
  size_t gemm_zero_bytes;
};

static PrepLayout prep_layout(const tcs_model* m, const tcs_trie_dev* t, int32_t B, void* buf) {
  const size_t es = dtype_bytes(m->dtype);
  const size_t n_int = t->n_int;
  const size_t qd = size_t(m->Hq) * m->hd, kd = size_t(m->Hkv) * m->hd;
  Carve c(buf);
  PrepLayout P{};
  P.a_nodes = c.take<char>(n_int * m->d * es);
  P.Qn = c.take<char>(n_int * qd * es);
  P.Kn = c.take<char>(n_int * kd * es);
  P.Vn = c.take<char>(n_int * kd * es);
  P.anc = c.take<char>(m->dtype == TCS_BF16 ? anc_bytes(t->n_int, m->Hq, m->hd) : 0);
  P.head = c.take<char>(lmhead_prep_bytes(m->dtype, B, t->n_int, t->n_nodes, m->d, m->V));
  // zero block of the output projection's ring GEMM (padding k-steps)
  const int32_t R = int32_t(size_t(B) * n_int);
  P.gemm_zero_bytes = m->dtype == TCS_BF16 && gemm_ring_ok(R, m->d, int32_t(qd))
                          ? gemm_ring_zero_bytes(int32_t(qd)) : 0;
  P.gemm_zero = c.take<char>(P.gemm_zero_bytes);
  P.node_qrow = c.take<int32_t>(t->n_nodes);
  P.total = c.used;
  return P;
}

// Per-batch workspace (tcs_classify_run).
struct RunLayout {
  size_t total;
  void *a_doc, *Kd, *Vd, *O, *h, *part, *ll, *act8, *asplit;
  float *y, *lse, *lp;
};

static RunLayout run_layout(const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d, void* ws) {
  const size_t es = dtype_bytes(m->dtype);
  const size_t R = size_t(d->B) * t->n_int;
  const size_t qd = size_t(m->Hq) * m->hd, kd = size_t(m->Hkv) * m->hd;
  Carve c(ws);
  RunLayout L{};
  if (!d->Kd) {
    const size_t T = d->total_tokens;
    L.a_doc = c.take<char>(T * m->d * es);
    L.Kd = c.take<char>(T * kd * es);
    L.Vd = c.take<char>(T * kd * es);
  }
  L.O = c.take<char>(R * qd * es);
  L.y = c.take<float>(R * m->d * gemm_resid_splits(m->dtype, int32_t(R), m->d, int32_t(qd)));
  L.h = c.take<char>(R * m->d * es);
  L.part = c.take<char>(lmhead_part_bytes(m->dtype, d->B, t->n_int, m->V));
  L.lse = c.take<float>(R);
  L.lp = c.take<float>(size_t(d->B) * t->n_nodes);
  L.ll = c.take<float>(size_t(d->B) * t->n_labels);
  L.act8 = c.take<char>(lmhead_act8_bytes(m->head_dtype, int32_t(R), m->d));
  L.asplit = c.take<char>(m->dtype == TCS_BF16 ? doc_attn_split_bytes(d->B, t->n_int, m->Hq, m->Hkv, m->hd) : 0);
  L.total = c.used;
  return L;
}

static int check_classify(const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d) {
  if (!m || !t || !d) return fail(TCS_EINVAL, "classify: null model/trie/docs");
  if (int rc = check_attn_dims(m->dtype, m->Hq, m->Hkv, m->hd)) return rc;
  if (!(m->head_dtype == m->dtype ||
        (m->dtype == TCS_BF16 && (m->head_dtype == TCS_FP8_E4M3 || m->head_dtype == TCS_FP8_E4M3_A8))))
    return fail(TCS_EUNSUPPORTED, "classify: head dtype %d with model dtype %d", int(m->head_dtype),
                int(m->dtype));
  if (m->d < 1 || m->V < 1) return fail(TCS_EINVAL, "classify: d=%d V=%d", m->d, m->V);
  if (m->dtype == TCS_BF16 && m->d % 64 != 0)
    return fail(TCS_EUNSUPPORTED, "classify: bf16 model needs d %% 64 == 0 (d=%d)", m->d);
  if (m->head_dtype == TCS_FP8_E4M3_A8 && m->d % 128 != 0)
    return fail(TCS_EUNSUPPORTED, "classify: W8A8 head needs d %% 128 == 0 (d=%d)", m->d);
  if (!m->E || !m->Wq || !m->Wk || !m->Wv || !m->Wo || !m->W ||
      ((m->head_dtype == TCS_FP8_E4M3 || m->head_dtype == TCS_FP8_E4M3_A8) && !m->W_scale))
    return fail(TCS_EINVAL, "classify: null weight pointer");
  if (t->n_nodes < 2 || t->n_int < 1 || t->n_labels < 1)
    return fail(TCS_EINVAL, "classify: trie with %d nodes, %d rows, %d labels", t->n_nodes, t->n_int,
                t->n_labels);
  if (!t->parent || !t->token || !t->child_begin || !t->child_count || !t->qnode || !t->qparent ||
      !t->label_node || !t->e_tok || !t->e_qrow || !t->e_child)
    return fail(TCS_EINVAL, "classify: null trie array");
  if (d->B < 0 || d->total_tokens < 0) return fail(TCS_EINVAL, "classify: B=%d tokens=%d", d->B, d->total_tokens);
  if (d->B > 0 && !d->doc_offsets) return fail(TCS_EINVAL, "classify: null doc_offsets");
  if (d->B > 0 && !d->Kd && !d->doc_tokens) return fail(TCS_EINVAL, "classify: docs need Kd/Vd or tokens");
  if (d->Kd && !d->Vd) return fail(TCS_EINVAL, "classify: Kd without Vd");
  if (int64_t(d->B) * t->n_int > INT32_MAX) return fail(TCS_EINVAL, "classify: too many rows");
  return TCS_OK;
}

static int check_model_trie(const tcs_model* m, const tcs_trie_dev* t) {
  if (!m || !t) return fail(TCS_EINVAL, "classify: null model/trie");
  tcs_docs none{};
  return check_classify(m, t, &none);
}

// Node input block, path partials and head gather lists for batches of B documents.
static int prepare_impl(void* stream, const tcs_model* m, const tcs_trie_dev* t, int32_t B,
                        void* buf) {
  const PrepLayout P = prep_layout(m, t, B, buf);
  const tcs_dtype dt = m->dtype;
  const int n_int = t->n_int;
  const int qd = m->Hq * m->hd, kd = m->Hkv * m->hd;
  const float scale = 1.0f / std::sqrt(float(m->hd));
  int rc;
  // a = RMSNorm(E[token]); q, k, v
  if ((rc = launch_embed_rmsnorm(stream, dt, m->E, t->qnode, t->token, n_int, m->d, m->V, m->eps, P.a_nodes))) return rc;
  if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, n_int, qd, m->d, P.a_nodes, m->d, m->Wq, m->d, P.Qn, qd, nullptr))) return rc;
  if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, n_int, kd, m->d, P.a_nodes, m->d, m->Wk, m->d, P.Kn, kd, nullptr))) return rc;
  if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, n_int, kd, m->d, P.a_nodes, m->d, m->Wv, m->d, P.Vn, kd, nullptr))) return rc;
  if (dt == TCS_BF16) {
    Carve c(P.anc);
    float* ml = c.take<float>(size_t(n_int) * m->Hq * 2);
    float* ao = c.take<float>(size_t(n_int) * m->Hq * m->hd);
    if ((rc = launch_anc_attn(stream, dt, n_int, m->Hq, m->Hkv, m->hd, P.Qn, P.Kn, P.Vn, t->qparent, scale, ml, ao))) return rc;
  }
  if ((rc = launch_zero_fill(stream, P.gemm_zero, P.gemm_zero_bytes))) return rc;
  if ((rc = launch_node_qrow(stream, t, P.node_qrow))) return rc;
  return launch_lmhead_prep(stream, dt, B, n_int, t->n_nodes, m->d, m->V, t->e_tok, t->e_qrow,
                            t->e_child, t->n_nodes - 1, P.head);
}

// One batch on prepared state.  letters: the trie is the letters' one-level trie and
// the head computes only the letter rows, with no log-sum-exp.
static int run_impl(void* stream, const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d,
                    const void* prep_buf, int32_t* label, float* prob, float* ll, void* ws,
                    bool letters = false) {
  const PrepLayout P = prep_layout(m, t, d->B, const_cast<void*>(prep_buf));
  const RunLayout L = run_layout(m, t, d, ws);
  const tcs_dtype dt = m->dtype;
  const int n_int = t->n_int, B = d->B, R = B * n_int;
  const int qd = m->Hq * m->hd, kd = m->Hkv * m->hd;
  const float scale = 1.0f / std::sqrt(float(m->hd));
  int rc;
  const void* Kd = d->Kd;
  const void* Vd = d->Vd;
  if (!Kd) {  // documents given as tokens: their k and v through the same input block
    const int T = d->total_tokens;
    if ((rc = launch_embed_rmsnorm(stream, dt, m->E, d->doc_tokens, nullptr, T, m->d, m->V, m->eps, L.a_doc))) return rc;
    if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, T, kd, m->d, L.a_doc, m->d, m->Wk, m->d, L.Kd, kd, nullptr))) return rc;
    if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, T, kd, m->d, L.a_doc, m->d, m->Wv, m->d, L.Vd, kd, nullptr))) return rc;
    Kd = L.Kd;
    Vd = L.Vd;
  }
  if (dt == TCS_F32) {
    rc = launch_attn_simt(stream, dt, B, n_int, m->Hq, m->Hkv, m->hd, P.Qn, P.Kn, P.Vn, Kd, Vd,
                          d->doc_offsets, t->qparent, scale, L.O);
  } else {
    Carve c(P.anc);
    const float* ml = c.take<float>(size_t(n_int) * m->Hq * 2);
    const float* ao = c.take<float>(size_t(n_int) * m->Hq * m->hd);
    rc = launch_doc_attn(stream, dt, B, n_int, m->Hq, m->Hkv, m->hd, P.Qn, Kd, Vd, d->doc_offsets,
                         ml, ao, scale, L.O, nullptr, nullptr, L.asplit);
  }
  if (rc) return rc;
  // y = x + O Wo^T ; h = RMSNorm(y)
  GemmResid res{m->E, t->token, t->qnode, n_int};
  if (dt == TCS_BF16 && gemm_ring_ok(R, m->d, qd))
    rc = launch_gemm_ring_resid(stream, R, m->d, qd, L.O, m->Wo, L.y, m->d, res, P.gemm_zero);
  else
    rc = launch_gemm_nt(stream, dt, GEMM_RESID, R, m->d, qd, L.O, qd, m->Wo, qd, L.y, m->d, &res);
  if (rc) return rc;
  if ((rc = launch_rownorm(stream, dt, L.y, R, m->d, gemm_resid_splits(dt, R, m->d, qd), m->eps,
                           L.h))) return rc;
  if (letters) {
    if ((rc = launch_letter_logits(stream, dt, m->head_dtype, B, n_int, t->n_nodes, m->d, L.h, m->W,
                                   m->W_scale, t->token, L.lp))) return rc;
    return launch_path_sum(stream, B, t, L.lp, ll ? ll : static_cast<float*>(L.ll), prob, label);
  }
  // the head leaves raw child logits in lp; the path sum subtracts lse itself
  if ((rc = launch_lmhead_run(stream, dt, m->head_dtype, B, n_int, t->n_nodes, m->d, m->V, L.h, m->W,
                              m->W_scale, t->e_tok, t->e_qrow, t->e_child, L.lse, L.lp, P.head,
                              L.part, false, L.act8))) return rc;
  return launch_path_sum(stream, B, t, L.lp, ll ? ll : static_cast<float*>(L.ll), prob, label,
                         L.lse, P.node_qrow);
}

size_t tcs_classify_prepared_bytes(const tcs_model* model, const tcs_trie_dev* trie, int32_t B) {
  if (B < 1 || check_model_trie(model, trie) || int64_t(B) * trie->n_int > INT32_MAX) return 0;
  return prep_layout(model, trie, B, nullptr).total;
}

int tcs_classify_prepare(tcs_stream stream, const tcs_model* m, const tcs_trie_dev* t, int32_t B,
                         tcs_prepared* prep) {
  clear_error();
  if (int rc = check_model_trie(m, t)) return rc;
  if (!prep || !prep->buf) return fail(TCS_EINVAL, "classify_prepare: null prepared buffer");
  if (B < 1 || int64_t(B) * t->n_int > INT32_MAX) return fail(TCS_EINVAL, "classify_prepare: B=%d", B);
  const size_t need = prep_layout(m, t, B, nullptr).total;
  if (prep->bytes < need)
    return fail(TCS_ECAPACITY, "classify_prepare: buffer %zu < %zu bytes", prep->bytes, need);
  prep->B = B;
  return prepare_impl(stream, m, t, B, prep->buf);
}

size_t tcs_classify_run_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                        const tcs_docs* docs) {
  if (check_classify(model, trie, docs)) return 0;
  return run_layout(model, trie, docs, nullptr).total;
}

int tcs_classify_run(tcs_stream stream, const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d,
                     const tcs_prepared* prep, int32_t* label, float* prob, float* ll, void* ws,
                     size_t ws_bytes) {
  clear_error();
  if (int rc = check_classify(m, t, d)) return rc;
  if (d->B == 0) return TCS_OK;
  if (!label) return fail(TCS_EINVAL, "classify: null label output");
  if (!prep || !prep->buf) return fail(TCS_EINVAL, "classify_run: null prepared state");
  if (prep->B != d->B)
    return fail(TCS_EINVAL, "classify_run: state prepared for B=%d, batch has B=%d", prep->B, d->B);
  if (prep->bytes < prep_layout(m, t, d->B, nullptr).total)
    return fail(TCS_ECAPACITY, "classify_run: prepared buffer too small");
  const size_t need = run_layout(m, t, d, nullptr).total;
  if (!ws || ws_bytes < need) return fail(TCS_ECAPACITY, "classify_run: workspace %zu < %zu bytes", ws_bytes, need);
  return run_impl(stream, m, t, d, prep->buf, label, prob, ll, ws);
}

int tcs_letters_run(tcs_stream stream, const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d,
                    const tcs_prepared* prep, int32_t* label, float* prob, float* ll, void* ws,
                    size_t ws_bytes) {
  clear_error();
  if (int rc = check_classify(m, t, d)) return rc;
  if (t->max_depth != 1 || t->n_int != 1)
    return fail(TCS_EINVAL, "letters: the trie must hold one-token labels only (depth %d, %d rows)",
                t->max_depth, t->n_int);
  if (m->head_dtype == TCS_FP8_E4M3_A8)
    return fail(TCS_EUNSUPPORTED, "letters: fp8 activations are for the full-vocabulary head only");
  if (d->B == 0) return TCS_OK;
  if (!label) return fail(TCS_EINVAL, "letters: null label output");
  if (!prep || !prep->buf) return fail(TCS_EINVAL, "letters: null prepared state");
  if (prep->B != d->B)
    return fail(TCS_EINVAL, "letters: state prepared for B=%d, batch has B=%d", prep->B, d->B);
  if (prep->bytes < prep_layout(m, t, d->B, nullptr).total)
    return fail(TCS_ECAPACITY, "letters: prepared buffer too small");
  const size_t need = run_layout(m, t, d, nullptr).total;
  if (!ws || ws_bytes < need) return fail(TCS_ECAPACITY, "letters: workspace %zu < %zu bytes", ws_bytes, need);
  return run_impl(stream, m, t, d, prep->buf, label, prob, ll, ws, true);
}

// ---------------------------------------------------------------- trie_decode

// Per-batch workspace of tcs_decode_run: document K/V (token documents), then per
// slot the attention output and the projection partials, and the per-document
// decoding state.
struct DecodeLayout {
  size_t total;
  void *a_doc, *Kd, *Vd, *O;
  float* y;
  int32_t *cur, *sel, *row_node, *n_sel, *runs;
  unsigned long long* best_key;
};

static DecodeLayout decode_layout(const tcs_model* m, const tcs_docs* d, void* ws) {
  const size_t es = dtype_bytes(m->dtype);
  const size_t B = d->B > 0 ? d->B : 1;
  const size_t qd = size_t(m->Hq) * m->hd, kd = size_t(m->Hkv) * m->hd;
  Carve c(ws);
  DecodeLayout L{};
  if (!d->Kd) {
    const size_t T = d->total_tokens;
    L.a_doc = c.take<char>(T * m->d * es);
    L.Kd = c.take<char>(T * kd * es);
    L.Vd = c.take<char>(T * kd * es);
  }
  L.O = c.take<char>(B * qd * es);
  L.y = c.take<float>(B * m->d * gemm_resid_splits(m->dtype, int32_t(B), m->d, int32_t(qd)));
  L.cur = c.take<int32_t>(B);
  L.sel = c.take<int32_t>(2 * B);
  L.row_node = c.take<int32_t>(B);
  L.n_sel = c.take<int32_t>(1);
  L.runs = c.take<int32_t>(B);
  L.best_key = c.take<unsigned long long>(B);
  L.total = c.used;
  return L;
}

static int check_decode(const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d) {
  if (int rc = check_classify(m, t, d)) return rc;
  if (!t->sub_label || !t->dec_node || !t->qrow)
    return fail(TCS_EINVAL, "decode: the trie needs its qrow, sub_label and dec_node arrays");
  if (t->max_decode_steps < 0 || t->max_decode_steps > t->max_depth)
    return fail(TCS_EINVAL, "decode: max_decode_steps %d outside [0, %d]", t->max_decode_steps,
                t->max_depth);
  if (t->max_children < 1 || t->max_children >= t->n_nodes)
    return fail(TCS_EINVAL, "decode: max_children %d outside [1, %d)", t->max_children, t->n_nodes);
  if (m->dtype == TCS_BF16 && (m->hd != 128 || m->Hq / m->Hkv > 64))
    return fail(TCS_EUNSUPPORTED, "decode: bf16 models need head_dim 128 (hd=%d)", m->hd);
  if (m->head_dtype == TCS_FP8_E4M3_A8)
    return fail(TCS_EUNSUPPORTED, "decode: fp8 activations are for the full-vocabulary head only");
  return TCS_OK;
}

size_t tcs_decode_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                  const tcs_docs* docs) {
  if (check_decode(model, trie, docs)) return 0;
  return decode_layout(model, docs, nullptr).total;
}

int tcs_decode_run(tcs_stream stream, const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d,
                   const tcs_prepared* prep, int32_t* label, int32_t* runs, void* ws,
                   size_t ws_bytes) {
  clear_error();
  if (int rc = check_decode(m, t, d)) return rc;
  if (d->B == 0) return TCS_OK;
  if (!label) return fail(TCS_EINVAL, "decode: null label output");
  if (!prep || !prep->buf) return fail(TCS_EINVAL, "decode: null prepared state");
  if (prep->B != d->B)
    return fail(TCS_EINVAL, "decode: state prepared for B=%d, batch has B=%d", prep->B, d->B);
  if (prep->bytes < prep_layout(m, t, d->B, nullptr).total)
    return fail(TCS_ECAPACITY, "decode: prepared buffer too small");
  const size_t need = decode_layout(m, d, nullptr).total;
  if (!ws || ws_bytes < need) return fail(TCS_ECAPACITY, "decode: workspace %zu < %zu bytes", ws_bytes, need);

  const PrepLayout P = prep_layout(m, t, d->B, const_cast<void*>(prep->buf));
  const DecodeLayout L = decode_layout(m, d, ws);
  const tcs_dtype dt = m->dtype;
  const int B = d->B, qd = m->Hq * m->hd, kd = m->Hkv * m->hd;
  const float scale = 1.0f / std::sqrt(float(m->hd));
  int32_t* const nruns = runs ? runs : L.runs;
  int rc;
  const void* Kd = d->Kd;
  const void* Vd = d->Vd;
  if (!Kd) {  // documents given as tokens: their k and v through the same input block
    const int T = d->total_tokens;
    if ((rc = launch_embed_rmsnorm(stream, dt, m->E, d->doc_tokens, nullptr, T, m->d, m->V, m->eps, L.a_doc))) return rc;
    if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, T, kd, m->d, L.a_doc, m->d, m->Wk, m->d, L.Kd, kd, nullptr))) return rc;
    if ((rc = launch_gemm_nt(stream, dt, GEMM_STORE, T, kd, m->d, L.a_doc, m->d, m->Wv, m->d, L.Vd, kd, nullptr))) return rc;
    Kd = L.Kd;
    Vd = L.Vd;
  }
  if ((rc = launch_decode_init(stream, B, t->dec_node, t->sub_label, t->qrow, L.cur, label, nruns,
                               L.sel, L.row_node, L.n_sel, L.best_key))) return rc;
  // every launch of a step returns at once when no document is left undecided
  const GemmResid res{m->E, t->token, L.row_node, B, L.n_sel};
  const int splits = gemm_resid_splits(dt, B, m->d, qd);
  for (int step = 0; step < t->max_decode_steps; ++step) {
    // one answer position per undecided document: its node's queries over the
    // document, merged with the node's own path
    if (dt == TCS_F32) {
      rc = launch_attn_simt(stream, dt, B, 1, m->Hq, m->Hkv, m->hd, P.Qn, P.Kn, P.Vn, Kd, Vd,
                            d->doc_offsets, t->qparent, scale, L.O, L.sel, L.n_sel);
    } else {
      Carve c(P.anc);
      const float* ml = c.take<float>(size_t(t->n_int) * m->Hq * 2);
      const float* ao = c.take<float>(size_t(t->n_int) * m->Hq * m->hd);
      rc = launch_doc_attn(stream, dt, B, 1, m->Hq, m->Hkv, m->hd, P.Qn, Kd, Vd, d->doc_offsets,
                           ml, ao, scale, L.O, L.sel, L.n_sel);
    }
    if (rc) return rc;
    if ((rc = launch_gemm_nt(stream, dt, GEMM_RESID, B, m->d, qd, L.O, qd, m->Wo, qd, L.y, m->d,
                             &res))) return rc;
    if ((rc = launch_decode_logits(stream, dt, m->head_dtype, B, m->d, splits, m->eps, L.y, m->W,
                                   m->W_scale,
                                   t->token, t->child_begin, t->child_count, L.row_node, L.n_sel,
                                   t->max_children, L.best_key))) return rc;
    if ((rc = launch_decode_advance(stream, B, t->child_begin, t->dec_node, t->sub_label, t->qrow,
                                    L.best_key, L.cur, label, nruns, L.sel, L.row_node,
                                    L.n_sel))) return rc;
  }
  return TCS_OK;
}

size_t tcs_classify_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                    const tcs_docs* docs) {
  if (check_classify(model, trie, docs)) return 0;
  const int32_t B = docs->B > 0 ? docs->B : 1;
  return prep_layout(model, trie, B, nullptr).total + run_layout(model, trie, docs, nullptr).total;
}

int tcs_classify(tcs_stream stream, const tcs_model* m, const tcs_trie_dev* t, const tcs_docs* d,
                 int32_t* label, float* prob, float* ll, void* ws, size_t ws_bytes) {
  clear_error();
  if (int rc = check_classify(m, t, d)) return rc;
  if (d->B == 0) return TCS_OK;
  if (!label) return fail(TCS_EINVAL, "classify: null label output");
  const size_t pb = prep_layout(m, t, d->B, nullptr).total;
  const size_t need = pb + run_layout(m, t, d, nullptr).total;
  if (!ws || ws_bytes < need)
    return fail(TCS_ECAPACITY, "classify: workspace %zu < %zu bytes", ws_bytes, need);
  if (int rc = prepare_impl(stream, m, t, d->B, ws)) return rc;
  return run_impl(stream, m, t, d, ws, label, prob, ll, static_cast<char*>(ws) + pb);
}

}  // extern "C"
