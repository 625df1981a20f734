/*
 * tcs.h -- C ABI of libtcs, the gfx950 (MI355X) trie_tree label scorer.
 *
 * The library scores every label of a token trie for a batch of documents in one
 * pass, the trie_tree method of "To Classify, Try a Trie Tree" (Quail blog),
 * section 3.2:
 *   - every internal trie node is one answer position; its query attends to the
 *     document's keys/values and to the nodes on its own root-to-node path
 *     (section 3.2, "Custom attention kernel");
 *   - the node's hidden state goes through the full-vocabulary output head, whose
 *     log-sum-exp turns each child edge's logit into a token log-probability
 *     (section 4.1: probabilities need every vocabulary row);
 *   - a label's log score is the sum of the token log-probs on its path; a label
 *     that ends where other labels continue also gets log(1 - P(continue))
 *     (section 3.2, prefix rule); scores are normalised over the labels and the
 *     best label is returned (section 3.2 normalisation, section 2: AI.CLASSIFY
 *     always returns one of the labels; probabilities sum to 1).
 *
 * Conventions for every entry point:
 *   - Ownership: all buffers belong to the caller.  Device entry points take
 *     device pointers, enqueue work on `stream` and return without waiting; the
 *     library never allocates, frees or retains memory.  Scratch memory comes in
 *     through a caller-sized workspace (see the *_workspace_bytes functions).
 *   - Layouts are row-major and densely packed unless a stride is given.
 *     bf16 tensors are 16-bit bfloat16 bit patterns; fp8 tensors are OCP E4M3FN
 *     bytes.  Weight matrices use the [out_features, in_features] layout, so every
 *     projection is y = x W^T.
 *   - Status: 0 on success or a negative TCS_E* code; tcs_last_error() then
 *     returns a message for the calling thread.  Device-side faults surface when
 *     the caller synchronises the stream.  Outputs are undefined after an error.
 *   - The library runs on gfx950 only.
 */
#ifndef TCS_H_
#define TCS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TCS_OK            0
#define TCS_EINVAL       -1  /* null pointer, bad dimension, token outside [0,V), empty label, M < 1 */
#define TCS_EDUPLICATE   -2  /* two labels with the same token sequence */
#define TCS_ECAPACITY    -3  /* output arrays too small; the required sizes are reported */
#define TCS_EUNSUPPORTED -4  /* head_dim, width or dtype combination this build does not run */
#define TCS_EHIP         -5  /* a HIP launch or runtime call failed (message has the HIP string) */
#define TCS_ENOTIMPL     -6

typedef enum {
  TCS_F32 = 0,       /* IEEE fp32 */
  TCS_BF16 = 1,      /* bfloat16 bit patterns */
  TCS_FP8_E4M3 = 2,  /* OCP E4M3FN bytes, with one fp32 scale per row */
  TCS_FP8_E4M3_A8 = 3 /* output head only: E4M3 weights with row scales as TCS_FP8_E4M3, and
                         each hidden row quantized to E4M3 before the head with its own
                         scale max|h|/448 (fp8 x fp8 matrix cores, "W8A8") */
} tcs_dtype;

/* hipStream_t without including HIP headers; NULL is the default stream. */
typedef void* tcs_stream;

/* ------------------------------------------------------------------ trie ---- */

/*
 * Canonical token trie (section 3.1: labels are token paths from the root, the
 * root is the ANSWER: token; labels with a common start share nodes).
 *
 * Node ids are the rank of (depth, token path compared lexicographically by token
 * id): breadth-first order with children in ascending token id, root = 0.  The
 * number of nodes is the number of distinct non-empty label prefixes plus one,
 * the state count of the minimal automaton ("Trie Automata for Constrained
 * Decoding over Large Finite Sets", Proposition 1).  A node with children is
 * internal and owns one query row; rows follow node-id order.  Edges (one per
 * non-root node) are listed sorted by (token, parent row).
 *
 * Every array pointer is caller-owned host memory of the capacity stated.
 */
typedef struct {
  /* capacities, set by the caller */
  int32_t cap_nodes;     /* entries in each per-node array, in qnode/qparent, and in each
                            edge array (edges need cap_nodes - 1) */
  int32_t cap_levels;    /* entries in level_offsets (needs max_depth + 2) */
  /* sizes, set by tcs_trie_build (also on TCS_ECAPACITY) */
  int32_t n_nodes, n_int, n_labels, max_depth;
  /* per node [cap_nodes] */
  int32_t* parent;       /* parent id, -1 at the root */
  int32_t* token;        /* token id; the root holds root_token */
  int32_t* depth;
  int32_t* child_begin;  /* id of the first child, 0 for a leaf */
  int32_t* child_count;
  int32_t* node_label;   /* label ending at the node, -1 if none */
  int32_t* qrow;         /* query row of an internal node, -1 for a leaf */
  /* per query row [cap_nodes] (n_int used) */
  int32_t* qnode;        /* node id of the row */
  int32_t* qparent;      /* row of the parent node, -1 for the root */
  /* per label [M] */
  int32_t* label_node;
  /* per level [cap_levels] */
  int32_t* level_offsets; /* first node of each depth, then n_nodes */
  /* per edge [cap_nodes] (n_nodes - 1 used), sorted by (e_tok, e_qrow) */
  int32_t* e_tok;
  int32_t* e_qrow;       /* query row of the edge's parent */
  int32_t* e_child;      /* node id of the edge's child */
  /* optional (may be NULL): derived arrays for the level-by-level path sums */
  int32_t* row_level_offsets; /* [cap_levels] first query row of each depth, then n_int */
  int32_t* label_row;    /* [M] row whose prefix sum a label's score starts from: its
                            node's row if the node is internal, else its parent's */
  /* optional (may be NULL): tables of greedy decoding (tcs_decode_run) */
  int32_t* sub_label;    /* [cap_nodes] the label if the node's subtree holds exactly one
                            label, else -1 */
  int32_t* dec_node;     /* [cap_nodes] where decoding goes on from the node: follow single
                            children while the subtree holds more than one label */
  int32_t max_decode_steps; /* set with the tables: the most model runs any label needs */
  int32_t max_children;     /* set with the tables: the most children of any node */
} tcs_trie;

/*
 * Build the trie of M labels given as CSR: label m is label_tokens[label_offsets[m]
 * .. label_offsets[m+1]).  Labels keep their input order as label ids.
 * Errors: TCS_EINVAL (M < 1, an empty label, a token or root_token outside [0,V)),
 * TCS_EDUPLICATE (two equal labels), TCS_ECAPACITY (out->n_nodes / max_depth hold
 * the sizes needed).  Host only; no GPU needed.
 */
int tcs_trie_build(const int32_t* label_offsets, const int32_t* label_tokens, int32_t M,
                   int32_t root_token, int32_t V, tcs_trie* out);

/*
 * Decision-word cut of a label set ("To Classify, Try a Trie Tree", section 3.2):
 * trie_tree scores a label through the last token of the word in which its token
 * prefix stops being shared with any other label.  For label m, k is the first position whose token prefix (tokens
 * 1..k) no other label shares; the word holding token k goes on while the next
 * token is a word continuation (word_cont[token] != 0), and d_m is the position of
 * its last token.  A label that shares all its prefixes -- it is the start of
 * another label -- keeps every token (d_m = its length) and is scored with the
 * prefix rule.  Label m of the output is label m cut to its first d_m tokens.
 *
 * Running tcs_trie_build and tcs_classify on the cut labels gives exactly the
 * decision-word scores: the cut labels are distinct, and one is the start of
 * another only where the labels were, with the same next tokens, so the prefix
 * rule is unchanged.  Label ids keep their order.
 *
 * label_offsets [M+1], label_tokens [label_offsets[M]]: labels as for
 * tcs_trie_build.  word_cont [V]: one byte per vocabulary token, nonzero for a
 * token that continues the previous token's word.  out_offsets [M+1] and
 * out_tokens [label_offsets[M]] (never more than that is written) receive the cut
 * labels as CSR; depth [M] (may be NULL) receives d_m.  All host memory, caller
 * owned.  Errors: TCS_EINVAL (a null pointer, M < 1, an empty label, a token
 * outside [0,V)), TCS_EDUPLICATE (two equal labels).  Host only; no GPU needed.
 */
int tcs_decision_truncate(const int32_t* label_offsets, const int32_t* label_tokens, int32_t M,
                          int32_t V, const uint8_t* word_cont, int32_t* out_offsets,
                          int32_t* out_tokens, int32_t* depth);

/* Device copy of the trie arrays needed by the kernels (all device pointers). */
typedef struct {
  int32_t n_nodes, n_int, n_labels, max_depth;
  const int32_t* parent;       /* [n_nodes] */
  const int32_t* token;        /* [n_nodes] */
  const int32_t* child_begin;  /* [n_nodes] */
  const int32_t* child_count;  /* [n_nodes] */
  const int32_t* qnode;        /* [n_int] */
  const int32_t* qparent;      /* [n_int] */
  const int32_t* label_node;   /* [n_labels] */
  const int32_t* e_tok;        /* [n_nodes-1] sorted */
  const int32_t* e_qrow;       /* [n_nodes-1] */
  const int32_t* e_child;      /* [n_nodes-1] */
  /* optional (NULL: the path sums walk each label's path instead) */
  const int32_t* qrow;               /* [n_nodes] */
  const int32_t* row_level_offsets;  /* [max_depth + 2] */
  const int32_t* label_row;          /* [n_labels] */
  /* optional (NULL unless tcs_decode_run is used) */
  const int32_t* sub_label;          /* [n_nodes] */
  const int32_t* dec_node;           /* [n_nodes] */
  int32_t max_decode_steps;
  int32_t max_children;
} tcs_trie_dev;

/* --------------------------------------------------------- tree attention ---- */

/*
 * Ancestor-masked tree attention (section 3.2, "Custom attention kernel": all
 * answer nodes of a document in one request; a node's keys are the document's and
 * those of its ancestors and itself, none from other branches).
 *
 * For document b, query row r (internal node u) and query head h, the keys are
 * the document's keys Kd[doc_offsets[b] .. doc_offsets[b+1]) followed by the node
 * keys of every row on the root-to-u path, u included (walk qparent from r).  KV
 * head of query head h is h / (Hq/Hkv).  Output is softmax(q.k * scale) . v.
 *
 *   dtype       TCS_F32 or TCS_BF16: storage of Qn/Kn/Vn/Kd/Vd/O; math in fp32.
 *   Qn          [n_int, Hq, hd]     node queries (shared by every document)
 *   Kn, Vn      [n_int, Hkv, hd]    node keys / values
 *   Kd, Vd      [sum L_b, Hkv, hd]  document keys / values, documents back to back
 *   doc_offsets [B+1] device        prefix sums of document lengths (L_b may be 0)
 *   qparent     [n_int] device      tcs_trie.qparent
 *   O           [B, n_int, Hq, hd]  output, rounded to dtype
 *   ws          workspace of tcs_tree_attn_workspace_bytes(n_int, Hq, hd) bytes
 * hd must be 64 or 128 and Hq a multiple of Hkv (else TCS_EUNSUPPORTED / TCS_EINVAL).
 */
size_t tcs_tree_attn_workspace_bytes(int32_t n_int, int32_t Hq, int32_t hd);
int tcs_tree_attn(tcs_stream stream, tcs_dtype dtype, int32_t B, int32_t n_int, int32_t Hq,
                  int32_t Hkv, int32_t hd, const void* Qn, const void* Kn, const void* Vn,
                  const void* Kd, const void* Vd, const int32_t* doc_offsets,
                  const int32_t* qparent, float scale, void* O, void* ws, size_t ws_bytes);

/*
 * tcs_tree_attn without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  Arguments, layouts and results are those of
 * tcs_tree_attn (same kernels, bit-identical output).  The scratch that
 * tcs_tree_attn takes from `ws` (tcs_tree_attn_workspace_bytes(n_int, Hq, hd)
 * bytes: the per-(row, head) path partials) lives instead in a device array inside
 * the library of TCS_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held until the
 * process ends; its address is looked up once per device on the first call with
 * that device current.  No memory is allocated or freed by the call.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and give undefined results; calls in
 * order on one stream are safe.  Each call rewrites every scratch entry it reads,
 * so nothing needs clearing between calls.
 * Errors: as tcs_tree_attn, and TCS_ECAPACITY when the scratch needed exceeds
 * TCS_NOALLOC_SCRATCH_BYTES (about 32,000 (row, head) pairs at head_dim 128, e.g.
 * 1,008 query rows with 32 heads), TCS_EHIP if the array's address cannot be found.
 */
#define TCS_NOALLOC_SCRATCH_BYTES (16u << 20)
int tcs_tree_attn_noalloc(tcs_stream stream, tcs_dtype dtype, int32_t B, int32_t n_int,
                          int32_t Hq, int32_t Hkv, int32_t hd, const void* Qn, const void* Kn,
                          const void* Vn, const void* Kd, const void* Vd,
                          const int32_t* doc_offsets, const int32_t* qparent, float scale,
                          void* O);

/* ------------------------------------------------------------- LM head ---- */

/*
 * Full-vocabulary output head with the log-sum-exp and the child-token gather
 * fused in (section 4.1: F_head = 2 d V per answer position; the [rows x V] logits
 * are never stored).
 *
 * Rows: r = b * n_int + q for document b and query row q (R = B * n_int rows).
 *   logit[r, v] = h[r] . W[v]            (times w_scale[v] for an fp8 head)
 *   lse[r]      = log sum_v exp(logit[r, v])
 *   lp[b, c]    = logit[b*n_int + e_qrow, e_tok] - lse[b*n_int + e_qrow] for every
 *                 edge (e_tok, e_qrow, e_child = c); lp[b, 0] = 0 for the root.
 *
 *   h_dtype     TCS_F32 or TCS_BF16: storage of h.
 *   w_dtype     h_dtype, or (with h_dtype TCS_BF16) TCS_FP8_E4M3 plus w_scale [V] fp32, or
 *               TCS_FP8_E4M3_A8: the same fp8 weights, and each row of h first quantized to
 *               E4M3 with its own scale max|h_r|/448 (codes and scales live in ws), the
 *               logit then being s_r * w_scale[v] * (codes_r . codes_v).
 *   h           [R, d];  W [V, d]
 *   edges       trie->e_tok / e_qrow / e_child, sorted by token
 *   lse         [R] fp32 out;  lp [B, n_nodes] fp32 out
 *   ws          workspace of tcs_lmhead_workspace_bytes(h_dtype, w_dtype, B, n_int, n_nodes,
 *               d, V) bytes (0 for invalid sizes or dtype pairs)
 * bf16 heads need d % 64 == 0, the W8A8 head d % 128 == 0.  Errors: TCS_EUNSUPPORTED (dtype
 * pair, d), TCS_EINVAL (sizes,
 * null pointers, w_scale missing for an fp8 head), TCS_ECAPACITY (short workspace).
 */
size_t tcs_lmhead_workspace_bytes(tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B, int32_t n_int,
                                  int32_t n_nodes, int32_t d, int32_t V);
int tcs_lmhead_lse_gather(tcs_stream stream, tcs_dtype h_dtype, tcs_dtype w_dtype, int32_t B,
                          int32_t n_int, int32_t n_nodes, int32_t d, int32_t V, const void* h,
                          const void* W, const float* w_scale, const int32_t* e_tok,
                          const int32_t* e_qrow, const int32_t* e_child, float* lse, float* lp,
                          void* ws, size_t ws_bytes);

/* ------------------------------------------------------------ path sums ---- */

/*
 * Per-label log score, label softmax and argmax (section 3.2).
 *   ll[b, m]  = sum of lp[b, .] over the path root -> label_node[m], plus
 *               log(1 - sum_{children c} exp(lp[b, c])) when label_node[m] has
 *               children (-inf if the children take all mass).  Up to 512 labels,
 *               or without the trie arrays for level-by-level sums, each label's
 *               path is walked with fp64 sums; past 512 labels with the arrays the
 *               sums run level by level as a pair of fp32 values (about 2^-33
 *               relative error per step).  The prefix term is fp64.
 *   prob[b,.] = softmax over m of ll[b, .]            (optional: prob may be NULL)
 *   label[b]  = argmax_m ll[b, m] of the returned (fp32) ll, lowest label id among
 *               equal maxima
 * lp is [B, n_nodes] fp32 with lp[b, 0] = 0; ll and prob are [B, M] fp32.
 */
int tcs_path_sum_softmax(tcs_stream stream, int32_t B, const tcs_trie_dev* trie, const float* lp,
                         float* ll, float* prob, int32_t* label);

/* ------------------------------------------------------------- classify ---- */

/*
 * Model of one answer position: a single attention layer and the output head.
 *   x = E[token]; a = RMSNorm(x); q,k,v = a Wq^T, a Wk^T, a Wv^T   (no positions)
 *   o = tree attention (above);  y = x + o Wo^T;  h = RMSNorm(y);  head(h)
 * RMSNorm has gain 1 and epsilon `eps`.  In bf16 models a, q, k, v, o and h are
 * stored (rounded to nearest-even) in bf16; y stays fp32.
 */
typedef struct {
  tcs_dtype dtype;       /* TCS_F32 or TCS_BF16: E, Wq, Wk, Wv, Wo and activations */
  tcs_dtype head_dtype;  /* dtype, or for bf16 models TCS_FP8_E4M3 (W8A16) or TCS_FP8_E4M3_A8
                            (W8A8, d % 128 == 0: tcs_classify / tcs_classify_run only;
                            tcs_letters_run and tcs_decode_run answer TCS_EUNSUPPORTED) */
  int32_t d, Hq, Hkv, hd, V;
  float eps;
  const void* E;         /* [V, d] token embeddings */
  const void* Wq;        /* [Hq*hd, d] */
  const void* Wk;        /* [Hkv*hd, d] */
  const void* Wv;        /* [Hkv*hd, d] */
  const void* Wo;        /* [d, Hq*hd] */
  const void* W;         /* [V, d] output head */
  const float* W_scale;  /* [V] for an fp8 head, else NULL */
} tcs_model;

/*
 * A batch of documents: either their precomputed keys/values (Kd, Vd) or their
 * token ids (doc_tokens), in which case the library computes each token's k and v
 * with the model's input block.
 */
typedef struct {
  int32_t B;
  int32_t total_tokens;          /* doc_offsets[B] */
  const int32_t* doc_offsets;    /* [B+1] device */
  const void* Kd;                /* [total_tokens, Hkv, hd] model dtype, or NULL */
  const void* Vd;
  const int32_t* doc_tokens;     /* [total_tokens] device, used when Kd is NULL */
} tcs_docs;

/*
 * The whole trie_tree pass on one stream: node input block, tree attention,
 * output projection + residual + RMSNorm, output head with LSE and gather, path
 * sums, label softmax and argmax.
 *   label [B] int32 out; prob [B, M] fp32 out or NULL; ll [B, M] fp32 out or NULL.
 *   ws    workspace of tcs_classify_workspace_bytes(model, trie, docs) bytes (the
 *         prepared state of tcs_classify_prepare followed by a run workspace).
 */
size_t tcs_classify_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                    const tcs_docs* docs);
int tcs_classify(tcs_stream stream, const tcs_model* model, const tcs_trie_dev* trie,
                 const tcs_docs* docs, int32_t* label, float* prob, float* ll, void* ws,
                 size_t ws_bytes);

/*
 * The same pass split at the label set.  In this single-layer model a trie node's
 * q, k and v come from its token alone and its attention over its ancestor chain
 * (section 3.2, custom attention kernel) does not involve the document, so they are computed once per label set; so are the output head's
 * gather lists, which depend only on the trie and the batch size B.  The pages run
 * one label set over a whole table of documents (section 2), so this work is paid
 * once per query rather than once per batch.
 *
 * tcs_classify_prepare fills a caller-owned device buffer of
 * tcs_classify_prepared_bytes(model, trie, B) bytes (prep->buf, prep->bytes set
 * by the caller; prep->B is written) with the node q/k/v, the per-(node, head) path
 * partials and the gather lists for batches of exactly B documents.  The buffer
 * must stay untouched while runs use it; the trie and weights must not change.
 * tcs_classify_run scores one batch (docs->B == prep->B) with that state on a
 * workspace of tcs_classify_run_workspace_bytes(model, trie, docs) bytes; it gives
 * the same results as tcs_classify.  Errors: EINVAL for a batch size other than
 * prep->B or null pointers; ECAPACITY for short buffers.
 */
typedef struct {
  int32_t B;     /* batch size the state was prepared for (written by prepare) */
  void* buf;     /* device buffer, caller-owned */
  size_t bytes;  /* its size */
} tcs_prepared;
size_t tcs_classify_prepared_bytes(const tcs_model* model, const tcs_trie_dev* trie, int32_t B);
int tcs_classify_prepare(tcs_stream stream, const tcs_model* model, const tcs_trie_dev* trie,
                         int32_t B, tcs_prepared* prep);
size_t tcs_classify_run_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                        const tcs_docs* docs);
int tcs_classify_run(tcs_stream stream, const tcs_model* model, const tcs_trie_dev* trie,
                     const tcs_docs* docs, const tcs_prepared* prep, int32_t* label, float* prob,
                     float* ll, void* ws, size_t ws_bytes);

/*
 * letters ("To Classify, Try a Trie Tree", section 3.3): the prompt shows each
 * label behind its own letter and the answer is one letter token.  The model runs
 * at one answer position per document, the ANSWER: position (the trie's root,
 * attending to the document and to itself); the M letter logits are read there,
 * rescaled to sum to 1 over the letters and the best letter's label is returned.
 * Since every label is one token, the output head computes only the M letter rows
 * (section 4.1): the vocabulary log-sum-exp would cancel in the rescale and is
 * never formed.
 *
 * `trie` is tcs_trie_build's trie of the M letter tokens as one-token labels
 * (label m = letter token m; max_depth 1, one query row), with root_token the
 * ANSWER: token.  `prep` comes from tcs_classify_prepare for that trie and B,
 * `ws` holds tcs_classify_run_workspace_bytes(model, trie, docs) bytes.
 * Outputs (device): label [B]; prob [B, M] (may be NULL): the rescaled
 * probabilities; ll [B, M] (may be NULL): the letter logits, i.e. log scores up to
 * a per-document constant.  Errors as tcs_classify_run, and TCS_EINVAL for a trie
 * with a label longer than one token.
 */
int tcs_letters_run(tcs_stream stream, const tcs_model* model, const tcs_trie_dev* trie,
                    const tcs_docs* docs, const tcs_prepared* prep, int32_t* label, float* prob,
                    float* ll, void* ws, size_t ws_bytes);

/*
 * trie_decode ("To Classify, Try a Trie Tree", section 3.1): the label is
 * generated greedily inside the trie.  Each document starts at the root (the
 * ANSWER: token).  Where labels branch (a node with several children and more
 * than one label below it) the model runs at that node -- its query attends to
 * the document and to the node's own path, as in tree attention -- and the child
 * whose token has the highest logit is taken (the lowest token id on ties; the
 * vocabulary normaliser is shared by the candidates, so logits decide and no
 * log-sum-exp is formed).  A node with one child is passed without a run; a
 * document stops once one label remains below its node.  All undecided documents
 * take one step together; a label that is the start of another is never returned
 * (there is no stop token: section 3.1, note 2).  No probabilities are produced.
 *
 * `trie` needs the optional qrow, sub_label and dec_node arrays, max_decode_steps
 * and max_children (tcs_trie_build fills them when given the arrays); `prep` comes
 * from tcs_classify_prepare for that trie and B; `ws` holds
 * tcs_decode_workspace_bytes(model, trie, docs) bytes (0: invalid arguments).
 * Runs max_decode_steps steps on `stream` with no host synchronisation; documents
 * that are decided early skip the later steps' work.
 * Outputs (device): label [B]; runs [B] (may be NULL): model runs per document.
 * Errors as tcs_classify_run; TCS_EINVAL without the decoding arrays;
 * TCS_EUNSUPPORTED for bf16 models with head_dim other than 128.
 */
size_t tcs_decode_workspace_bytes(const tcs_model* model, const tcs_trie_dev* trie,
                                  const tcs_docs* docs);
int tcs_decode_run(tcs_stream stream, const tcs_model* model, const tcs_trie_dev* trie,
                   const tcs_docs* docs, const tcs_prepared* prep, int32_t* label, int32_t* runs,
                   void* ws, size_t ws_bytes);

/* ----------------------------------------------------------- measurement ---- */
/*
 * Per-kernel timing, for measuring a kernel against its roofline from inside a
 * timed run (not part of the scoring method).  While timing is enabled, every
 * launch of a timed kernel is bracketed by two HIP events recorded on the stream
 * it is launched on; tcs_timing_read waits for the recorded events of one timer,
 * returns their summed duration and launch count, and forgets them.
 *
 *   tcs_timing_enable(1)  starts recording (events are created on demand and
 *                         pooled; they are HIP events, not device memory).
 *   tcs_timing_enable(0)  stops recording, drops unread records and destroys the
 *                         pooled events.
 *   tcs_timing_read(timer, &ms, &n)  ms = total milliseconds, n = launches since
 *                         the last read; TCS_EINVAL for an unknown timer or NULL
 *                         outputs, TCS_EHIP if an event query fails.
 *
 * Launches from several host threads at once are recorded safely, but a timer's
 * total then mixes their streams.
 */
typedef enum {
  TCS_TIMER_HEAD = 0,     /* the output-head GEMM + LSE/gather kernel (any dtype) */
  TCS_TIMER_DOC_ATTN = 1, /* the document part of the tree attention */
  TCS_TIMER_COUNT = 2
} tcs_timer;
int tcs_timing_enable(int enable);
int tcs_timing_read(int timer, double* total_ms, int32_t* launches);

/* Message for the last failing call on this thread ("" if none). */
const char* tcs_last_error(void);

/* Library version string. */
const char* tcs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TCS_H_ */
