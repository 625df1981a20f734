"""Plain, slow, fp64 oracle of the trie_tree label-scoring path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP library and imports nothing from it.

Sources (cited by page title and section):
  [CT] "To Classify, Try a Trie Tree" (Quail blog): section 3.1 (the label trie,
       root = the ANSWER: token), section 3.2 (trie_tree: label probability is the
       product of its token probabilities; normalisation over labels; the rule for
       a label that is a prefix of another; a node's keys are the document's and
       its ancestors', no other branch's), section 4.1 (full-vocabulary output head).
  [EX] Quail documentation, "Execution", section "Label scoring" (worked example:
       refund 0.8 x 0.6 = 0.48 against praise 0.3).
  [QI] "Building an Ultra-High Throughput AI-SQL Engine", section 3.2.4 (partial
       attention results merged by their log-sum-exp / online softmax).
  [CT] also section 3.1 (trie_decode: greedy generation inside the trie, the model
       only where labels branch, stopping once one label remains; note 2: a label
       that is the start of another is never returned), section 4.3 (requests per
       document, b = mean over labels of the branching nodes on their paths),
       section 3.3 (letters: one letter token per label, read at the ANSWER:
       position and rescaled over the letters) and section 4.1 (when every label is
       one token only the label tokens' head rows are computed).
  [TA] "Trie Automata for Constrained Decoding over Large Finite Sets",
       Proposition 1 (the trie is the minimal automaton: one state per distinct
       prefix).

Readings taken where the pages leave a step open (each is also listed with its
reason in the design notes):
  R1  every label is scored over its full root-to-leaf token path;
  R2  every internal trie node (a node with children) runs the model;
  R3  a prefix label ending at an internal node gets log(1 - sum of its children's
      probabilities) -- the section 3.2 prefix rule generalised to several children;
  R4  a node attends to the document keys and to its ancestors *and itself*;
  R5  no positional encoding; one attention layer: pre-RMSNorm, GQA (query head h
      reads KV head h // (Hq/Hkv)), scale 1/sqrt(hd), output projection, residual,
      final RMSNorm (gain 1, eps 1e-6), then the LM head;
  R6  bf16 workloads round to bf16 (nearest-even) exactly where a bf16 tensor is
      stored: the normalised node input a, the node q/k/v, the attention output O
      and the final hidden state h.  The residual sum y is not rounded;
  R7  the fp8 head holds E4M3FN codes with one fp32 scale per vocabulary row; the
      scale multiplies the dot product;
  R8  argmax ties go to the lowest label id;
  R9  decision-word form ([CT] 3.2): a word is a token plus the tokens after it that
      carry a word-continuation flag (a per-vocabulary input); a label "leaves all
      others" at its first token k such that no other label starts with its first
      k tokens; a label that never does (it is the start of another label) is
      scored over all its tokens, with the prefix rule of R3;
  R10 letters ([CT] 3.3): the letter tokens are M distinct vocabulary ids (an
      input); the one answer position is the root, attending to the document and
      itself as in R4; the returned scores are the letter logits (log scores up to a
      per-document constant, as the vocabulary log-sum-exp is never formed);
  R11 trie_decode ties go to the lowest token id; a decode run at a node is the
      model over [root, path tokens] attending to the document (as in R4/R5);
  R12 W8A8 head ("Building an Ultra-High Throughput AI-SQL Engine", fp8 weights and
      activations): each stored hidden row h (bf16 values) is quantized before the
      head with s = fl32(max|h| / 448) and codes = E4M3(fl32(h / s)), nearest value,
      ties to the even code, saturating at 448 (an all-zero row keeps s = 0); the
      logit is s * s_w * sum(codes_h * codes_w).  The scales are fp32 numbers, as
      the pages' per-row scales are, and the quotient h / s that the rounding to a
      code decides on is taken in that same fp32 precision (correctly rounded):
      where floating point decides an integer code, both sides take the decision in
      the precision the format fixes.

Parity status: every function below is pinned by the non-GPU oracle tests
(library routines, closed forms, the worked example, brute-force scoring).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "TCS_OK", "TCS_EINVAL", "TCS_EDUPLICATE", "TrieError", "Trie", "build_trie",
    "round_bf16", "decode_bf16", "decode_e4m3", "rmsnorm", "OracleModel",
    "node_layer", "doc_kv_from_tokens", "tree_attention", "hidden_states",
    "lm_head_lse", "head_logits_at", "edge_logprobs", "log1mexp", "path_log_likelihoods",
    "label_softmax", "classify", "bruteforce_ll", "label_ll_on_paths",
    "decision_depths", "truncate_labels", "letters_classify", "greedy_walk", "trie_decode",
    "e4m3_encode", "quantize_rows_e4m3",
]

TCS_OK = 0
TCS_EINVAL = -1
TCS_EDUPLICATE = -2


class TrieError(ValueError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


# =========================================================================== trie ([CT] 3.1)

@dataclass
class Trie:
    n_nodes: int
    n_int: int
    n_labels: int
    max_depth: int
    parent: np.ndarray        # [N]   parent node id, -1 at the root
    token: np.ndarray         # [N]   token id of the node (root: root_token)
    depth: np.ndarray         # [N]
    child_begin: np.ndarray   # [N]   first child id, 0 when the node has no child
    child_count: np.ndarray   # [N]
    node_label: np.ndarray    # [N]   label ending at the node, -1 if none
    label_node: np.ndarray    # [M]
    qrow: np.ndarray          # [N]   query row of an internal node, -1 for a leaf
    qnode: np.ndarray         # [N_int] node id of each query row
    qparent: np.ndarray       # [N_int] query row of the parent, -1 for the root
    level_offsets: np.ndarray  # [max_depth + 2]
    e_tok: np.ndarray         # [N-1] edges sorted by (token, parent query row)
    e_qrow: np.ndarray        # [N-1]
    e_child: np.ndarray       # [N-1]


def build_trie(labels, root_token: int, V: int) -> Trie:
    """Token trie of the labels ([CT] 3.1): each label is a root-to-node path.

    Insert the labels in input order into a dict of children, then number the
    nodes breadth-first with each node's children visited in ascending token id.
    That numbering is the rank of (depth, token path compared lexicographically).
    """
    M = len(labels)
    if M < 1:
        raise TrieError(TCS_EINVAL, "need at least one label")
    if not (0 <= root_token < V):
        raise TrieError(TCS_EINVAL, "root token out of range")
    root = {"children": {}, "label": -1}
    for m, lab in enumerate(labels):
        if len(lab) == 0:
            raise TrieError(TCS_EINVAL, f"label {m} is empty")
        node = root
        for t in lab:
            t = int(t)
            if not (0 <= t < V):
                raise TrieError(TCS_EINVAL, f"label {m} has token {t} outside [0, {V})")
            node = node["children"].setdefault(t, {"children": {}, "label": -1})
        if node["label"] >= 0:
            raise TrieError(TCS_EDUPLICATE, f"label {m} duplicates label {node['label']}")
        node["label"] = m

    # breadth-first numbering, children in ascending token order
    order = [(root, -1, int(root_token), 0)]
    head = 0
    while head < len(order):
        node, _, _, dep = order[head]
        for t in sorted(node["children"]):
            order.append((node["children"][t], head, t, dep + 1))
        head += 1
    N = len(order)
    parent = np.array([p for (_, p, _, _) in order], dtype=np.int32)
    token = np.array([t for (_, _, t, _) in order], dtype=np.int32)
    depth = np.array([d for (_, _, _, d) in order], dtype=np.int32)
    child_count = np.array([len(n["children"]) for (n, _, _, _) in order], dtype=np.int32)
    child_begin = np.zeros(N, dtype=np.int32)
    for u in range(N - 1, 0, -1):      # smallest child id of each parent
        child_begin[parent[u]] = u
    node_label = np.array([n["label"] for (n, _, _, _) in order], dtype=np.int32)
    label_node = np.full(M, -1, dtype=np.int32)
    for u in range(N):
        if node_label[u] >= 0:
            label_node[node_label[u]] = u
    internal = child_count > 0
    qnode = np.nonzero(internal)[0].astype(np.int32)
    qrow = np.full(N, -1, dtype=np.int32)
    qrow[qnode] = np.arange(len(qnode), dtype=np.int32)
    qparent = np.array([qrow[parent[u]] if u > 0 else -1 for u in qnode], dtype=np.int32)
    D = int(depth.max())
    level_offsets = np.searchsorted(depth, np.arange(D + 2), side="left").astype(np.int32)
    children = np.arange(1, N)
    e_q = qrow[parent[children]]
    e_t = token[children]
    perm = np.lexsort((e_q, e_t))
    return Trie(
        n_nodes=N, n_int=len(qnode), n_labels=M, max_depth=D, parent=parent, token=token,
        depth=depth, child_begin=child_begin, child_count=child_count, node_label=node_label,
        label_node=label_node, qrow=qrow, qnode=qnode, qparent=qparent,
        level_offsets=level_offsets, e_tok=e_t[perm].astype(np.int32),
        e_qrow=e_q[perm].astype(np.int32), e_child=children[perm].astype(np.int32))


def _path_rows(trie: Trie, r: int):
    """Query rows from the root down to row r (ancestors and r itself)."""
    rows = []
    while r >= 0:
        rows.append(r)
        r = int(trie.qparent[r])
    return rows[::-1]


def _path_nodes(trie: Trie, u: int):
    """Node ids from the root's first child down to node u (root excluded)."""
    nodes = []
    while u > 0:
        nodes.append(u)
        u = int(trie.parent[u])
    return nodes[::-1]


# =========================================================================== number formats

def round_bf16(x):
    """Round fp64 values to the nearest bf16 value (ties to even), returned as fp64.

    bf16 keeps 8 significant bits and fp32's exponent range; below 2^-126 the
    quantum is fixed at 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    r = np.ldexp(np.round(np.ldexp(x, -q)), q)
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)


def decode_bf16(bits):
    """bf16 bit patterns (uint16) -> fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3(codes):
    """OCP E4M3FN bytes -> fp64: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinities.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def e4m3_encode(x):
    """Values -> OCP E4M3FN codes (R12): the nearest finite E4M3 value, ties to the
    even code, magnitudes from 448 up saturating to 448; the sign is kept.

    The candidates are the 127 non-negative finite values decode_e4m3 gives for
    codes 0..126, in increasing order: the two neighbours of |x| are compared.
    """
    x = np.asarray(x, dtype=np.float64)
    vals = decode_e4m3(np.arange(127))
    a = np.abs(x)
    up = np.clip(np.searchsorted(vals, a, side="left"), 1, 126)   # vals[up-1] < a <= vals[up]
    below, above = up - 1, up
    d_below = a - vals[below]
    d_above = vals[above] - a
    code = np.where(d_above < d_below, above, below)
    tie = d_above == d_below
    code = np.where(tie, np.where(above % 2 == 0, above, below), code)
    code = np.where(a >= 448.0, 126, code)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows_e4m3(h):
    """Per-row E4M3 quantization of hidden states (R12): s = fl32(max|h| / 448),
    codes = e4m3_encode(fl32(h / s)); rows of zeros get s = 0 and zero codes.
    h: [R, d] (values representable in fp32).  Returns (codes uint8 [R, d], s [R])."""
    h32 = np.asarray(h, dtype=np.float32)
    amax = np.abs(h32).max(axis=1)
    s = (amax / np.float32(448.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = (h32 / safe[:, None]).astype(np.float32)
    codes = e4m3_encode(q.astype(np.float64))
    codes[s == 0] = 0
    return codes, s.astype(np.float64)


def rmsnorm(x, eps: float = 1e-6):
    """x / sqrt(mean(x^2) + eps) over the last axis, gain 1 (reading R5)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


# =========================================================================== model

class OracleModel:
    """fp64 copies of the stored weights plus the rounding rule of the workload."""

    def __init__(self, inp: dict):
        cfg = inp["cfg"]
        self.cfg = cfg
        self.bf16 = cfg.dtype == "bf16"
        dec = decode_bf16 if self.bf16 else (lambda a: np.asarray(a, dtype=np.float64))
        self.E = dec(inp["E"])
        self.Wq = dec(inp["Wq"])
        self.Wk = dec(inp["Wk"])
        self.Wv = dec(inp["Wv"])
        self.Wo = dec(inp["Wo"])
        self.act8 = cfg.head == "fp8a8"
        if cfg.head in ("fp8", "fp8a8"):
            self.W = decode_e4m3(inp["W"])
            self.W_scale = np.asarray(inp["W_scale"], dtype=np.float64)
        else:
            self.W = dec(inp["W"])
            self.W_scale = None
        self.Hq, self.Hkv, self.hd = cfg.Hq, cfg.Hkv, cfg.hd
        self.scale = 1.0 / np.sqrt(cfg.hd)

    def rnd(self, x):
        return round_bf16(x) if self.bf16 else np.asarray(x, dtype=np.float64)


def node_layer(model: OracleModel, tokens):
    """Input block for a set of tokens (R5, R6).

    x = E[token]; a = RMSNorm(x) (stored: rounded); q, k, v = a Wq^T, a Wk^T, a Wv^T
    (stored: rounded).  Returns x [n, d], q [n, Hq, hd], k, v [n, Hkv, hd].
    """
    x = model.E[np.asarray(tokens)]
    a = model.rnd(rmsnorm(x))
    n = x.shape[0]
    q = model.rnd(a @ model.Wq.T).reshape(n, model.Hq, model.hd)
    k = model.rnd(a @ model.Wk.T).reshape(n, model.Hkv, model.hd)
    v = model.rnd(a @ model.Wv.T).reshape(n, model.Hkv, model.hd)
    return x, q, k, v


def doc_kv_from_tokens(model: OracleModel, doc_tokens):
    """Document keys/values of a token-id document: the node_layer k and v of each token."""
    _, _, k, v = node_layer(model, doc_tokens)
    return k, v


def tree_attention(qn, kn, vn, trie: Trie, Kd, Vd, doc_offsets, scale, docs=None, rows=None):
    """Ancestor-masked tree attention ([CT] 3.2 custom attention kernel; R4, R5).

    For document b, query row r (an internal node u) and query head h, the keys are
    the document's keys K_d[b, 0..L_b-1] followed by the keys of the nodes on the
    root-to-u path (u included); scores q.k * scale, softmax, weighted sum of values.
    Returns O[len(docs), len(rows), Hq, hd] in fp64 (unrounded).
    """
    Hq, Hkv = qn.shape[1], kn.shape[1]
    group = Hq // Hkv
    kv_of_head = np.arange(Hq) // group
    docs = range(len(doc_offsets) - 1) if docs is None else docs
    rows = range(trie.n_int) if rows is None else rows
    out = np.zeros((len(docs), len(rows), Hq, qn.shape[2]))
    for bi, b in enumerate(docs):
        Kb = np.asarray(Kd[doc_offsets[b]:doc_offsets[b + 1]], dtype=np.float64)
        Vb = np.asarray(Vd[doc_offsets[b]:doc_offsets[b + 1]], dtype=np.float64)
        for ri, r in enumerate(rows):
            path = _path_rows(trie, r)
            keys = np.concatenate([Kb, kn[path]], axis=0)[:, kv_of_head, :]   # [nk, Hq, hd]
            vals = np.concatenate([Vb, vn[path]], axis=0)[:, kv_of_head, :]
            s = np.einsum("hd,khd->hk", qn[r], keys) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[bi, ri] = np.einsum("hk,khd->hd", p, vals)
    return out


def hidden_states(model: OracleModel, x_nodes, O):
    """y = x + concat_h(O_h) Wo^T (not rounded); h = RMSNorm(y) (stored: rounded).

    O: [..., Hq, hd] already rounded to its storage type; x_nodes broadcasts over
    the leading document axis.
    """
    Of = O.reshape(O.shape[:-2] + (-1,))
    y = x_nodes + Of @ model.Wo.T
    return model.rnd(rmsnorm(y))


def head_logits_at(model: OracleModel, h, cols=None):
    """Logits h W^T for all vocabulary rows (or the listed ones); fp8 heads scale
    each dot product by the row's scale (R7); a W8A8 head first quantizes each
    hidden row to E4M3 with its own scale (R12)."""
    W = model.W if cols is None else model.W[cols]
    if getattr(model, "act8", False):
        codes, sh = quantize_rows_e4m3(h)
        z = (decode_e4m3(codes) @ W.T) * sh[:, None]
    else:
        z = h @ W.T
    if model.W_scale is not None:
        z = z * (model.W_scale if cols is None else model.W_scale[cols])
    return z


def lm_head_lse(model: OracleModel, h, chunk: int = 512):
    """Full-vocabulary log-sum-exp per hidden state ([CT] 4.1: all vocab rows are
    needed to turn scores into probabilities).  h: [R, d] -> lse [R]."""
    h = np.asarray(h, dtype=np.float64)
    lse = np.empty(h.shape[0])
    for r0 in range(0, h.shape[0], chunk):
        z = head_logits_at(model, h[r0:r0 + chunk])
        m = z.max(axis=1)
        lse[r0:r0 + chunk] = m + np.log(np.exp(z - m[:, None]).sum(axis=1))
    return lse


def edge_logprobs(model: OracleModel, trie: Trie, h, lse):
    """Token log-probability of every trie edge, per document.

    h: [B, N_int, d], lse: [B, N_int].  For the edge parent(c) -> c,
    lp[b, c] = logit[b, qrow(parent c), token c] - lse[b, qrow(parent c)];
    lp[b, root] = 0.  Returns lp [B, N].
    """
    B = h.shape[0]
    lp = np.zeros((B, trie.n_nodes))
    for c in range(1, trie.n_nodes):
        r = trie.qrow[trie.parent[c]]
        z = head_logits_at(model, h[:, r, :], cols=[trie.token[c]])[:, 0]
        lp[:, c] = z - lse[:, r]
    return lp


def log1mexp(x):
    """log(1 - e^x) for x <= 0, split at -ln 2 (Maechler's log1mexp); -inf for x >= 0."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(x > -np.log(2.0), np.log(-np.expm1(np.minimum(x, 0.0))),
                       np.log1p(-np.exp(np.minimum(x, 0.0))))
    return np.where(x >= 0.0, -np.inf, out)


def path_log_likelihoods(trie: Trie, lp):
    """Per-label log score ([CT] 3.2; R1, R3).

    LL[b, m] = sum of lp over the path root -> label_node[m]; a label ending at an
    internal node adds log(1 - sum_{children c} e^{lp[b, c]}) -- the probability
    of not continuing with any child.  lp: [B, N] -> LL [B, M].
    """
    lp = np.asarray(lp, dtype=np.float64)
    B = lp.shape[0]
    LL = np.zeros((B, trie.n_labels))
    for m in range(trie.n_labels):
        u = int(trie.label_node[m])
        LL[:, m] = lp[:, _path_nodes(trie, u)].sum(axis=1)
        if trie.child_count[u] > 0:
            cs = np.arange(trie.child_begin[u], trie.child_begin[u] + trie.child_count[u])
            z = lp[:, cs]
            mx = z.max(axis=1)
            lse_c = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
            LL[:, m] += log1mexp(lse_c)
    return LL


def label_softmax(LL):
    """P(m) = score(m) / sum of scores ([CT] 3.2 normalisation), computed as a
    softmax of the log scores; label = argmax, lowest id on ties (R8)."""
    LL = np.asarray(LL, dtype=np.float64)
    mx = LL.max(axis=1, keepdims=True)
    e = np.exp(LL - mx)
    P = e / e.sum(axis=1, keepdims=True)
    return P, np.argmax(LL, axis=1).astype(np.int32)


# =========================================================================== whole path

def classify(inp: dict, docs=None, model: OracleModel | None = None, trie: Trie | None = None):
    """The whole trie_tree pass for the listed documents (all by default).

    Returns a dict with trie, node q/k/v, O (rounded), h, lse, lp, ll, prob, label.
    """
    model = model or OracleModel(inp)
    trie = trie or build_trie(inp["labels"], inp["root_token"], inp["cfg"].V)
    offs = inp["doc_offsets"]
    docs = list(range(len(offs) - 1)) if docs is None else list(docs)
    x, qn, kn, vn = node_layer(model, trie.token[trie.qnode])
    # keys/values of the listed documents only, back to back
    if inp["cfg"].doc_mode == "tokens":
        toks = np.concatenate([inp["doc_tokens"][offs[b]:offs[b + 1]] for b in docs])
        Kd, Vd = doc_kv_from_tokens(model, toks)
    else:
        dec = decode_bf16 if model.bf16 else (lambda a: np.asarray(a, dtype=np.float64))
        Kd = dec(np.concatenate([inp["Kd"][offs[b]:offs[b + 1]] for b in docs]))
        Vd = dec(np.concatenate([inp["Vd"][offs[b]:offs[b + 1]] for b in docs]))
    sub = np.zeros(len(docs) + 1, dtype=np.int64)
    sub[1:] = np.cumsum([offs[b + 1] - offs[b] for b in docs])
    O = model.rnd(tree_attention(qn, kn, vn, trie, Kd, Vd, sub, model.scale))
    h = hidden_states(model, x[None], O)
    B, n_int, d = h.shape
    lse = lm_head_lse(model, h.reshape(-1, d)).reshape(B, n_int)
    lp = edge_logprobs(model, trie, h, lse)
    ll = path_log_likelihoods(trie, lp)
    prob, label = label_softmax(ll)
    return dict(trie=trie, x=x, qn=qn, kn=kn, vn=vn, Kd=Kd, Vd=Vd, O=O, h=h, lse=lse, lp=lp,
                ll=ll, prob=prob, label=label, docs=docs)


def bruteforce_ll(inp: dict, doc: int, label_ids=None, model: OracleModel | None = None,
                  upto=None):
    """Score labels one at a time by running the whole sequence causally.

    The direct definition of [CT] 3.2: P(m) = prod_k P(x_k | prompt, x_<k).  For
    label m with tokens t_1..t_k the sequence is [root, t_1, ..., t_k]; position j
    attends to every document key and to sequence positions 0..j (a causal mask);
    log P(t_{j+1}) = logit_j[t_{j+1}] - logsumexp(logit_j).  When other labels
    continue label m, the log-probability of not taking any of their next tokens
    is added ([CT] 3.2 prefix rule).  No trie is built.

    `upto` [M] (optional) scores only the first upto[m] tokens of label m: the
    decision-word score of [CT] 3.2 with upto = decision_depths(...).  The prefix
    rule is applied only when the whole label is scored.
    """
    model = model or OracleModel(inp)
    labels = [list(map(int, l)) for l in inp["labels"]]
    root = int(inp["root_token"])
    offs = inp["doc_offsets"]
    if inp["cfg"].doc_mode == "tokens":
        Kb, Vb = doc_kv_from_tokens(model, inp["doc_tokens"][offs[doc]:offs[doc + 1]])
    else:
        dec = decode_bf16 if model.bf16 else (lambda a: np.asarray(a, dtype=np.float64))
        Kb = dec(inp["Kd"][offs[doc]:offs[doc + 1]])
        Vb = dec(inp["Vd"][offs[doc]:offs[doc + 1]])
    L = Kb.shape[0]
    group = model.Hq // model.Hkv
    label_ids = range(len(labels)) if label_ids is None else label_ids
    out = []
    for m in label_ids:
        k_m = len(labels[m]) if upto is None else int(upto[m])
        seq = [root] + labels[m][:k_m]
        n = len(seq)
        x, q, k, v = node_layer(model, seq)
        keys = np.concatenate([Kb, k], axis=0)            # [L + n, Hkv, hd]
        vals = np.concatenate([Vb, v], axis=0)
        allowed = np.zeros((n, L + n), dtype=bool)
        allowed[:, :L] = True
        for j in range(n):
            allowed[j, L:L + j + 1] = True
        O = np.zeros((n, model.Hq, model.hd))
        for h in range(model.Hq):
            g = h // group
            s = (q[:, h, :] @ keys[:, g, :].T) * model.scale
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            O[:, h, :] = p @ vals[:, g, :]
        hid = model.rnd(rmsnorm(x + model.rnd(O).reshape(n, -1) @ model.Wo.T))
        z = head_logits_at(model, hid)
        mx = z.max(axis=1)
        lse = mx + np.log(np.exp(z - mx[:, None]).sum(axis=1))
        ll = sum(z[j, seq[j + 1]] - lse[j] for j in range(n - 1))
        cont = [] if k_m < len(labels[m]) else \
            sorted({l[len(labels[m])] for l in labels
                    if len(l) > len(labels[m]) and l[:len(labels[m])] == labels[m]})
        if cont:
            pstop = 1.0 - np.exp(z[n - 1, cont] - lse[n - 1]).sum()
            ll += np.log(pstop) if pstop > 0 else -np.inf
        out.append(ll)
    return np.array(out)


class _Rows:
    """Row view of a compact array: row r of the full index space -> compact[idx[r]]."""

    def __init__(self, compact, idx, n_rows):
        self.compact, self.idx = compact, idx
        self.shape = (n_rows,) + compact.shape[1:]

    def __getitem__(self, r):
        if isinstance(r, (list, tuple, np.ndarray)):
            return self.compact[[self.idx[int(x)] for x in r]]
        return self.compact[self.idx[int(r)]]


def label_ll_on_paths(inp: dict, doc: int, label_ids, model: OracleModel | None = None,
                      trie: Trie | None = None):
    """LL of the listed labels for one document, computed from the query rows on
    their paths only (the same steps as `classify`, restricted to those rows).

    Lets a large trie be checked on sampled labels without scoring every row.
    """
    model = model or OracleModel(inp)
    trie = trie or build_trie(inp["labels"], inp["root_token"], inp["cfg"].V)
    need_rows, need_edges = set(), set()
    for m in label_ids:
        u = int(trie.label_node[m])
        v = u
        while v > 0:
            need_edges.add(v)
            need_rows.add(int(trie.qrow[trie.parent[v]]))
            v = int(trie.parent[v])
        if trie.child_count[u] > 0:
            need_rows.add(int(trie.qrow[u]))
            need_edges.update(range(trie.child_begin[u], trie.child_begin[u] + trie.child_count[u]))
    rows = sorted(need_rows)
    idx = {r: i for i, r in enumerate(rows)}
    x, q, k, v = node_layer(model, trie.token[trie.qnode[rows]])
    offs = inp["doc_offsets"]
    if inp["cfg"].doc_mode == "tokens":
        Kd, Vd = doc_kv_from_tokens(model, inp["doc_tokens"])
    else:
        Kd = decode_bf16(inp["Kd"][offs[doc]:offs[doc + 1]]) if model.bf16 else \
            np.asarray(inp["Kd"][offs[doc]:offs[doc + 1]], dtype=np.float64)
        Vd = decode_bf16(inp["Vd"][offs[doc]:offs[doc + 1]]) if model.bf16 else \
            np.asarray(inp["Vd"][offs[doc]:offs[doc + 1]], dtype=np.float64)
        offs = np.zeros(doc + 2, dtype=np.int64)   # only document `doc` is visited
        offs[doc + 1] = Kd.shape[0]
    n = trie.n_int
    O = model.rnd(tree_attention(_Rows(q, idx, n), _Rows(k, idx, n), _Rows(v, idx, n), trie, Kd, Vd,
                                 offs, model.scale, docs=[doc], rows=rows))
    h = hidden_states(model, x[None], O)[0]
    lse = lm_head_lse(model, h)
    lp = np.zeros((1, trie.n_nodes))
    for c in need_edges:
        i = idx[int(trie.qrow[trie.parent[c]])]
        lp[0, c] = head_logits_at(model, h[i:i + 1], cols=[trie.token[c]])[0, 0] - lse[i]
    with np.errstate(all="ignore"):
        ll = path_log_likelihoods(trie, lp)[0]
    return ll[list(label_ids)], dict(rows=rows, lse=lse, h=h)


# =========================================================================== decision words ([CT] 3.2)

def decision_depths(labels, word_cont):
    """d_m for every label: the number of its tokens the decision-word form scores.

    [CT] 3.2: a label is scored up to the last token of the word in which it leaves
    every other label.  Count, for every token prefix, how many labels start with
    it.  Label m leaves the others at the first k whose prefix of length k is
    counted once (only m has it).  The word holding token k runs on while the
    next token carries the continuation flag (word_cont[t] != 0), so d_m is k
    plus that run.  When no prefix of m is its own (m is the start of another
    label), d_m is the whole length (reading R9).  Duplicate labels are an error.
    """
    labels = [list(map(int, l)) for l in labels]
    if len({tuple(l) for l in labels}) != len(labels):
        raise TrieError(TCS_EDUPLICATE, "two labels are equal")
    count: dict = {}
    for lab in labels:
        for k in range(1, len(lab) + 1):
            count[tuple(lab[:k])] = count.get(tuple(lab[:k]), 0) + 1
    out = np.zeros(len(labels), dtype=np.int64)
    for m, lab in enumerate(labels):
        n = len(lab)
        k = n
        for j in range(1, n + 1):
            if count[tuple(lab[:j])] == 1:
                k = j
                break
        while k < n and word_cont[lab[k]]:
            k += 1
        out[m] = k
    return out


def truncate_labels(labels, depths):
    """Label m cut to its first depths[m] tokens."""
    return [list(map(int, l[:int(d)])) for l, d in zip(labels, depths)]


# =========================================================================== letters ([CT] 3.3)

def letters_classify(inp: dict, letters, docs=None, model: OracleModel | None = None):
    """letters: one answer position (the root, ANSWER:) per document; the logits of
    the M letter tokens are read there and rescaled over the letters.

    [CT] 3.3: P_hat(m) = P(letter_m) / sum_m' P(letter_m'); the vocabulary
    normaliser of P cancels, so only the M letter rows of the head are used
    ([CT] 4.1, V_out = M).  Returns dict(z [B, M] letter logits, prob, label).
    """
    model = model or OracleModel(inp)
    letters = [int(t) for t in letters]
    root = int(inp["root_token"])
    offs = inp["doc_offsets"]
    docs = list(range(len(offs) - 1)) if docs is None else list(docs)
    x, q, k, v = node_layer(model, [root])
    group = model.Hq // model.Hkv
    z = np.zeros((len(docs), len(letters)))
    for i, b in enumerate(docs):
        if inp["cfg"].doc_mode == "tokens":
            Kb, Vb = doc_kv_from_tokens(model, inp["doc_tokens"][offs[b]:offs[b + 1]])
        else:
            dec = decode_bf16 if model.bf16 else (lambda a: np.asarray(a, dtype=np.float64))
            Kb, Vb = dec(inp["Kd"][offs[b]:offs[b + 1]]), dec(inp["Vd"][offs[b]:offs[b + 1]])
        keys = np.concatenate([Kb, k], axis=0)      # the document, then the answer position
        vals = np.concatenate([Vb, v], axis=0)
        O = np.zeros((model.Hq, model.hd))
        for h in range(model.Hq):
            s = keys[:, h // group, :] @ q[0, h, :] * model.scale
            p = np.exp(s - s.max())
            O[h] = (p / p.sum()) @ vals[:, h // group, :]
        hid = hidden_states(model, x[None], model.rnd(O)[None, None])[0, 0]
        z[i] = head_logits_at(model, hid[None], cols=letters)[0]
    prob, label = label_softmax(z)
    return dict(z=z, prob=prob, label=label, docs=docs)


# =========================================================================== trie_decode ([CT] 3.1)

def greedy_walk(labels, choose):
    """Walk the label set the way trie_decode generates ([CT] 3.1).

    The state is the token prefix generated so far (empty = the ANSWER: root).
    While more than one label starts with the prefix: if those labels agree on the
    next token, take it with no model run; else ask `choose(prefix, tokens)` for
    one of the distinct next tokens (a model run).  A label equal to the prefix
    while longer ones remain is never the answer (no stop token, [CT] note 2).
    Returns (label id, number of `choose` calls).
    """
    labels = [tuple(map(int, l)) for l in labels]
    prefix, runs = (), 0
    while True:
        remaining = [m for m, l in enumerate(labels) if l[:len(prefix)] == prefix]
        if len(remaining) == 1:
            return remaining[0], runs
        nxt = sorted({labels[m][len(prefix)] for m in remaining if len(labels[m]) > len(prefix)})
        if len(nxt) == 1:
            prefix += (nxt[0],)
            continue
        runs += 1
        prefix += (int(choose(prefix, nxt)),)


def _sequence_last_hidden(model: OracleModel, Kb, Vb, seq):
    """Hidden state at the last position of the token sequence `seq` placed after
    the document: every position attends to the document and causally to the
    sequence (R4, R5)."""
    n = len(seq)
    x, q, k, v = node_layer(model, seq)
    keys = np.concatenate([Kb, k], axis=0)
    vals = np.concatenate([Vb, v], axis=0)
    L = Kb.shape[0]
    group = model.Hq // model.Hkv
    O = np.zeros((model.Hq, model.hd))
    for h in range(model.Hq):
        s = keys[:L + n, h // group, :] @ q[n - 1, h, :] * model.scale
        p = np.exp(s - s.max())
        O[h] = (p / p.sum()) @ vals[:L + n, h // group, :]
    return hidden_states(model, x[n - 1][None], model.rnd(O)[None])[0]


def trie_decode(inp: dict, docs=None, model: OracleModel | None = None):
    """trie_decode for the listed documents ([CT] 3.1): at each branching point the
    model runs on [root, prefix] and the next token is the candidate with the
    highest logit (lowest token id on ties, R11); the vocabulary normaliser is the
    same for all candidates, so logits decide.

    Returns dict(label [B], runs [B] model runs per document, gap [B]: the smallest
    difference between the two best candidate logits over the document's runs).
    """
    model = model or OracleModel(inp)
    root = int(inp["root_token"])
    offs = inp["doc_offsets"]
    docs = list(range(len(offs) - 1)) if docs is None else list(docs)
    labels, runs, gaps = [], [], []
    for b in docs:
        if inp["cfg"].doc_mode == "tokens":
            Kb, Vb = doc_kv_from_tokens(model, inp["doc_tokens"][offs[b]:offs[b + 1]])
        else:
            dec = decode_bf16 if model.bf16 else (lambda a: np.asarray(a, dtype=np.float64))
            Kb, Vb = dec(inp["Kd"][offs[b]:offs[b + 1]]), dec(inp["Vd"][offs[b]:offs[b + 1]])
        gap = [np.inf]

        def choose(prefix, cands):
            hid = _sequence_last_hidden(model, Kb, Vb, [root] + list(prefix))
            z = head_logits_at(model, hid[None], cols=cands)[0]
            srt = np.sort(z)
            gap[0] = min(gap[0], srt[-1] - srt[-2])
            return cands[int(np.argmax(z))]

        m, r = greedy_walk(inp["labels"], choose)
        labels.append(m)
        runs.append(r)
        gaps.append(gap[0])
    return dict(label=np.array(labels, dtype=np.int32), runs=np.array(runs, dtype=np.int32),
                gap=np.array(gaps), docs=docs)
