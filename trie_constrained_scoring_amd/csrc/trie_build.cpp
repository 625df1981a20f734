// Host construction of the canonical token trie (tcs_trie_build).
//
// The label trie of "To Classify, Try a Trie Tree", section 3.1: each label is a
// path of tokens from the root (the ANSWER: token); labels that start alike share
// nodes.  Construction: insert every label into a hash map keyed by
// (parent, token), then renumber breadth-first with children in ascending token
// order, which ranks nodes by (depth, token path).
#include <algorithm>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "tcs_internal.h"

namespace {

struct Edge {
  int32_t parent;  // provisional id
  int32_t token;
  int32_t child;   // provisional id
};

// Shared argument checks of the label-set entry points (CSR labels over [0, V)).
int check_labels(const char* fn, const int32_t* label_offsets, const int32_t* label_tokens,
                 int32_t M, int32_t V) {
  using tcs::fail;
  if (!label_offsets) return fail(TCS_EINVAL, "%s: null label_offsets", fn);
  if (M < 1) return fail(TCS_EINVAL, "%s: need at least one label (M=%d)", fn, M);
  if (V < 1) return fail(TCS_EINVAL, "%s: vocabulary size %d", fn, V);
  if (label_offsets[0] != 0) return fail(TCS_EINVAL, "%s: label_offsets[0] must be 0", fn);
  for (int32_t m = 0; m < M; ++m) {
    if (label_offsets[m + 1] <= label_offsets[m])
      return fail(TCS_EINVAL, "%s: label %d is empty", fn, m);
  }
  const int64_t T = label_offsets[M];
  if (T > 0 && !label_tokens) return fail(TCS_EINVAL, "%s: null label_tokens", fn);
  for (int64_t i = 0; i < T; ++i) {
    if (label_tokens[i] < 0 || label_tokens[i] >= V)
      return fail(TCS_EINVAL, "%s: token %d at position %lld outside [0,%d)", fn,
                  label_tokens[i], (long long)i, V);
  }
  return TCS_OK;
}

inline uint64_t edge_key(int32_t node, int32_t token) {
  return (static_cast<uint64_t>(static_cast<uint32_t>(node)) << 32) |
         static_cast<uint32_t>(token);
}

}  // namespace

extern "C" int tcs_trie_build(const int32_t* label_offsets, const int32_t* label_tokens,
                              int32_t M, int32_t root_token, int32_t V, tcs_trie* out) {
  using tcs::fail;
  tcs::clear_error();
  if (!out) return fail(TCS_EINVAL, "trie_build: null pointer");
  if (int rc = check_labels("trie_build", label_offsets, label_tokens, M, V)) return rc;
  if (root_token < 0 || root_token >= V)
    return fail(TCS_EINVAL, "trie_build: root token %d outside [0,%d)", root_token, V);
  const int64_t T = label_offsets[M];

  // 1. insert: provisional ids in creation order, root = 0
  std::unordered_map<uint64_t, int32_t> child_of;
  child_of.reserve(static_cast<size_t>(T) * 2 + 1);
  std::vector<Edge> edges;
  edges.reserve(T);
  std::vector<int32_t> label_at(1, -1);  // label ending at provisional node
  std::vector<int32_t> label_node_prov(M);
  for (int32_t m = 0; m < M; ++m) {
    int32_t node = 0;
    for (int32_t i = label_offsets[m]; i < label_offsets[m + 1]; ++i) {
      const uint64_t key = edge_key(node, label_tokens[i]);
      auto it = child_of.find(key);
      if (it == child_of.end()) {
        const int32_t id = static_cast<int32_t>(label_at.size());
        child_of.emplace(key, id);
        edges.push_back({node, label_tokens[i], id});
        label_at.push_back(-1);
        node = id;
      } else {
        node = it->second;
      }
    }
    if (label_at[node] >= 0)
      return fail(TCS_EDUPLICATE, "trie_build: label %d duplicates label %d", m, label_at[node]);
    label_at[node] = m;
    label_node_prov[m] = node;
  }
  const int32_t N = static_cast<int32_t>(label_at.size());

  // 2. children of each provisional node, ascending token
  std::sort(edges.begin(), edges.end(), [](const Edge& a, const Edge& b) {
    return a.parent != b.parent ? a.parent < b.parent : a.token < b.token;
  });
  std::vector<int32_t> kid_begin(N + 1, 0);
  for (const Edge& e : edges) kid_begin[e.parent + 1]++;
  for (int32_t u = 0; u < N; ++u) kid_begin[u + 1] += kid_begin[u];

  // 3. breadth-first renumbering
  std::vector<int32_t> order;      // canonical id -> provisional id
  std::vector<int32_t> canon(N);   // provisional id -> canonical id
  std::vector<int32_t> depth_c;
  order.reserve(N);
  depth_c.reserve(N);
  order.push_back(0);
  depth_c.push_back(0);
  canon[0] = 0;
  for (size_t head = 0; head < order.size(); ++head) {
    const int32_t p = order[head];
    for (int32_t k = kid_begin[p]; k < kid_begin[p + 1]; ++k) {
      canon[edges[k].child] = static_cast<int32_t>(order.size());
      order.push_back(edges[k].child);
      depth_c.push_back(depth_c[head] + 1);
    }
  }
  const int32_t D = depth_c.back();
  int32_t n_int = 0;
  for (int32_t u = 0; u < N; ++u) n_int += kid_begin[u + 1] > kid_begin[u];

  out->n_nodes = N;
  out->n_int = n_int;
  out->n_labels = M;
  out->max_depth = D;
  if (out->cap_nodes < N || out->cap_levels < D + 2)
    return fail(TCS_ECAPACITY, "trie_build: needs %d nodes and %d levels (capacity %d / %d)", N,
                D + 2, out->cap_nodes, out->cap_levels);
  int32_t* arrs[] = {out->parent, out->token, out->depth, out->child_begin, out->child_count,
                     out->node_label, out->qrow, out->qnode, out->qparent, out->label_node,
                     out->level_offsets, out->e_tok, out->e_qrow, out->e_child};
  for (int32_t* a : arrs)
    if (!a) return fail(TCS_EINVAL, "trie_build: null output array");

  // provisional parent of each provisional node
  std::vector<int32_t> prov_parent(N, -1);
  std::vector<int32_t> prov_token(N, root_token);
  for (const Edge& e : edges) {
    prov_parent[e.child] = e.parent;
    prov_token[e.child] = e.token;
  }
  int32_t row = 0;
  for (int32_t c = 0; c < N; ++c) {
    const int32_t p = order[c];
    const int32_t nk = kid_begin[p + 1] - kid_begin[p];
    out->parent[c] = c == 0 ? -1 : canon[prov_parent[p]];
    out->token[c] = prov_token[p];
    out->depth[c] = depth_c[c];
    out->child_count[c] = nk;
    out->child_begin[c] = nk ? canon[edges[kid_begin[p]].child] : 0;
    out->node_label[c] = label_at[p];
    if (nk) {
      out->qrow[c] = row;
      out->qnode[row] = c;
      ++row;
    } else {
      out->qrow[c] = -1;
    }
  }
  for (int32_t r = 0; r < n_int; ++r) {
    const int32_t u = out->qnode[r];
    out->qparent[r] = u == 0 ? -1 : out->qrow[out->parent[u]];
  }
  for (int32_t m = 0; m < M; ++m) out->label_node[m] = canon[label_node_prov[m]];
  for (int32_t dd = 0, c = 0; dd <= D + 1; ++dd) {
    while (c < N && depth_c[c] < dd) ++c;
    out->level_offsets[dd] = c;
  }
  // edges sorted by (token, parent row)
  std::vector<int32_t> idx(N > 0 ? N - 1 : 0);
  for (int32_t i = 0; i + 1 < N; ++i) idx[i] = i + 1;
  std::sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) {
    const int32_t ta = out->token[a], tb = out->token[b];
    if (ta != tb) return ta < tb;
    return out->qrow[out->parent[a]] < out->qrow[out->parent[b]];
  });
  for (int32_t i = 0; i + 1 < N; ++i) {
    const int32_t c = idx[i];
    out->e_tok[i] = out->token[c];
    out->e_qrow[i] = out->qrow[out->parent[c]];
    out->e_child[i] = c;
  }
  // rows follow node order, so the rows of one depth are contiguous
  if (out->row_level_offsets) {
    for (int32_t dd = 0, r = 0; dd <= D + 1; ++dd) {
      while (r < n_int && depth_c[out->qnode[r]] < dd) ++r;
      out->row_level_offsets[dd] = r;
    }
  }
  if (out->label_row) {
    for (int32_t m = 0; m < M; ++m) {
      const int32_t u = out->label_node[m];
      out->label_row[m] = out->child_count[u] > 0 ? out->qrow[u] : out->qrow[out->parent[u]];
    }
  }
  // greedy-decoding tables: labels per subtree, bottom-up (children have larger ids)
  if (out->sub_label && out->dec_node) {
    std::vector<int32_t> count(N, 0);
    for (int32_t c = N - 1; c >= 0; --c) {
      count[c] += out->node_label[c] >= 0;
      int32_t one = out->node_label[c];
      for (int32_t k = 0; k < out->child_count[c]; ++k) {
        const int32_t ch = out->child_begin[c] + k;
        if (count[ch] > 0 && one < 0) one = out->sub_label[ch];
        count[c] += count[ch];
      }
      out->sub_label[c] = count[c] == 1 ? one : -1;
    }
    for (int32_t c = 0; c < N; ++c) {
      int32_t w = c;
      while (out->child_count[w] == 1 && out->sub_label[w] < 0) w = out->child_begin[w];
      out->dec_node[c] = w;
    }
    // model runs on the way to each label: the undecided nodes decoding stops at.  A
    // label that ends above such a node (the start of another label) is never
    // reached; its count stops there.
    int32_t most = 0;
    for (int32_t m = 0; m < M; ++m) {
      const int32_t lab = out->label_node[m];
      int32_t runs = 0;
      for (int32_t w = out->dec_node[0]; out->sub_label[w] < 0;) {
        if (out->depth[lab] <= out->depth[w]) break;
        int32_t v = lab;  // the child of w on the label's path
        while (out->depth[v] > out->depth[w] + 1) v = out->parent[v];
        if (out->parent[v] != w) break;
        ++runs;
        w = out->dec_node[v];
      }
      most = std::max(most, runs);
    }
    out->max_decode_steps = most;
    int32_t widest = 0;
    for (int32_t c = 0; c < N; ++c) widest = std::max(widest, out->child_count[c]);
    out->max_children = widest;
  }
  return TCS_OK;
}

// Decision-word cut of every label ("To Classify, Try a Trie Tree", section 3.2).
// One pass inserts the labels into a (node, token) map and counts, per node, the
// labels that pass through it; label m separates from the rest at the first node
// on its path that no other label passes, and its word then runs on over the continuation tokens.
extern "C" int tcs_decision_truncate(const int32_t* label_offsets, const int32_t* label_tokens,
                                     int32_t M, int32_t V, const uint8_t* word_cont,
                                     int32_t* out_offsets, int32_t* out_tokens, int32_t* depth) {
  using tcs::fail;
  tcs::clear_error();
  if (int rc = check_labels("decision_truncate", label_offsets, label_tokens, M, V)) return rc;
  if (!word_cont || !out_offsets || !out_tokens)
    return fail(TCS_EINVAL, "decision_truncate: null pointer");
  const int64_t T = label_offsets[M];

  std::unordered_map<uint64_t, int32_t> child_of;
  child_of.reserve(static_cast<size_t>(T) * 2 + 1);
  std::vector<int32_t> through(1, M);   // labels passing each node (root: all)
  std::vector<int32_t> ends(1, -1);     // label ending at each node
  std::vector<int32_t> path(T);         // node reached after each label token
  for (int32_t m = 0; m < M; ++m) {
    int32_t node = 0;
    for (int32_t i = label_offsets[m]; i < label_offsets[m + 1]; ++i) {
      auto ins = child_of.emplace(edge_key(node, label_tokens[i]),
                                  static_cast<int32_t>(through.size()));
      if (ins.second) {
        through.push_back(0);
        ends.push_back(-1);
      }
      node = ins.first->second;
      ++through[node];
      path[i] = node;
    }
    if (ends[node] >= 0)
      return fail(TCS_EDUPLICATE, "decision_truncate: label %d duplicates label %d", m,
                  ends[node]);
    ends[node] = m;
  }

  out_offsets[0] = 0;
  for (int32_t m = 0; m < M; ++m) {
    const int32_t b = label_offsets[m], n = label_offsets[m + 1] - b;
    int32_t k = n;  // a label that is the start of another keeps every token
    for (int32_t j = 0; j < n; ++j) {
      if (through[path[b + j]] == 1) {
        k = j + 1;
        break;
      }
    }
    while (k < n && word_cont[label_tokens[b + k]]) ++k;
    if (depth) depth[m] = k;
    std::memcpy(out_tokens + out_offsets[m], label_tokens + b, sizeof(int32_t) * k);
    out_offsets[m + 1] = out_offsets[m] + k;
  }
  return TCS_OK;
}
