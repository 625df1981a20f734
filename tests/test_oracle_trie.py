"""Pins of the oracle's trie builder (CPU only).

What fixes the trie independently of the builder:
  * the running example of "To Classify, Try a Trie Tree" (sections 3.1-3.2): 10
    labels, root with 7 children, 3 nodes with more than one child, 8 nodes with
    children, 18 nodes, maximum depth 4;
  * Proposition 1 of "Trie Automata for Constrained Decoding over Large Finite
    Sets": the trie is the minimal automaton, one state per distinct non-empty
    prefix plus the root;
  * the canonical numbering, checked against a brute-force sort of all prefixes.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
from synth import config, make_inputs


def prefixes_of(labels):
    ps = set()
    for l in labels:
        for k in range(1, len(l) + 1):
            ps.add(tuple(l[:k]))
    return ps


def node_paths(trie):
    paths = []
    for u in range(trie.n_nodes):
        p = []
        while u > 0:
            p.append(int(trie.token[u]))
            u = int(trie.parent[u])
        paths.append(tuple(p[::-1]))
    return paths


def test_running_example_counts():
    inp = make_inputs(config(1), weights=False)
    t = O.build_trie(inp["labels"], inp["root_token"], 1000)
    assert t.n_labels == 10
    assert t.n_nodes == 18
    assert t.n_int == 8                       # nodes with children
    assert int((t.child_count > 1).sum()) == 3  # branching nodes: root, refund, shipping
    assert t.max_depth == 4
    assert t.child_count[0] == 7
    assert sorted(t.child_count[t.child_count > 1].tolist()) == [2, 3, 7]
    # trie_decode's expected requests per document b = (1/M) sum c_m = 1.5 (section 4.3)
    c = []
    for m in range(t.n_labels):
        u, n = int(t.label_node[m]), 0
        while u > 0:
            u = int(t.parent[u])
            n += int(t.child_count[u] > 1)
        c.append(n)
    assert np.mean(c) == 1.5


label_sets = st.lists(st.lists(st.integers(0, 5), min_size=1, max_size=6), min_size=1, max_size=25)


@settings(max_examples=300, deadline=None)
@given(label_sets)
def test_minimal_automaton_and_canonical_order(raw):
    labels, seen = [], set()
    for l in raw:
        if tuple(l) not in seen:
            seen.add(tuple(l))
            labels.append(l)
    t = O.build_trie(labels, 7, 8)
    pre = prefixes_of(labels)
    assert t.n_nodes == len(pre) + 1                          # Proposition 1
    # canonical ids: rank of (depth, token path) over all prefixes; root first
    expect = [()] + sorted(pre, key=lambda p: (len(p), p))
    assert node_paths(t) == expect
    # children contiguous and ascending; levels contiguous
    for u in range(t.n_nodes):
        kids = [c for c in range(t.n_nodes) if t.parent[c] == u]
        assert t.child_count[u] == len(kids)
        if kids:
            assert kids == list(range(t.child_begin[u], t.child_begin[u] + len(kids)))
            assert [t.token[c] for c in kids] == sorted(t.token[c] for c in kids)
        else:
            assert t.child_begin[u] == 0
    for dd in range(t.max_depth + 1):
        lv = np.nonzero(t.depth == dd)[0]
        assert lv.tolist() == list(range(t.level_offsets[dd], t.level_offsets[dd + 1]))
    assert t.level_offsets[-1] == t.n_nodes
    # labels end where their path ends, in input order
    paths = node_paths(t)
    for m, l in enumerate(labels):
        assert paths[t.label_node[m]] == tuple(l)
        assert t.node_label[t.label_node[m]] == m
    assert (t.node_label >= 0).sum() == len(labels)
    # query rows: internal nodes in id order
    internal = [u for u in range(t.n_nodes) if t.child_count[u] > 0]
    assert t.qnode.tolist() == internal
    for r, u in enumerate(internal):
        assert t.qrow[u] == r
        assert t.qparent[r] == (t.qrow[t.parent[u]] if u > 0 else -1)
    # edges: every non-root node once, sorted by (token, parent row)
    assert sorted(t.e_child.tolist()) == list(range(1, t.n_nodes))
    keys = list(zip(t.e_tok.tolist(), t.e_qrow.tolist()))
    assert keys == sorted(keys)
    for tk, q, c in zip(t.e_tok, t.e_qrow, t.e_child):
        assert t.token[c] == tk and t.qrow[t.parent[c]] == q


def test_errors():
    with pytest.raises(O.TrieError) as e:
        O.build_trie([[1, 2], []], 0, 10)
    assert e.value.code == O.TCS_EINVAL
    with pytest.raises(O.TrieError) as e:
        O.build_trie([[1, 2], [1, 10]], 0, 10)
    assert e.value.code == O.TCS_EINVAL
    with pytest.raises(O.TrieError) as e:
        O.build_trie([[1, 2], [3], [1, 2]], 0, 10)
    assert e.value.code == O.TCS_EDUPLICATE
    with pytest.raises(O.TrieError) as e:
        O.build_trie([], 0, 10)
    assert e.value.code == O.TCS_EINVAL
    with pytest.raises(O.TrieError) as e:
        O.build_trie([[1]], 10, 10)
    assert e.value.code == O.TCS_EINVAL


def test_prefix_label_node_is_internal():
    t = O.build_trie([[4], [4, 2], [4, 3]], 0, 8)
    u = t.label_node[0]
    assert t.child_count[u] == 2 and t.qrow[u] >= 0


@pytest.mark.parametrize("cid,nlo,nhi", [(3, 2500, 4500), (4, 18000, 26000)])
def test_zipf_label_sets_are_prefix_free_and_sized(cid, nlo, nhi):
    inp = make_inputs(config(cid), weights=False)
    labels = inp["labels"]
    t = O.build_trie(labels, inp["root_token"], config(cid).V)
    assert nlo <= t.n_nodes <= nhi
    # prefix-free: every label ends at a leaf
    assert np.all(t.child_count[t.label_node] == 0)
    assert t.n_nodes == len(prefixes_of(labels)) + 1
