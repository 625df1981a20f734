"""Pins of the oracle's scoring: the worked example, the prefix rule, the
invariants the pages state, and brute-force per-label sequence scoring."""
import json
import os

import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    p = g["token_probabilities"]
    # tokens: refund = [10, 11], praise = [20]
    trie = O.build_trie([[10, 11], [20]], 0, 32)
    lp = np.zeros((1, trie.n_nodes))
    for c in range(1, trie.n_nodes):
        tok = trie.token[c]
        lp[0, c] = np.log({10: p["refund_tok1"], 11: p["refund_tok2_given_tok1"], 20: p["praise_tok"]}[tok])
    ll = O.path_log_likelihoods(trie, lp)
    np.testing.assert_allclose(np.exp(ll[0, 0]), g["printed"]["refund_sequence_probability"], rtol=1e-14)
    prob, label = O.label_softmax(ll)
    assert ["refund", "praise"][label[0]] == g["printed"]["trie_tree_selects"]
    s = g["printed"]["refund_sequence_probability"] + p["praise_tok"]
    np.testing.assert_allclose(prob[0], [0.48 / s, 0.3 / s], rtol=1e-14)
    np.testing.assert_allclose(prob[0], [0.6153846153846154, 0.38461538461538464], rtol=1e-14)


def test_prefix_rule():
    g = json.load(open(os.path.join(GOLD, "prefix_rule.json")))
    c = g["case"]
    trie = O.build_trie([[5], [5, 9]], 0, 16)      # "refund", "refund request"
    lp = np.zeros((1, trie.n_nodes))
    lp[0, trie.label_node[0]] = np.log(c["p_refund"])
    lp[0, trie.label_node[1]] = np.log(c["p_request_given_refund"])
    ll = O.path_log_likelihoods(trie, lp)
    np.testing.assert_allclose(np.exp(ll[0]), [g["expected_scores"]["refund"],
                                               g["expected_scores"]["refund request"]], rtol=1e-14)


def test_prefix_rule_several_children():
    trie = O.build_trie([[5], [5, 9], [5, 8, 1]], 0, 16)
    u = trie.label_node[0]
    kids = list(range(trie.child_begin[u], trie.child_begin[u] + trie.child_count[u]))
    lp = np.zeros((1, trie.n_nodes))
    lp[0, u] = np.log(0.5)
    lp[0, kids] = np.log([0.2, 0.3])
    ll = O.path_log_likelihoods(trie, lp)
    np.testing.assert_allclose(np.exp(ll[0, 0]), 0.5 * (1 - 0.5), rtol=1e-14)


def test_invariants_random():
    rng = np.random.default_rng(0)
    labels = [[1, 2, 3], [1, 2, 4], [1, 5], [6], [6, 7], [8, 9, 10, 11]]
    trie = O.build_trie(labels, 0, 16)
    # lp from a proper next-token distribution at every internal node
    lp = np.zeros((50, trie.n_nodes))
    for r in range(trie.n_int):
        u = trie.qnode[r]
        kids = np.arange(trie.child_begin[u], trie.child_begin[u] + trie.child_count[u])
        w = rng.random((50, len(kids) + 3))
        w /= w.sum(axis=1, keepdims=True)
        lp[:, kids] = np.log(w[:, :len(kids)])
    ll = O.path_log_likelihoods(trie, lp)
    prob, label = O.label_softmax(ll)
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, rtol=1e-14)
    assert np.all((label >= 0) & (label < len(labels)))
    assert np.all(prob[np.arange(50), label] == prob.max(axis=1))
    # an edge shared by all labels leaves the probabilities unchanged
    shared = O.build_trie([[3] + l for l in labels], 0, 16)
    lp2 = np.zeros((50, shared.n_nodes))
    lp2[:, 1] = np.log(0.37)
    for c in range(2, shared.n_nodes):
        path = []
        u = c
        while u > 1:
            path.append(int(shared.token[u]))
            u = int(shared.parent[u])
        tpath = tuple(path[::-1])
        c0 = next(v for v in range(1, trie.n_nodes) if _path(trie, v) == tpath)
        lp2[:, c] = lp[:, c0]
    ll2 = O.path_log_likelihoods(shared, lp2)
    p2, l2 = O.label_softmax(ll2)
    np.testing.assert_allclose(ll2, ll + np.log(0.37), rtol=1e-13)
    np.testing.assert_allclose(p2, prob, rtol=1e-12)
    assert np.array_equal(l2, label)


def _path(trie, u):
    p = []
    while u > 0:
        p.append(int(trie.token[u]))
        u = int(trie.parent[u])
    return tuple(p[::-1])


def test_single_label_has_probability_one():
    trie = O.build_trie([[4, 2, 7]], 0, 8)
    lp = np.log(np.random.default_rng(1).random((5, trie.n_nodes)))
    lp[:, 0] = 0
    prob, label = O.label_softmax(O.path_log_likelihoods(trie, lp))
    assert np.all(prob == 1.0) and np.all(label == 0)


def test_argmax_ties_take_lowest_id():
    prob, label = O.label_softmax(np.array([[-1.0, -0.5, -0.5, -3.0]]))
    assert label[0] == 1


LABEL_SETS = [
    [[3, 4], [3, 5, 6], [7], [8, 9]],
    [[3], [3, 4], [3, 4, 5], [3, 6], [9, 9, 9]],          # prefix labels, nested
    [[11, 2, 3, 4, 5], [11, 2, 3, 4, 6], [11, 7], [12]],  # single-child chains
]


@pytest.mark.parametrize("dtype,head", [("f32", "same"), ("bf16", "same"), ("bf16", "fp8")])
@pytest.mark.parametrize("li", range(len(LABEL_SETS)))
@pytest.mark.parametrize("Hq,Hkv", [(2, 1), (4, 2)])
def test_bruteforce_equals_tree(dtype, head, li, Hq, Hkv):
    """Per-label causal scoring of each full sequence equals the trie pass."""
    labels = LABEL_SETS[li]
    cfg = config(1, V=40, d=32, Hq=Hq, Hkv=Hkv, hd=16, dtype=dtype, head=head,
                 doc_lens=(3, 7), trie=("explicit", labels), std=0.5)
    inp = make_inputs(cfg, seed=100 + li)
    res = O.classify(inp)
    for b in range(2):
        bf = O.bruteforce_ll(inp, b)
        np.testing.assert_allclose(res["ll"][b], bf, rtol=0, atol=1e-10)


def test_bruteforce_equals_tree_kv_docs():
    cfg = config(2, V=64, d=64, Hq=4, Hkv=2, hd=32, doc_lens=(4, 1, 6),
                 trie=("explicit", LABEL_SETS[1]), std=0.3)
    inp = make_inputs(cfg, seed=7)
    res = O.classify(inp)
    for b in range(3):
        np.testing.assert_allclose(res["ll"][b], O.bruteforce_ll(inp, b), rtol=0, atol=1e-10)


def test_classify_running_example_tiny():
    inp = make_inputs(config(1))
    res = O.classify(inp)
    assert res["ll"].shape == (4, 10)
    np.testing.assert_allclose(res["prob"].sum(axis=1), 1.0, rtol=1e-13)
    for b in range(4):
        np.testing.assert_allclose(res["ll"][b], O.bruteforce_ll(inp, b), rtol=0, atol=1e-10)
