"""Pins of the decision-word form of trie_tree in the oracle ("To Classify, Try a
Trie Tree", section 3.2): the depths and model runs the page gives for the
running example, hand-worked cases, brute-force sequence scoring of the truncated
labels, and the invariants that follow from the definition."""
import json
import os

import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _running_words():
    g = json.load(open(os.path.join(GOLD, "decision_words.json")))
    words = sorted({w for lab in g["labels"] for w in lab} | {g["root"]})
    tok = {w: i for i, w in enumerate(words)}
    labels = [[tok[w] for w in lab] for lab in g["labels"]]
    cont = np.zeros(len(words), dtype=np.uint8)
    for w in g["continuation_tokens"]:
        cont[tok[w]] = 1
    return g, tok, labels, cont


def test_running_example_depths_and_model_runs():
    g, tok, labels, cont = _running_words()
    d = O.decision_depths(labels, cont)
    names = [" ".join(l).replace(" -", "-") for l in g["labels"]]
    for name, scored in g["printed"]["scored_tokens"].items():
        m = names.index(name)
        assert O.truncate_labels(labels, d)[m] == [tok[w] for w in scored], name
    full = O.build_trie(labels, tok[g["root"]], len(tok))
    assert full.n_int == g["printed"]["nodes_with_children_in_full_trie"]
    cut = O.build_trie(O.truncate_labels(labels, d), tok[g["root"]], len(tok))
    runs = sorted(int(cut.token[u]) for u in cut.qnode)
    assert runs == sorted(tok[w] for w in g["printed"]["model_runs_at"])


def test_synthetic_running_example_runs_four_nodes():
    inp = make_inputs(config(2), weights=False)
    d = O.decision_depths(inp["labels"], inp["word_cont"])
    assert list(d) == [1, 2, 2, 2, 2, 2, 1, 2, 1, 1]
    cut = O.build_trie(O.truncate_labels(inp["labels"], d), inp["root_token"], 151936)
    assert cut.n_int == 4


@pytest.mark.parametrize("labels,cont,expect", [
    # a label that is the start of another never leaves it: scored in full
    ([[5], [5, 9]], [], [1, 2]),
    # leaves at token 2, whose word runs on through the continuation token 3
    ([[1, 2, 3, 4], [1, 5, 6]], [3], [3, 2]),
    # a shared word start, then the labels part inside the word
    ([[1, 2, 3], [1, 2, 4]], [2], [3, 3]),
    # a continuation flag before the point of leaving does not move it
    ([[1, 2, 7, 8], [1, 3]], [2, 3], [2, 2]),
    # every token continues a word: each label is one word, scored in full
    ([[1, 2, 3], [1, 4], [6]], list(range(10)), [3, 2, 1]),
    # single-token labels are unchanged
    ([[1], [2], [3]], [1, 2, 3], [1, 1, 1]),
    # a prefix label inside a word: "refund" ends where "refund-request" goes on
    ([[1], [1, 2, 3], [1, 4]], [2], [1, 2, 2]),
])
def test_decision_depth_cases(labels, cont, expect):
    flags = np.zeros(10, dtype=np.uint8)
    flags[cont] = 1
    assert list(O.decision_depths(labels, flags)) == expect


def test_decision_depths_reject_duplicates():
    with pytest.raises(O.TrieError):
        O.decision_depths([[1, 2], [3], [1, 2]], np.zeros(5, dtype=np.uint8))


def _truncated(inp):
    d = O.decision_depths(inp["labels"], inp["word_cont"])
    cut = O.truncate_labels(inp["labels"], d)
    return d, O.build_trie(cut, inp["root_token"], inp["cfg"].V)


def test_truncated_trie_scoring_matches_bruteforce():
    """The trie pass over the cut labels gives the per-label sequence score of
    tokens 1..d_m computed without any trie."""
    inp = make_inputs(config(1))
    d, trie = _truncated(inp)
    res = O.classify(inp, trie=trie)
    for b in range(inp["cfg"].B):
        bf = O.bruteforce_ll(inp, b, upto=d)
        np.testing.assert_allclose(res["ll"][b], bf, rtol=1e-10, atol=1e-12)


def test_truncated_prefix_labels_match_bruteforce():
    """Prefix labels with the decision-word cut: the stop rule of the cut trie sees
    the same continuations as the full label set."""
    labels = [[3], [3, 7], [3, 7, 8, 9], [3, 11, 12], [20, 21, 22], [20, 21, 23, 24], [30]]
    inp = make_inputs(config(1, trie=("explicit", labels), B=2, L=24))
    flags = np.zeros(inp["cfg"].V, dtype=np.uint8)
    flags[[8, 12, 24]] = 1
    inp["word_cont"] = flags
    d, trie = _truncated(inp)
    assert list(d) == [1, 2, 3, 3, 3, 4, 1]
    res = O.classify(inp, trie=trie)
    for b in range(2):
        np.testing.assert_allclose(res["ll"][b], O.bruteforce_ll(inp, b, upto=d), rtol=1e-10,
                                   atol=1e-12)


def test_truncation_only_drops_nonpositive_terms():
    """Leaving out token log-probs (each <= 0) can only raise a non-prefix label's
    score; with every token a word continuation nothing is cut."""
    inp = make_inputs(config(1, trie=("zipf", 40, 2, 6, 1.2), B=2, L=16))
    d, trie = _truncated(inp)
    assert (d < np.array([len(l) for l in inp["labels"]])).any()
    full = O.classify(inp)
    cut = O.classify(inp, trie=trie)
    assert (cut["ll"] >= full["ll"] - 1e-12).all()
    same = make_inputs(config(1, trie=("zipf", 40, 2, 6, 1.2), B=2, L=16))
    same["word_cont"] = np.ones(same["cfg"].V, dtype=np.uint8)
    d1, trie1 = _truncated(same)
    assert list(d1) == [len(l) for l in same["labels"]]
    np.testing.assert_array_equal(O.classify(same, trie=trie1)["ll"], full["ll"])


def test_truncated_labels_are_distinct_and_keep_prefix_pairs():
    """The cut labels are pairwise distinct, and a cut label is the start of another
    cut label exactly when the uncut one was (the prefix rule is unchanged)."""
    for cid, kw in ((3, {}), (1, dict(trie=("zipf", 300, 1, 5, 1.0)))):
        inp = make_inputs(config(cid, **kw), weights=False)
        labels = inp["labels"]
        d = O.decision_depths(labels, inp["word_cont"])
        cut = O.truncate_labels(labels, d)
        assert len({tuple(c) for c in cut}) == len(cut)
        full_set = {tuple(l) for l in labels}
        cut_set = {tuple(c) for c in cut}
        for l, c in zip(labels, cut):
            was = any(tuple(l[:k]) in full_set for k in range(1, len(l)))
            now = any(tuple(c[:k]) in cut_set for k in range(1, len(c)))
            assert was == now
