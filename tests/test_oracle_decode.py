"""Pins of the oracle's trie_decode ("To Classify, Try a Trie Tree", section 3.1,
section 4.3 and note 2): the branching nodes and requests per document the page
gives for the running example, the prefix-label rule, and agreement with greedy
choices made from the trie pass's own edge log-probabilities."""
import json
import os

import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _words(g, key="labels"):
    words = sorted({w for lab in g[key] for w in lab} | {"ANSWER:"})
    tok = {w: i for i, w in enumerate(words)}
    return tok, [[tok[w] for w in lab] for lab in g[key]]


def test_running_example_requests_per_document():
    g = json.load(open(os.path.join(GOLD, "trie_decode_requests.json")))
    tok, labels = _words(g)
    runs, seen = [], set()
    for m in range(len(labels)):
        def follow(prefix, cands, m=m):
            seen.add(prefix[-1] if prefix else tok["ANSWER:"])
            return labels[m][len(prefix)]
        got, r = O.greedy_walk(labels, follow)
        assert got == m
        runs.append(r)
    p = g["printed"]
    assert sorted(seen) == sorted(tok[w] for w in p["branching_nodes"])
    assert runs.count(1) == p["labels_decided_at_answer"]
    assert runs.count(2) == p["labels_needing_a_second_step"]
    assert np.mean(runs) == p["requests_per_document"]


def test_prefix_label_is_never_returned():
    g = json.load(open(os.path.join(GOLD, "trie_decode_requests.json")))
    ex = g["printed"]["prefix_example"]
    tok, labels = _words(ex)
    never = labels.index([tok[ex["never_returned"]]])
    # whatever the model prefers, the walk ends at another label
    for pick in (min, max):
        got, runs = O.greedy_walk(labels, lambda prefix, cands: pick(cands))
        assert got != never
    # a chain with no branching point needs no model run
    assert O.greedy_walk([[1, 2, 3]], lambda p, c: 1 / 0) == (0, 0)
    assert O.greedy_walk([[1, 2, 3], [1, 2, 3, 4]], lambda p, c: 1 / 0) == (1, 0)


@pytest.mark.parametrize("cfg", [
    config(1),
    config(1, trie=("explicit", [[3], [3, 4], [3, 4, 5], [3, 6], [9, 9, 9], [9, 9], [1]])),
    config(2, V=600, d=64, Hq=4, Hkv=2, hd=32, B=4, L=20, trie=("zipf", 25, 2, 6, 1.2)),
])
def test_decode_agrees_with_trie_pass_choices(cfg):
    """At every branching point the decode picks the child with the largest edge
    log-probability of the trie pass (tree attention + full log-sum-exp), which
    shares the normaliser across siblings."""
    inp = make_inputs(cfg, seed=11)
    dec = O.trie_decode(inp)
    tri = O.classify(inp)
    trie = tri["trie"]
    for i, b in enumerate(dec["docs"]):
        def choose(prefix, cands):
            u = 0
            for t in prefix:
                u = next(c for c in range(trie.child_begin[u], trie.child_begin[u] + trie.child_count[u])
                         if trie.token[c] == t)
            kids = {int(trie.token[c]): c for c in range(trie.child_begin[u],
                                                        trie.child_begin[u] + trie.child_count[u])}
            assert sorted(kids) == list(cands)
            lp = [tri["lp"][b, kids[t]] for t in cands]
            return cands[int(np.argmax(lp))]
        m, r = O.greedy_walk(inp["labels"], choose)
        assert (m, r) == (dec["label"][i], dec["runs"][i])


def test_one_token_labels_decode_like_letters():
    cfg = config(1, trie=("zipf", 20, 1, 1, 1.0))
    inp = make_inputs(cfg, seed=3)
    dec = O.trie_decode(inp)
    one = dict(inp, letters=np.array([l[0] for l in inp["labels"]], dtype=np.int32))
    let = O.letters_classify(one, one["letters"])
    np.testing.assert_array_equal(dec["label"], let["label"])
    assert (dec["runs"] == 1).all()
