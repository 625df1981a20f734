"""Parity of the decision-word form of trie_tree ("To Classify, Try a Trie Tree",
section 3.2: a label is scored through the last token of the word in which its
prefix stops being shared).  The library cuts the labels on the host (tcs_decision_truncate) and runs
the unchanged classify pass on the cut trie; the oracle cuts them from the
definition and scores the cut trie in fp64."""
import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, make_inputs
from tests.gpu_util import check_labels, golden_fingerprint, load_golden, say

pytestmark = pytest.mark.gpu


def cut_both(cfg, inp):
    """(library cut trie, oracle cut trie); the two cuts agree token for token."""
    offs, toks, depth = tcs.decision_truncate(inp["label_offsets"], inp["label_tokens"], cfg.V,
                                              inp["word_cont"])
    d = O.decision_depths(inp["labels"], inp["word_cont"])
    np.testing.assert_array_equal(depth, d)
    t = tcs.trie_build(offs, toks, inp["root_token"], cfg.V)
    o = O.build_trie(O.truncate_labels(inp["labels"], d), inp["root_token"], cfg.V)
    return t, o


def run_cut(cfg, inp, t):
    import torch
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    label, prob, ll = tcs.classify(model, td, docs, prepared=prep)
    torch.cuda.synchronize()
    out = label.cpu().numpy(), prob.cpu().numpy(), ll.cpu().numpy()
    del model, docs, prep
    torch.cuda.empty_cache()
    return out


SMALL = {
    "tiny-f32": (config(1), None),
    "tiny-f32-ragged": (config(1, doc_lens=(1, 32, 7, 0, 19)), None),
    "running-bf16-small": (config(2, V=3000, d=256, B=6, L=100, doc_lens=(100, 1, 257, 0, 64, 130)),
                           None),
    "zipf-bf16-small": (config(3, V=4096, d=128, Hq=8, Hkv=2, B=3, L=50,
                               trie=("zipf", 60, 2, 9, 1.2)), None),
    # prefix labels, a cut inside a word, a label that is one long word
    "prefix-words-bf16-small": (config(2, V=2000, d=128, Hq=4, Hkv=2, hd=64, B=5, L=40,
                                       trie=("explicit", [[3], [3, 7], [3, 7, 8, 9], [3, 11, 12],
                                                          [20, 21, 22], [20, 21, 23, 24], [30],
                                                          [40, 41, 42, 43, 44]])),
                                [8, 12, 24, 41, 42, 43, 44]),
    "fp8-small": (config(5, V=2500, d=192, Hq=4, Hkv=1, B=4, L=300), None),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decision_word_small_vs_oracle(dev, name):
    cfg, cont = SMALL[name]
    inp = make_inputs(cfg, seed=107)
    if cont is not None:
        inp["word_cont"] = np.zeros(cfg.V, dtype=np.uint8)
        inp["word_cont"][cont] = 1
    t, o_trie = cut_both(cfg, inp)
    label, prob, ll = run_cut(cfg, inp, t)
    o = O.classify(inp, trie=o_trie)
    check_labels(ll, prob, label, o["ll"], o["prob"], o["label"],
                 f"decision-word[{name}] rows {t.n_int}")


def test_decision_word_running_example_full_size(dev):
    """Running example at full size (B = 64, 512-token documents, Qwen3-4B shapes):
    the cut trie has the four rows the page names; sampled documents vs the oracle."""
    cfg = config(2)
    inp = make_inputs(cfg)
    t, o_trie = cut_both(cfg, inp)
    assert t.n_int == 4
    label, prob, ll = run_cut(cfg, inp, t)
    docs = [0, 1, cfg.B // 2, cfg.B - 1]
    o = O.classify(inp, docs=docs, trie=o_trie)
    check_labels(ll[docs], prob[docs], label[docs], o["ll"], o["prob"], o["label"],
                 f"decision-word[running example full, docs {docs}]")


def test_decision_word_max_label_set_full_size(dev):
    """255-label Zipf trie at full size (B = 32, 1024-token documents), decision-word
    form: every label's score, probability and the chosen label of the stored
    documents against the whole fp64 oracle pass on the oracle's own cut
    (tests/golden, written from oracle/ only); properties on every document."""
    g = load_golden("classify_max_label_set_255_decision_words.json")
    cfg = config(3)
    inp = make_inputs(cfg)
    assert golden_fingerprint(inp, g["docs"]) == g["fingerprint"], "inputs differ from the golden's"
    t, o_trie = cut_both(cfg, inp)
    assert (t.n_nodes, t.n_int) == (g["n_nodes"], g["n_int"])
    label, prob, ll = run_cut(cfg, inp, t)
    docs = g["docs"]
    o_ll = np.array(g["ll"], dtype=np.float64)
    o_prob, o_label = O.label_softmax(o_ll)
    assert o_label.tolist() == g["label"]
    check_labels(ll[docs], prob[docs], label[docs], o_ll, o_prob, o_label,
                 f"decision-word[config 3 full, rows {t.n_int}, every label of docs {docs}]")
    ll64 = ll.astype(np.float64)
    p_ref = np.exp(ll64 - ll64.max(axis=1, keepdims=True))
    p_ref /= p_ref.sum(axis=1, keepdims=True)
    assert np.abs(prob - p_ref).max() < 1e-4
    assert np.array_equal(label, np.argmax(ll, axis=1))
