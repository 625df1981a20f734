"""Pins of the oracle's letters method ("To Classify, Try a Trie Tree", section 3.3):
the rescaled letter probabilities equal the label softmax of the trie pass over the
letters as one-token labels (the vocabulary normaliser cancels, section 4.1), and
the per-letter sequence scores computed with no trie."""
import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs


def _letter_inputs(cfg, seed=5):
    inp = make_inputs(cfg, seed=seed)
    one = dict(inp)
    one["labels"] = [[int(t)] for t in inp["letters"]]
    return inp, one


@pytest.mark.parametrize("cfg", [
    config(1),
    config(1, doc_lens=(3, 0, 17)),
    config(2, V=600, d=64, Hq=4, Hkv=2, hd=32, B=3, L=20),
    config(5, V=500, d=64, Hq=2, Hkv=1, hd=32, B=2, L=30),
])
def test_letters_equals_trie_softmax_over_one_token_labels(cfg):
    inp, one = _letter_inputs(cfg)
    let = O.letters_classify(inp, inp["letters"])
    tri = O.classify(one)
    np.testing.assert_allclose(let["prob"], tri["prob"], rtol=1e-10, atol=1e-13)
    np.testing.assert_array_equal(let["label"], tri["label"])
    # the letter logits differ from the full log-probabilities by one constant per document
    diff = let["z"] - tri["ll"]
    np.testing.assert_allclose(diff - diff[:, :1], 0.0, atol=1e-10)


def test_letters_matches_sequence_scoring():
    cfg = config(1, trie=("zipf", 30, 1, 1, 1.0))
    inp, one = _letter_inputs(cfg)
    let = O.letters_classify(inp, inp["letters"])
    for b in range(cfg.B):
        bf = O.bruteforce_ll(one, b)
        p = np.exp(bf - bf.max())
        np.testing.assert_allclose(let["prob"][b], p / p.sum(), rtol=1e-10, atol=1e-13)


def test_letters_subset_of_documents():
    inp, _ = _letter_inputs(config(1))
    full = O.letters_classify(inp, inp["letters"])
    part = O.letters_classify(inp, inp["letters"], docs=[2, 0])
    np.testing.assert_array_equal(part["z"], full["z"][[2, 0]])
