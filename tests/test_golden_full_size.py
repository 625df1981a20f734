"""The stored full-size oracle goldens (tests/golden/classify_*.json) against the
oracle itself: the regenerated inputs have the golden's fingerprint, its trie sizes
are the oracle trie's, and sampled labels of every stored document, scored again
through the oracle's path-restricted pass, give the stored log-likelihoods.  This
keeps a golden from going stale when the oracle or the input generator changes."""
import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs
from tests.golden.make_full_size_goldens import GOLDENS, fingerprint, oracle_trie
from tests.gpu_util import load_golden

_INPUTS = {}


def _inputs(cid):
    if cid not in _INPUTS:
        _INPUTS.clear()
        _INPUTS[cid] = make_inputs(config(cid))
    return _INPUTS[cid]


@pytest.mark.parametrize("fname,cid,docs,form", GOLDENS)
def test_golden_matches_oracle(fname, cid, docs, form):
    g = load_golden(fname)
    inp = _inputs(cid)
    assert g["docs"] == docs and g["config_id"] == cid
    assert fingerprint(inp, docs) == g["fingerprint"]
    trie = oracle_trie(inp, form)
    assert (g["n_labels"], g["n_nodes"], g["n_int"]) == (trie.n_labels, trie.n_nodes, trie.n_int)
    ll = np.array(g["ll"])
    assert ll.shape == (len(docs), trie.n_labels)
    prob, label = O.label_softmax(ll)
    assert label.tolist() == g["label"]
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, rtol=1e-12)
    model = O.OracleModel(inp)
    rng = np.random.default_rng(cid)
    for i, b in enumerate(docs):
        ids = sorted(set(rng.choice(trie.n_labels, 2, replace=False).tolist() + [g["label"][i]]))
        got, _ = O.label_ll_on_paths(inp, b, ids, model=model, trie=trie)
        np.testing.assert_allclose(got, ll[i, ids], rtol=0, atol=1e-9)
