"""Pins of the oracle's path-restricted pass, `label_ll_on_paths`.

It scores the listed labels of one document from the query rows on their paths
only, which is how the largest tries can be checked label by label.  It must give
the same log-likelihoods as the full trie pass (`classify`) and as per-label
sequence scoring with no trie at all (`bruteforce_ll`, the direct definition of
"To Classify, Try a Trie Tree", section 3.2: a label's probability is the product
of its tokens' probabilities, with the prefix rule for a label that others
continue).  A dropped ancestor row, a missed child edge of a prefix label or a
wrong document slice would break one of these."""
import numpy as np
import pytest

import oracle as O
from synth import config, make_inputs
from synth.gen import zipf_copy_prefix_labels


def _labels_with_prefixes(seed, V, M):
    """Zipf copy-prefix labels plus, for a few of them, their own shorter starts
    as extra labels (prefix labels, some with several children)."""
    rng = np.random.default_rng(seed)
    labels = zipf_copy_prefix_labels(rng, V, M, 2, 6, 1.2)
    seen = {tuple(l) for l in labels}
    for l in list(labels[:: max(1, M // 6)]):
        for k in (1, len(l) - 1):
            p = tuple(l[:k])
            if 0 < k < len(l) and p not in seen:
                labels.append(list(p))
                seen.add(p)
    return labels


CASES = {
    # token documents (fp32, the library's tiny configuration), ragged with an empty one
    "tokens-f32": lambda labels: config(1, V=60, d=32, Hq=2, Hkv=1, hd=16, std=0.4,
                                        doc_lens=(5, 0, 9, 1), trie=("explicit", labels)),
    # key/value documents (bf16 storage, GQA), ragged with an empty one
    "kv-bf16": lambda labels: config(2, V=60, d=64, Hq=4, Hkv=2, hd=16, std=0.3,
                                     doc_lens=(7, 1, 0, 12), trie=("explicit", labels)),
    # fp8 head with row scales
    "kv-fp8": lambda labels: config(5, V=60, d=64, Hq=4, Hkv=1, hd=16, std=0.3,
                                    doc_lens=(3, 11), trie=("explicit", labels)),
}


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("case", list(CASES))
def test_label_ll_on_paths_equals_full_pass(case, seed):
    labels = _labels_with_prefixes(seed, 60, 24)
    cfg = CASES[case](labels)
    inp = make_inputs(cfg, seed=40 + seed)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    assert any(trie.child_count[trie.label_node[m]] > 0 for m in range(trie.n_labels)), \
        "case needs a prefix label"
    full = O.classify(inp)
    model = O.OracleModel(inp)
    M = len(inp["labels"])
    rng = np.random.default_rng(seed)
    for b in range(len(inp["doc_offsets"]) - 1):
        ids = sorted(rng.choice(M, 7, replace=False).tolist())
        # every prefix label of the set, and one label whose path is a single chain
        ids = sorted(set(ids) | {m for m in range(M) if trie.child_count[trie.label_node[m]] > 0})
        got, info = O.label_ll_on_paths(inp, b, ids, model=model, trie=trie)
        np.testing.assert_allclose(got, full["ll"][b, ids], rtol=0, atol=1e-12)
        # only rows on the listed labels' paths were computed
        assert len(info["rows"]) <= trie.n_int


@pytest.mark.parametrize("case", ["tokens-f32", "kv-bf16"])
def test_label_ll_on_paths_equals_sequence_scoring(case):
    labels = _labels_with_prefixes(5, 60, 16)
    cfg = CASES[case](labels)
    inp = make_inputs(cfg, seed=77)
    M = len(inp["labels"])
    for b in range(len(inp["doc_offsets"]) - 1):
        ids = list(range(0, M, 2))
        got, _ = O.label_ll_on_paths(inp, b, ids)
        np.testing.assert_allclose(got, O.bruteforce_ll(inp, b, label_ids=ids), rtol=0, atol=1e-10)


def test_label_ll_on_paths_single_row_and_last_document():
    """A label set whose listed label needs only the root row, scored for the last
    document of a ragged batch: the restricted pass still slices that document."""
    labels = [[3], [4, 5], [4, 6, 7]]
    cfg = config(2, V=16, d=64, Hq=2, Hkv=1, hd=32, std=0.3, doc_lens=(2, 9, 4),
                 trie=("explicit", labels))
    inp = make_inputs(cfg, seed=5)
    full = O.classify(inp)
    got, info = O.label_ll_on_paths(inp, 2, [0])
    assert info["rows"] == [0]
    np.testing.assert_allclose(got, full["ll"][2, [0]], rtol=0, atol=1e-12)
