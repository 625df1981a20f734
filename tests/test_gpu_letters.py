"""Parity of the letters method ("To Classify, Try a Trie Tree", section 3.3) through
tcs_letters_run: one answer position per document, the M letter rows of the
head, probabilities rescaled over the letters.  The oracle computes the same from
its definition in fp64 (pinned on the CPU to the trie softmax over one-token
labels)."""
import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, make_inputs
from tests.gpu_util import check_labels, say

pytestmark = pytest.mark.gpu


def run_letters(cfg, inp):
    import torch
    letters = np.asarray(inp["letters"], dtype=np.int32)
    offs = np.arange(len(letters) + 1, dtype=np.int32)
    t = tcs.trie_build(offs, letters, inp["root_token"], cfg.V)
    assert t.n_int == 1 and t.max_depth == 1
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    outs = []
    for _ in range(2):  # two batches on the same prepared state
        label, prob, ll = tcs.letters(model, td, docs, prep)
        torch.cuda.synchronize()
        outs.append((label.cpu().numpy(), prob.cpu().numpy(), ll.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    del model, docs, prep
    torch.cuda.empty_cache()
    return outs[0]


SMALL = {
    "tiny-f32": config(1),
    "tiny-f32-ragged": config(1, doc_lens=(1, 32, 7, 0, 19)),
    "running-bf16-small": config(2, V=3000, d=256, B=6, L=100, doc_lens=(100, 1, 257, 0, 64, 130)),
    "many-letters-bf16": config(3, V=4096, d=128, Hq=8, Hkv=2, B=3, L=50,
                                trie=("zipf", 700, 2, 9, 1.2)),
    "fp8-small": config(5, V=2500, d=192, Hq=4, Hkv=1, B=4, L=300),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_letters_small_vs_oracle(dev, name):
    cfg = SMALL[name]
    inp = make_inputs(cfg, seed=109)
    label, prob, ll = run_letters(cfg, inp)
    o = O.letters_classify(inp, inp["letters"])
    check_labels(ll, prob, label, o["z"], o["prob"], o["label"], f"letters[{name}]")


@pytest.mark.parametrize("cid", [2, 4, 5])
def test_letters_full_size(dev, cid):
    """Full-size workloads (10 letters over 64 x 512-token documents; 5000 letters over
    8 x 256; 10 letters over 128 x 4096 with the fp8 head): every document for the
    first two, sampled documents for the last."""
    cfg = config(cid)
    inp = make_inputs(cfg)
    label, prob, ll = run_letters(cfg, inp)
    docs = list(range(cfg.B)) if cid != 5 else [0, 1, cfg.B // 2, cfg.B - 1]
    o = O.letters_classify(inp, inp["letters"], docs=docs)
    check_labels(ll[docs], prob[docs], label[docs], o["z"], o["prob"], o["label"],
                 f"letters[config {cid} full, {len(docs)} docs]")
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, atol=1e-4)
    say(f"letters[config {cid}]: M={len(inp['letters'])}")


def test_letters_runs_on_two_streams(dev):
    """tcs_letters_run on two HIP streams at once, each with its own workspace, gives
    the single-stream results bit for bit."""
    import torch
    cfg = SMALL["running-bf16-small"]
    inp = make_inputs(cfg, seed=119)
    letters = np.asarray(inp["letters"], dtype=np.int32)
    t = tcs.trie_build(np.arange(len(letters) + 1, dtype=np.int32), letters, inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    ref = [x.cpu().numpy() for x in tcs.letters(model, td, docs, prep)]
    nbytes = tcs.classify_run_workspace_bytes(model, td, docs)
    streams = [torch.cuda.Stream() for _ in range(2)]
    ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    outs = [tcs.letters(model, td, docs, prep, ws=ws[i % 2], stream=streams[i % 2]) for i in range(6)]
    torch.cuda.synchronize()
    for o in outs:
        for a, b in zip(o, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b)
