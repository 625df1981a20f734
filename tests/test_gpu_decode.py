"""Parity of trie_decode ("To Classify, Try a Trie Tree", section 3.1) through
tcs_decode_run: greedy generation inside the label trie, one answer position per
undecided document per step.  The oracle walks the label prefixes and runs the
model on each [root, prefix] sequence in fp64 (pinned on the CPU to the page's
requests per document and to the trie pass's own choices).  Labels and run counts
must match wherever the oracle's two best candidate logits are more than GAP apart
at every step; elsewhere the label must still be one decoding can return."""
import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, make_inputs
from tests.gpu_util import GAP, say

pytestmark = pytest.mark.gpu


def run_decode(cfg, inp):
    import torch
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    outs = []
    for _ in range(2):  # two batches on the same prepared state and workspace size
        label, runs = tcs.trie_decode(model, td, docs, prep)
        torch.cuda.synchronize()
        outs.append((label.cpu().numpy(), runs.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        np.testing.assert_array_equal(a, b)
    del model, docs, prep
    torch.cuda.empty_cache()
    return outs[0]


def check_decode(label, runs, o, labels, what):
    label, runs = label[o["docs"]], runs[o["docs"]]
    sure = o["gap"] > GAP
    np.testing.assert_array_equal(label[sure], o["label"][sure], err_msg=what)
    np.testing.assert_array_equal(runs[sure], o["runs"][sure], err_msg=what)
    returnable = {m for m, l in enumerate(labels)
                  if not any(len(l2) > len(l) and list(l2[:len(l)]) == list(l) for l2 in labels)}
    assert all(int(x) in returnable for x in label), what
    say(f"{what}: labels compared {int(sure.sum())}/{len(sure)}, mean runs {runs.mean():.3f}")


SMALL = {
    "tiny-f32": config(1),
    "tiny-f32-ragged": config(1, doc_lens=(1, 32, 7, 0, 19)),
    "running-bf16-small": config(2, V=3000, d=256, B=6, L=100, doc_lens=(100, 1, 257, 0, 64, 130)),
    "zipf-bf16-small": config(3, V=4096, d=128, Hq=8, Hkv=2, B=5, L=50,
                              trie=("zipf", 60, 2, 9, 1.2)),
    "prefix-bf16-small": config(2, V=2000, d=128, Hq=4, Hkv=2, B=6, L=40,
                                trie=("explicit", [[3], [3, 4], [3, 4, 5], [3, 6], [9, 9, 9], [9, 9],
                                                   [1], [7, 8, 9, 10], [7, 8, 9, 11]])),
    "fp8-small": config(5, V=2500, d=192, Hq=4, Hkv=1, B=4, L=300),
    "single-label-bf16": config(2, V=2000, d=128, Hq=4, Hkv=2, B=3, L=20,
                                trie=("explicit", [[4, 2, 7]])),
    "deep-chain-bf16": config(2, V=2000, d=128, Hq=4, Hkv=2, B=3, L=30,
                              trie=("explicit", [list(range(100, 140)), [5], [100, 101, 7]])),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_small_vs_oracle(dev, name):
    cfg = SMALL[name]
    inp = make_inputs(cfg, seed=113)
    label, runs = run_decode(cfg, inp)
    o = O.trie_decode(inp)
    check_decode(label, runs, o, inp["labels"], f"decode[{name}]")


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_decode_full_size(dev, cid):
    """Full-size workloads: every document for configs 2-4, sampled documents for
    the 128 x 4096-token batch with the fp8 head."""
    cfg = config(cid)
    inp = make_inputs(cfg)
    label, runs = run_decode(cfg, inp)
    docs = list(range(cfg.B)) if cid != 5 else [0, 1, cfg.B // 2, cfg.B - 1]
    o = O.trie_decode(inp, docs=docs)
    check_decode(label, runs, o, inp["labels"], f"decode[config {cid} full]")


def test_decode_runs_on_two_streams(dev):
    """Batches in flight, as bench.py runs them (here two): tcs_decode_run on two HIP streams
    at once, each with its own workspace (the per-document decoding state lives
    there), gives the single-stream labels and run counts."""
    import torch
    cfg = config(3, V=4096, d=128, Hq=8, Hkv=2, B=40, L=50, trie=("zipf", 60, 2, 9, 1.2))
    inp = make_inputs(cfg, seed=117)
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    ref = [x.cpu().numpy() for x in tcs.trie_decode(model, td, docs, prep)]
    nbytes = tcs.decode_workspace_bytes(model, td, docs)
    streams = [torch.cuda.Stream() for _ in range(2)]
    ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    torch.cuda.synchronize()
    outs = [tcs.trie_decode(model, td, docs, prep, ws=ws[i % 2], stream=streams[i % 2])
            for i in range(6)]
    torch.cuda.synchronize()
    for o in outs:
        for a, b in zip(o, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b)
    say(f"decode on two streams: 6 batches == single-stream run (max steps {t.max_decode_steps})")
