"""End-to-end parity of tcs_classify against the oracle on all five workloads,
at full size (sampled documents or labels where the oracle would take too long)
and on small shapes with ragged documents and prefix labels."""
import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, make_inputs
from tests.gpu_util import LL_TOL, check_labels, golden_fingerprint, load_golden, say

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def run_gpu(cfg, inp, prepared=False):
    """tcs_classify, or (prepared) tcs_classify_prepare + tcs_classify_run as bench.py
    times it."""
    torch = _torch()
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B) if prepared else None
    label, prob, ll = tcs.classify(model, td, docs, prepared=prep)
    torch.cuda.synchronize()
    out = label.cpu().numpy(), prob.cpu().numpy(), ll.cpu().numpy()
    del model, docs
    torch.cuda.empty_cache()
    return out


SMALL = {
    "tiny-f32": config(1),
    "tiny-f32-ragged": config(1, doc_lens=(1, 32, 7, 0, 19)),
    "running-bf16-small": config(2, V=3000, d=256, B=6, L=100, doc_lens=(100, 1, 257, 0, 64, 130)),
    "zipf-bf16-small": config(3, V=4096, d=128, Hq=8, Hkv=2, B=3, L=50,
                              trie=("zipf", 40, 2, 9, 1.2)),
    "prefix-bf16-small": config(2, V=2000, d=128, Hq=4, Hkv=2, hd=64, B=5, L=40,
                                trie=("explicit", [[3], [3, 4], [3, 4, 5], [3, 6], [9, 9, 9], [9, 9], [1]])),
    "fp8-small": config(5, V=2500, d=192, Hq=4, Hkv=1, B=4, L=300),
    # W8A8 head: hidden rows quantized to E4M3 per row; the second case has 320
    # rows, a full and a ragged row tile
    "fp8a8-small": config(5, V=2500, d=384, Hq=4, Hkv=1, B=4, L=300, head="fp8a8"),
    "fp8a8-rows": config(5, V=3000, d=256, Hq=4, Hkv=1, B=40, L=50, head="fp8a8"),
    # one label (probability 1, always chosen); a 40-token chain beside short labels
    "single-label-bf16": config(2, V=2000, d=128, Hq=4, Hkv=2, hd=64, B=3, L=20,
                                trie=("explicit", [[4, 2, 7]])),
    "deep-chain-bf16": config(2, V=2000, d=128, Hq=4, Hkv=2, hd=128, B=3, L=30,
                              trie=("explicit", [list(range(100, 140)), [5], [100, 101, 7]])),
    # 12 deep with a label that is a prefix of another: the per-label walk over parent
    # arrays staged in LDS, with the head's log-sum-exp folded in and the prefix term
    "deep-prefix-bf16": config(2, V=2000, d=128, Hq=4, Hkv=2, hd=128, B=4, L=30,
                               trie=("explicit", [list(range(100, 112)), list(range(100, 110)), [5],
                                                  [100, 101, 7]])),
    # few-row output projection on the K-split kernel: ragged row and column tiles,
    # 128- and 256-row tiles, even and uneven K splits (R = B x 8 internal nodes)
    "proj-split-bm128": config(2, V=2000, d=320, Hq=4, Hkv=2, hd=128, B=25, L=24),
    "proj-split-bm128-s5": config(2, V=2000, d=1280, Hq=8, Hkv=2, hd=128, B=75, L=8),
    "proj-split-bm256": config(2, V=3000, d=384, Hq=6, Hkv=2, hd=128, B=90, L=16),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_classify_small_vs_oracle(dev, name):
    cfg = SMALL[name]
    inp = make_inputs(cfg, seed=101)
    label, prob, ll = run_gpu(cfg, inp)
    o = O.classify(inp)
    check_labels(ll, prob, label, o["ll"], o["prob"], o["label"], f"classify[{name}]")


@pytest.mark.parametrize("name", ["tiny-f32", "running-bf16-small", "zipf-bf16-small", "fp8-small"])
def test_prepared_run_equals_classify(dev, name):
    """tcs_classify_run on prepared state gives tcs_classify's results bit for bit,
    for two batches in a row on the same state; a batch of another size is refused."""
    torch = _torch()
    cfg = SMALL[name]
    inp = make_inputs(cfg, seed=101)
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    ref = [x.cpu().numpy() for x in tcs.classify(model, td, docs)]
    prep = tcs.Prepared(model, td, docs.B)
    for _ in range(2):
        got = [x.cpu().numpy() for x in tcs.classify(model, td, docs, prepared=prep)]
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            np.testing.assert_array_equal(a, b)
    other = tcs.Prepared(model, td, docs.B + 1)
    with pytest.raises(tcs.TcsError):
        tcs.classify(model, td, docs, prepared=other)
    say(f"prepared[{name}]: run == classify on 2 batches")


def test_classify_many_rows_projection(dev):
    """Enough rows (8 documents x 1881 internal nodes, d = 2560, Hq*hd = 4096) that the
    output projection runs on the ring GEMM: sampled documents against the oracle."""
    cfg = config(3, V=2000, B=8, L=64, trie=("zipf", 1000, 2, 6, 1.2))
    inp = make_inputs(cfg, seed=103)
    label, prob, ll = run_gpu(cfg, inp, prepared=True)
    n_int = O.build_trie(inp["labels"], inp["root_token"], cfg.V).n_int
    assert cfg.B * n_int >= 13056, "needs >= 512 output tiles"
    docs = [0, cfg.B - 1]
    o = O.classify(inp, docs=docs)
    check_labels(ll[docs], prob[docs], label[docs], o["ll"], o["prob"], o["label"],
                 f"classify[ring projection, R={cfg.B * n_int}]")


@pytest.fixture(scope="module")
def cfg2():
    cfg = config(2)
    return cfg, make_inputs(cfg)


def test_prepared_runs_on_three_streams(dev, cfg2):
    """Three batches in flight, as bench.py runs them: tcs_classify_run on three HIP
    streams at once, each with its own workspace, on one prepared state
    (running-example shape, B = 64) gives the single-stream results bit for bit."""
    torch = _torch()
    cfg, inp = cfg2
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    prep = tcs.Prepared(model, td, docs.B)
    ref = [x.cpu().numpy() for x in tcs.classify(model, td, docs, prepared=prep)]
    nbytes = tcs.classify_run_workspace_bytes(model, td, docs)
    streams = [torch.cuda.Stream() for _ in range(3)]
    ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    outs = [tcs.classify(model, td, docs, ws=ws[i % 3], prepared=prep, stream=streams[i % 3])
            for i in range(6)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        for a, b in zip(o, ref):
            np.testing.assert_array_equal(a.cpu().numpy(), b)
    say("three streams: 6 batches == single-stream run")


@pytest.fixture(scope="module")
def cfg5():
    cfg = config(5)
    return cfg, make_inputs(cfg)


@pytest.fixture(scope="module")
def cfg5a8():
    cfg = config(5, head="fp8a8")
    return cfg, make_inputs(cfg)


@pytest.fixture(scope="module")
def cfg2b32():
    cfg = config(2, B=32)
    return cfg, make_inputs(cfg)


@pytest.fixture(scope="module")
def cfg5b16():
    cfg = config(5, B=16)
    return cfg, make_inputs(cfg)


@pytest.fixture(scope="module")
def cfg5a8b16():
    cfg = config(5, B=16, head="fp8a8")
    return cfg, make_inputs(cfg)


# cfg2b32 (256 head rows) and the B = 16 cases (128 rows) run the head on 128-row
# tiles over the full vocabulary; the others on 256-row tiles
@pytest.mark.parametrize("which", ["cfg2", "cfg5", "cfg5a8", "cfg2b32", "cfg5b16", "cfg5a8b16"])
def test_classify_full_size_sampled_docs(dev, which, request):
    """Running-example trie at full size: every label of sampled documents."""
    cfg, inp = request.getfixturevalue(which)
    label, prob, ll = run_gpu(cfg, inp, prepared=True)
    docs = [0, 1, cfg.B // 2, cfg.B - 1]
    o = O.classify(inp, docs=docs)
    check_labels(ll[docs], prob[docs], label[docs], o["ll"], o["prob"], o["label"],
                 f"classify[config {cfg.id} full, docs {docs}]")
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, atol=1e-4)


GOLDEN_FULL = {3: "classify_max_label_set_255.json", 4: "classify_large_finite_set_5000.json"}


@pytest.mark.parametrize("cid", [3, 4])
def test_classify_full_size_every_label_vs_oracle(dev, cid):
    """Large tries at full size (255 labels, B = 32 x 1,024 tokens; 5,000 labels,
    B = 8 x 256), in the prepared launch configuration bench.py times: every label's
    log-likelihood, probability and the chosen label of the stored documents against
    the whole fp64 oracle pass (tests/golden, written by make_full_size_goldens.py
    from oracle/ only).  A third document is checked on sampled labels through the
    oracle's path-restricted pass, and properties that hold at any size on all."""
    g = load_golden(GOLDEN_FULL[cid])
    cfg = config(cid)
    inp = make_inputs(cfg)
    assert golden_fingerprint(inp, g["docs"]) == g["fingerprint"], "inputs differ from the golden's"
    label, prob, ll = run_gpu(cfg, inp, prepared=True)
    docs = g["docs"]
    o_ll = np.array(g["ll"], dtype=np.float64)
    o_prob, o_label = O.label_softmax(o_ll)
    assert o_label.tolist() == g["label"]
    check_labels(ll[docs], prob[docs], label[docs], o_ll, o_prob, o_label,
                 f"classify[config {cid} full, every label of docs {docs}]")
    # another document, sampled labels, through the path-restricted oracle pass
    b = next(x for x in range(cfg.B // 2, cfg.B) if x not in docs)
    M = len(inp["labels"])
    ids = sorted(set(np.random.default_rng(cid).choice(M, 6, replace=False).tolist() + [int(label[b])]))
    o_part, _ = O.label_ll_on_paths(inp, b, ids)
    err = np.abs(ll[b, ids] - o_part).max()
    assert err <= LL_TOL, (b, ids, ll[b, ids], o_part)
    say(f"classify[config {cid} full]: doc {b}, {len(ids)} sampled labels, max |dll| {err:.2e}")
    # properties that hold at any size, on every document
    ll64 = ll.astype(np.float64)
    p_ref = np.exp(ll64 - ll64.max(axis=1, keepdims=True))
    p_ref /= p_ref.sum(axis=1, keepdims=True)
    assert np.abs(prob - p_ref).max() < 1e-4
    np.testing.assert_allclose(prob.sum(axis=1), 1.0, atol=1e-4)
    assert np.array_equal(label, np.argmax(ll, axis=1))
