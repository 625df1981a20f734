"""Per-kernel parity on the GPU: each HIP entry point, fed seeded synthetic inputs,
against the fp64 oracle on the same inputs."""
import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, labels_to_csr, make_inputs
from tests.gpu_util import check_labels, say, to_bf16_exact

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


# ------------------------------------------------------------------ path sums

def _proper_lp(trie, B, rng):
    """Edge log-probs drawn as proper next-token distributions (children share
    part of the mass, the rest goes to other tokens)."""
    lp = np.zeros((B, trie.n_nodes))
    for r in range(trie.n_int):
        u = trie.qnode[r]
        cb, cc = trie.child_begin[u], trie.child_count[u]
        w = rng.dirichlet(np.ones(cc + 2), size=B)
        lp[:, cb:cb + cc] = np.log(w[:, :cc])
    return lp.astype(np.float32)


def _run_path_sum(labels, root, V, lp, with_prob=True, walk=False):
    """tcs_path_sum_softmax; walk=True leaves out the level-by-level arrays, so every
    label's path is walked whatever the trie's size."""
    torch = _torch()
    t = tcs.trie_build(*labels_to_csr(labels), root, V)
    td = tcs.TrieDevice(t)
    if walk:
        td.struct.row_level_offsets = None
        td.struct.label_row = None
    ll, prob, label = tcs.path_sum_softmax(torch.from_numpy(lp).cuda(), td, with_prob=with_prob)
    torch.cuda.synchronize()
    return ll.cpu().numpy(), (prob.cpu().numpy() if prob is not None else None), label.cpu().numpy()


def test_path_sum_worked_example(dev):
    # Quail execution docs, label scoring: refund 0.8 x 0.6 = 0.48 vs praise 0.3
    trie = O.build_trie([[10, 11], [20]], 0, 32)
    lp = np.zeros((1, trie.n_nodes), dtype=np.float32)
    for c in range(1, trie.n_nodes):
        lp[0, c] = np.log({10: 0.8, 11: 0.6, 20: 0.3}[trie.token[c]])
    ll, prob, label = _run_path_sum([[10, 11], [20]], 0, 32, lp)
    np.testing.assert_allclose(np.exp(ll[0, 0]), 0.48, rtol=1e-6)
    np.testing.assert_allclose(prob[0], [0.48 / 0.78, 0.3 / 0.78], atol=1e-6)
    assert label[0] == 0


PATH_CASES = {
    "running": ("cfg", 2),
    "zipf255": ("cfg", 3),
    "zipf5000": ("cfg", 4),
    "prefix": ("labels", [[3], [3, 4], [3, 4, 5], [3, 6], [9, 9, 9], [9, 9], [1]]),
    # depth 12 with prefix labels: the walk with the parent arrays staged in LDS
    "prefix-deep": ("labels", [[5, 1, 2, 3, 4, 5, 6, 7, 8], [5, 1, 2, 3, 4, 5, 6, 7],
                               [5, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11], [5, 1, 2, 3, 9], [2],
                               [3] * 10, [3] * 12, [3] * 11 + [4]]),
    "single": ("labels", [[4, 2, 7]]),
}


@pytest.mark.parametrize("case", list(PATH_CASES))
@pytest.mark.parametrize("with_prob", [True, False])
def test_path_sum_vs_oracle(dev, case, with_prob):
    kind, val = PATH_CASES[case]
    if kind == "cfg":
        inp = make_inputs(config(val), weights=False) if val != 5 else None
        labels, root, V = inp["labels"], inp["root_token"], config(val).V
    else:
        labels, root, V = val, 0, 16
    trie = O.build_trie(labels, root, V)
    rng = np.random.default_rng(len(labels))
    B = 37
    lp = _proper_lp(trie, B, rng)
    ll, prob, label = _run_path_sum(labels, root, V, lp, with_prob)
    o_ll = O.path_log_likelihoods(trie, lp.astype(np.float64))
    o_p, o_lab = O.label_softmax(o_ll)
    fin = np.isfinite(o_ll)
    assert np.abs(ll[fin] - o_ll[fin]).max() < 1e-4
    if with_prob:
        assert np.abs(prob - o_p).max() < 1e-5
        np.testing.assert_allclose(prob.sum(axis=1), 1.0, atol=1e-5)
    check_labels(ll, prob, label, o_ll, o_p, o_lab, f"path_sum[{case}]")


@pytest.mark.parametrize("cid,B", [(4, 300), (3, 600)])
def test_path_sum_many_docs_per_workgroup(dev, cid, B):
    """Many documents: on the 5000-label trie the level-by-level kernel has more
    documents than workgroups, so workgroups score several in turn, each loaded
    while the previous one is scored; the 255-label trie takes the per-label walk,
    one workgroup per document."""
    inp = make_inputs(config(cid), weights=False)
    labels, root, V = inp["labels"], inp["root_token"], config(cid).V
    trie = O.build_trie(labels, root, V)
    lp = _proper_lp(trie, B, np.random.default_rng(cid))
    ll, prob, label = _run_path_sum(labels, root, V, lp)
    o_ll = O.path_log_likelihoods(trie, lp.astype(np.float64))
    o_p, o_lab = O.label_softmax(o_ll)
    assert np.abs(ll - o_ll).max() < 1e-4
    assert np.abs(prob - o_p).max() < 1e-5
    check_labels(ll, prob, label, o_ll, o_p, o_lab, f"path_sum[config {cid}, B={B}]")


def test_path_sum_ties_take_lowest_label(dev):
    labels = [[1], [2], [3], [4]]
    trie = O.build_trie(labels, 0, 8)
    lp = np.zeros((3, trie.n_nodes), dtype=np.float32)
    lp[:, 1:] = np.log(0.2)
    lp[1, 3] = np.log(0.3)    # token 3 (label 2) wins in doc 1
    lp[2, 2:4] = np.log(0.3)  # labels 1 and 2 tie in doc 2
    _, prob, label = _run_path_sum(labels, 0, 8, lp)
    assert label.tolist() == [0, 2, 1]


# ------------------------------------------------------------------ output head

HEAD_CASES = {
    # name: (V, d, n_int source, B, head kind)
    "small-bf16": dict(V=1000, d=128, labels=("zipf", 40, 2, 6, 1.2), B=13, head="bf16"),
    "small-fp8": dict(V=777, d=192, labels=("zipf", 40, 2, 6, 1.2), B=9, head="fp8"),
    "small-f32": dict(V=1000, d=64, labels=("running",), B=4, head="f32"),
    "ragged-vocab": dict(V=257, d=64, labels=("zipf", 12, 1, 4, 1.0), B=3, head="bf16"),
    # row-tile counts (72 rows per document) for the head's tile order, in the tile
    # size the launcher picks for these vocabularies: 32 tiles of 128 rows (one group
    # of 32), 39 of 256 (one group of 32 + a 7-row strip), 146 of 128 (four groups +
    # strips of 6 and 6 and 6)
    "rows-56-docs": dict(V=1000, d=128, labels=("zipf", 40, 2, 6, 1.2), B=56, head="bf16"),
    "rows-138-docs": dict(V=1000, d=128, labels=("zipf", 40, 2, 6, 1.2), B=138, head="bf16"),
    "rows-259-docs-fp8": dict(V=777, d=192, labels=("zipf", 40, 2, 6, 1.2), B=259, head="fp8"),
}


def _head_case(name):
    c = HEAD_CASES[name]
    dtype = "f32" if c["head"] == "f32" else "bf16"
    cfg = config(3, V=c["V"], d=c["d"], Hq=2, Hkv=1, hd=64, B=c["B"], L=1, dtype=dtype,
                 head="fp8" if c["head"] == "fp8" else "same", trie=c["labels"])
    return cfg, make_inputs(cfg, seed=17)


def _head_inputs(cfg, inp, rows, rng):
    if cfg.dtype == "bf16":
        h = O.round_bf16(rng.standard_normal((rows, cfg.d)))
    else:
        h = rng.standard_normal((rows, cfg.d)).astype(np.float32).astype(np.float64)
    return h


def _gpu_head(cfg, inp, trie_np, h, B):
    torch = _torch()
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    model = tcs.Model(cfg, inp)
    hd = (to_bf16_exact(h) if cfg.dtype == "bf16" else torch.from_numpy(h.astype(np.float32))).cuda()
    lse, lp = tcs.lmhead_lse_gather(hd, model.t["W"], td, B, w_scale=model.t["W_scale"])
    torch.cuda.synchronize()
    return lse.cpu().numpy(), lp.cpu().numpy()


@pytest.mark.parametrize("name", list(HEAD_CASES))
def test_lmhead_vs_oracle(dev, name):
    cfg, inp = _head_case(name)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    B = cfg.B
    rng = np.random.default_rng(3)
    h = _head_inputs(cfg, inp, B * trie.n_int, rng)
    lse, lp = _gpu_head(cfg, inp, trie, h, B)
    model = O.OracleModel(inp)
    o_lse = O.lm_head_lse(model, h)
    o_lp = O.edge_logprobs(model, trie, h.reshape(B, trie.n_int, -1), o_lse.reshape(B, trie.n_int))
    e1 = np.abs(lse - o_lse).max()
    e2 = np.abs(lp - o_lp).max()
    say(f"lmhead[{name}] R={B * trie.n_int} ({-(-B * trie.n_int // 256)} row tiles) V={cfg.V}: "
        f"max |dlse| {e1:.2e} max |dlp| {e2:.2e}")
    assert e1 < 2e-4 and e2 < 2e-4
    assert np.all(lp[:, 0] == 0)


def test_lmhead_zero_hidden_gives_log_vocab(dev):
    cfg, inp = _head_case("small-bf16")
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    B = 5
    lse, lp = _gpu_head(cfg, inp, trie, np.zeros((B * trie.n_int, cfg.d)), B)
    np.testing.assert_allclose(lse, np.log(cfg.V), atol=2e-6)
    np.testing.assert_allclose(lp[:, 1:], -np.log(cfg.V), atol=2e-6)


# Full-size head (Qwen3-4B shapes: d = 2,560, 40 k-steps of 64 with no padding;
# V = 151,936, 594 vocabulary tiles over several persistent rounds), element by
# element against the oracle.  Rows R = 8 B on the running-example trie; the
# launcher takes 128-row tiles at R = 128 and 256 and 256-row tiles from 512 rows;
# past 4,096 rows the partials are stored tile-major (sampled documents checked).
# A dropped 256-entry vocabulary tile would move lse by about 1.7e-3.
FULL_HEAD = {
    "bf16-R128": ("bf16", 16, None),
    "bf16-R256": ("bf16", 32, None),
    "bf16-R512": ("bf16", 64, None),
    "fp8-R1024": ("fp8", 128, None),
    "w8a8-R1024": ("fp8a8", 128, None),
    "bf16-R4160": ("bf16", 520, [0, 1, 31, 32, 255, 256, 300, 511, 512, 519]),
}


@pytest.fixture(scope="module")
def full_head_inputs():
    """Weights of the running-example (bf16 head) and long-document (fp8 head)
    workloads; a one-token batch, since only the weights are used."""
    cache = {}

    def get(kind):
        base = 5 if kind in ("fp8", "fp8a8") else 2
        if cache.get("base") != base:
            cache.clear()
            cache["base"] = base
            cache["inp"] = make_inputs(config(base, B=1, L=1))
        if kind not in cache:
            # the W8A8 head reads the same E4M3 weights; only the activations differ
            cfg = config(base, B=1, L=1, head={"fp8": "fp8", "fp8a8": "fp8a8"}.get(kind, "same"))
            inp = dict(cache["inp"], cfg=cfg)
            cache[kind] = (cfg, inp, tcs.Model(cfg, inp), O.OracleModel(inp))
        return cache[kind]
    return get


@pytest.mark.parametrize("name", list(FULL_HEAD))
def test_lmhead_full_size_vs_oracle(dev, full_head_inputs, name):
    torch = _torch()
    kind, B, docs = FULL_HEAD[name]
    cfg, inp, model, omodel = full_head_inputs(kind)
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    R = B * trie.n_int
    h = O.round_bf16(np.random.default_rng(R).standard_normal((R, cfg.d)))
    say(f"lmhead-full[{name}]: R={R} d={cfg.d} V={cfg.V}")
    lse, lp = tcs.lmhead_lse_gather(to_bf16_exact(h).cuda(), model.t["W"], td, B,
                                    w_scale=model.t["W_scale"], act8=(kind == "fp8a8"))
    torch.cuda.synchronize()
    lse = lse.cpu().numpy().reshape(B, trie.n_int)
    lp = lp.cpu().numpy()
    docs = list(range(B)) if docs is None else docs
    hs = h.reshape(B, trie.n_int, cfg.d)[docs]
    o_lse = O.lm_head_lse(omodel, hs.reshape(-1, cfg.d)).reshape(len(docs), trie.n_int)
    o_lp = O.edge_logprobs(omodel, trie, hs, o_lse)
    e1 = np.abs(lse[docs] - o_lse).max()
    e2 = np.abs(lp[docs] - o_lp).max()
    say(f"lmhead-full[{name}]: {len(docs)} docs compared, max |dlse| {e1:.2e} max |dlp| {e2:.2e}")
    assert e1 < 2e-4 and e2 < 2e-4
    assert np.all(lp[:, 0] == 0)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(lp))


# ------------------------------------------------------------------ tree attention

ATTN_CASES = {
    # rows per (document, KV head) <= 64 -> key-streaming kernel (hd 128) or the
    # 32-row / 4-key-slice kernel (hd 64); more rows -> 128-row kernel
    "running-hd128": dict(labels=("running",), Hq=8, Hkv=2, hd=128, lens=(0, 1, 31, 32, 129, 300)),
    "running-hd128-g8": dict(labels=("running",), Hq=16, Hkv=2, hd=128, lens=(3, 64, 257, 1000)),
    "running-hd128-long": dict(labels=("running",), Hq=4, Hkv=1, hd=128, lens=(4113, 2, 4096)),
    "running-hd64": dict(labels=("running",), Hq=4, Hkv=1, hd=64, lens=(5, 64, 200)),
    "zipf-hd128": dict(labels=("zipf", 30, 2, 6, 1.2), Hq=8, Hkv=2, hd=128, lens=(0, 33, 97)),
    "zipf-hd64-g8": dict(labels=("zipf", 20, 2, 5, 1.2), Hq=8, Hkv=1, hd=64, lens=(7, 70)),
    "f32": dict(labels=("running",), Hq=2, Hkv=1, hd=64, lens=(3, 40), dtype="f32"),
}


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_tree_attn_vs_oracle(dev, name):
    torch = _torch()
    c = ATTN_CASES[name]
    dtype = c.get("dtype", "bf16")
    cfg = config(2, V=5000, d=64, Hq=c["Hq"], Hkv=c["Hkv"], hd=c["hd"], dtype=dtype,
                 trie=c["labels"], doc_lens=c["lens"])
    inp = make_inputs(cfg, seed=23, weights=False)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    rng = np.random.default_rng(5)
    rnd = O.round_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    n = trie.n_int
    qn = rnd(rng.standard_normal((n, cfg.Hq, cfg.hd)))
    kn = rnd(rng.standard_normal((n, cfg.Hkv, cfg.hd)))
    vn = rnd(rng.standard_normal((n, cfg.Hkv, cfg.hd)))
    Kd = O.decode_bf16(inp["Kd"]) if dtype == "bf16" else inp["Kd"].astype(np.float64)
    Vd = O.decode_bf16(inp["Vd"]) if dtype == "bf16" else inp["Vd"].astype(np.float64)
    scale = 1.0 / np.sqrt(cfg.hd)
    want = O.tree_attention(qn, kn, vn, trie, Kd, Vd, inp["doc_offsets"], scale)
    conv = (lambda a: to_bf16_exact(a).cuda()) if dtype == "bf16" else \
        (lambda a: torch.from_numpy(a.astype(np.float32)).cuda())
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    out = tcs.tree_attn(conv(qn), conv(kn), conv(vn), conv(Kd), conv(Vd),
                        torch.from_numpy(inp["doc_offsets"]).cuda(), td["qparent"], scale)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    if dtype == "bf16":
        # O is stored in bf16: compare with the oracle's value rounded the same way.
        # Allowed: one bf16 ulp of the value (a rounding flip), plus an absolute 4e-6
        # for outputs near zero, where fp32 accumulation error exceeds their ulp.
        ref = O.round_bf16(want)
        ulp = np.ldexp(1.0, np.frexp(np.abs(ref) + 1e-30)[1] - 8)
        off = np.maximum(np.abs(got - ref) - 4e-6, 0.0) / ulp
        exact = float((got == ref).mean())
        say(f"tree_attn[{name}] n_int={n}: exact bf16 match {exact:.4f}, max off {off.max():.2f} ulp")
        assert off.max() <= 1.0 and exact >= 0.99
    else:
        err = np.abs(got - want)
        say(f"tree_attn[{name}] n_int={n}: max |dO| {err.max():.2e}")
        assert np.all(err <= 1e-5 + 1e-5 * np.abs(want))


def test_tree_attn_many_rows_many_docs(dev):
    """Many query rows and many documents, so the many-row kernel scores several
    documents per workgroup (their queries and path partials read once): sampled
    documents across the batch, including empty ones, against the oracle."""
    torch = _torch()
    B = 80
    lens = tuple(int(x) for x in np.random.default_rng(11).integers(0, 70, size=B))
    lens = (0,) + lens[1:-1] + (65,)
    cfg = config(2, V=20000, d=64, Hq=8, Hkv=2, hd=128, trie=("zipf", 1000, 2, 6, 1.2), doc_lens=lens)
    inp = make_inputs(cfg, seed=29, weights=False)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    rng = np.random.default_rng(6)
    n = trie.n_int
    assert n * 4 > 64 * 4, "needs the many-row kernel"
    qn = O.round_bf16(rng.standard_normal((n, cfg.Hq, cfg.hd)))
    kn = O.round_bf16(rng.standard_normal((n, cfg.Hkv, cfg.hd)))
    vn = O.round_bf16(rng.standard_normal((n, cfg.Hkv, cfg.hd)))
    Kd, Vd = O.decode_bf16(inp["Kd"]), O.decode_bf16(inp["Vd"])
    scale = 1.0 / np.sqrt(cfg.hd)
    docs = [0, 1, 2, 3, 4, 5, 39, 40, 78, 79]
    want = O.tree_attention(qn, kn, vn, trie, Kd, Vd, inp["doc_offsets"], scale, docs=docs)
    conv = lambda a: to_bf16_exact(a).cuda()
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    out = tcs.tree_attn(conv(qn), conv(kn), conv(vn), conv(Kd), conv(Vd),
                        torch.from_numpy(inp["doc_offsets"]).cuda(), td["qparent"], scale)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()[docs]
    ref = O.round_bf16(want)
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref) + 1e-30)[1] - 8)
    off = np.maximum(np.abs(got - ref) - 4e-6, 0.0) / ulp
    exact = float((got == ref).mean())
    say(f"tree_attn[many rows, B={B}] n_int={n}: exact bf16 match {exact:.4f}, max off {off.max():.2f} ulp")
    assert off.max() <= 1.0 and exact >= 0.99


def test_path_sum_walk_and_levels_agree_on_large_trie(dev):
    """The 5000-label trie through both path kernels: the level-by-level one (its
    arrays given) and the per-label walk (arrays left out), each against the oracle."""
    inp = make_inputs(config(4), weights=False)
    labels, root, V = inp["labels"], inp["root_token"], config(4).V
    trie = O.build_trie(labels, root, V)
    lp = _proper_lp(trie, 9, np.random.default_rng(44))
    o_ll = O.path_log_likelihoods(trie, lp.astype(np.float64))
    o_p, o_lab = O.label_softmax(o_ll)
    got = {}
    for walk in (False, True):
        ll, prob, label = _run_path_sum(labels, root, V, lp, walk=walk)
        assert np.abs(ll - o_ll).max() < 1e-4
        assert np.abs(prob - o_p).max() < 1e-5
        got[walk] = ll
    assert np.abs(got[True] - got[False]).max() < 1e-4
