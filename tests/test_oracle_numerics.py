"""Pins of the oracle's numeric building blocks against library routines and
closed forms (CPU only)."""
import numpy as np
import pytest
import scipy.special
import torch

import oracle as O
from synth import config, make_inputs
from synth.gen import _bf16_bits_from_f32


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(3.0)
    # force exact ties: low 16 bits 0x8000, with both even and odd kept mantissas
    ties = (x.view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), np.float32([0.0, -0.0, 1e-40, -3e-39, 3.3e38])])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_generator_bf16_bits_decode():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(10000).astype(np.float32)
    bits = _bf16_bits_from_f32(x)
    np.testing.assert_array_equal(O.decode_bf16(bits), O.round_bf16(x.astype(np.float64)))


def test_decode_e4m3_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    np.testing.assert_array_equal(got[ok], want[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_fp8_head_rows_reach_448():
    cfg = config(5, V=300, d=64, Hq=2, Hkv=1, hd=64, B=1, L=4)
    inp = make_inputs(cfg)
    q = O.decode_e4m3(inp["W"])
    assert np.all(np.abs(q).max(axis=1) == 448.0)
    # nearest-even quantisation: torch's own fp32 -> e4m3 cast of the decoded value is a fixed point
    tq = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(tq, q)


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96)) * 0.05
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(x), want, rtol=1e-13, atol=0)


def _canonical_internal(labels):
    pre = set()
    for l in labels:
        for k in range(1, len(l) + 1):
            pre.add(tuple(l[:k]))
    order = [()] + sorted(pre, key=lambda p: (len(p), p))
    internal = [p for p in order if any(q[:len(p)] == p and len(q) > len(p) for q in pre)]
    return internal


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (8, 2)])
def test_tree_attention_matches_torch_sdpa(Hq, Hkv):
    """Ancestor-masked attention equals torch's SDPA with an explicit mask built from
    the label strings (node w visible to node u iff w's token path is a prefix of u's)."""
    rng = np.random.default_rng(3)
    labels = [[1, 2, 3], [1, 2, 4], [1, 5], [6], [6, 7, 8, 9], [2]]
    trie = O.build_trie(labels, 0, 16)
    internal = _canonical_internal(labels)
    assert len(internal) == trie.n_int
    hd = 16
    n = trie.n_int
    qn = rng.standard_normal((n, Hq, hd))
    kn = rng.standard_normal((n, Hkv, hd))
    vn = rng.standard_normal((n, Hkv, hd))
    lens = [5, 1, 9]
    offs = np.concatenate([[0], np.cumsum(lens)])
    Kd = rng.standard_normal((offs[-1], Hkv, hd))
    Vd = rng.standard_normal((offs[-1], Hkv, hd))
    scale = 0.3
    got = O.tree_attention(qn, kn, vn, trie, Kd, Vd, offs, scale)
    for b, L in enumerate(lens):
        mask = np.zeros((n, L + n), dtype=bool)
        mask[:, :L] = True
        for i, pu in enumerate(internal):
            for j, pw in enumerate(internal):
                mask[i, L + j] = pu[:len(pw)] == pw
        q = torch.from_numpy(qn.transpose(1, 0, 2).copy())[None]
        k = torch.from_numpy(np.concatenate([Kd[offs[b]:offs[b + 1]], kn]).transpose(1, 0, 2).copy())[None]
        v = torch.from_numpy(np.concatenate([Vd[offs[b]:offs[b + 1]], vn]).transpose(1, 0, 2).copy())[None]
        want = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=torch.from_numpy(mask), scale=scale, enable_gqa=True)[0]
        np.testing.assert_allclose(got[b], want.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_tree_attention_zero_query_is_uniform_mean():
    rng = np.random.default_rng(4)
    labels = [[1, 2, 3, 4], [1, 2, 5], [7]]
    trie = O.build_trie(labels, 0, 8)
    n, hd, Hq, Hkv = trie.n_int, 8, 2, 1
    kn = rng.standard_normal((n, Hkv, hd))
    vn = rng.standard_normal((n, Hkv, hd))
    Kd = rng.standard_normal((6, Hkv, hd))
    Vd = rng.standard_normal((6, Hkv, hd))
    got = O.tree_attention(np.zeros((n, Hq, hd)), kn, vn, trie, Kd, Vd, np.array([0, 6]), 1.0)
    for r in range(n):
        u = trie.qnode[r]
        path = [u]
        while path[-1] > 0:
            path.append(trie.parent[path[-1]])
        rows = [trie.qrow[w] for w in path]
        want = (Vd[:, 0].sum(0) + vn[rows, 0].sum(0)) / (6 + trie.depth[u] + 1)
        for h in range(Hq):
            np.testing.assert_allclose(got[0, r, h], want, rtol=1e-13, atol=1e-14)


def _tiny_model(dtype="f32", head="same", V=50, d=32, Hq=2, Hkv=1, hd=16, labels=None, B=2, L=5):
    lab = labels or [[3, 4], [3, 5, 6], [7], [8, 9]]
    cfg = config(1, V=V, d=d, Hq=Hq, Hkv=Hkv, hd=hd, dtype=dtype, head=head, B=B, L=L,
                 trie=("explicit", lab))
    inp = make_inputs(cfg, seed=11)
    return inp, O.OracleModel(inp)


def test_lse_of_zero_hidden_is_log_vocab():
    for dtype, head in (("f32", "same"), ("bf16", "same"), ("bf16", "fp8")):
        inp, model = _tiny_model(dtype, head)
        h = np.zeros((3, model.cfg.d))
        np.testing.assert_allclose(O.lm_head_lse(model, h), np.log(model.cfg.V), rtol=0, atol=1e-13)
        trie = O.build_trie(inp["labels"], inp["root_token"], model.cfg.V)
        lp = O.edge_logprobs(model, trie, np.zeros((1, trie.n_int, model.cfg.d)),
                             np.full((1, trie.n_int), np.log(model.cfg.V)))
        np.testing.assert_allclose(lp[0, 1:], -np.log(model.cfg.V), rtol=0, atol=1e-13)
        assert lp[0, 0] == 0.0


def test_lse_matches_scipy():
    for dtype, head in (("f32", "same"), ("bf16", "fp8")):
        inp, model = _tiny_model(dtype, head)
        rng = np.random.default_rng(5)
        h = rng.standard_normal((9, model.cfg.d)) * 3
        z = h @ model.W.T
        if head == "fp8":
            z = z * model.W_scale[None, :]
        np.testing.assert_allclose(O.lm_head_lse(model, h, chunk=4),
                                   scipy.special.logsumexp(z, axis=1), rtol=1e-14, atol=1e-12)


def test_fp8_head_equals_dequantised_matrix():
    inp, model = _tiny_model("bf16", "fp8")
    rng = np.random.default_rng(6)
    h = rng.standard_normal((4, model.cfg.d))
    deq = O.decode_e4m3(inp["W"]) * inp["W_scale"][:, None].astype(np.float64)
    np.testing.assert_allclose(O.head_logits_at(model, h), h @ deq.T, rtol=1e-12, atol=1e-12)


def test_log1mexp_branches():
    x = np.array([-1e-12, -0.1, -np.log(2.0), -0.9, -5.0, -40.0, 0.0, 1e-3])
    # reference: the series log(1 - e^x) = -sum_k e^{kx}/k, summed in extended precision
    k = np.arange(1, 4001, dtype=np.longdouble)
    want = np.array([-(np.exp(k * np.longdouble(v)) / k).sum() for v in x[:6]], dtype=np.float64)
    got = O.log1mexp(x)
    np.testing.assert_allclose(got[1:6], want[1:6], rtol=1e-14)
    np.testing.assert_allclose(got[0], np.log(1e-12), rtol=1e-9)
    assert got[6] == -np.inf and got[7] == -np.inf


def test_flop_constant_of_the_head():
    """0.78 GFLOP per answer position for the full Qwen3-4B head (cost model, section 4.2)."""
    assert round(2 * 2560 * 151936 / 1e9, 2) == 0.78
