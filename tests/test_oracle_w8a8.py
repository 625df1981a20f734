"""Pins of the oracle's E4M3 activation quantization (reading R12 of the oracle: the
W8A8 head's per-row scale and codes): exact round trips, ties to the even code,
saturation, agreement with the input generator's separately written weight
encoder, and the logit formula on a small case."""
import numpy as np

import oracle as O
from synth import config, make_inputs
from synth.gen import _e4m3_codes


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = O.decode_e4m3(codes)
    back = O.e4m3_encode(vals)
    # +0 and -0 both decode to 0; the sign bit is kept
    np.testing.assert_array_equal(back, codes)


def test_encode_ties_go_to_the_even_code():
    vals = O.decode_e4m3(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    got = O.e4m3_encode(mids).astype(int)
    lo = np.arange(126)
    np.testing.assert_array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    # just off the midpoint the nearer value wins
    np.testing.assert_array_equal(O.e4m3_encode(mids * (1 - 1e-9)).astype(int), lo)
    np.testing.assert_array_equal(O.e4m3_encode(mids * (1 + 1e-9)).astype(int), lo + 1)


def test_encode_saturates_and_keeps_sign():
    assert list(O.e4m3_encode([448.0, 460.0, 1e9, -1e9, -448.0])) == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    # subnormal steps of 2^-9: 0.5 and 1.5 steps are ties (to codes 0 and 2), 0.75 rounds up
    assert list(O.e4m3_encode([2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 3 * 2.0 ** -11, -2.0 ** -6])) == \
        [1, 0, 2, 1, 0x88]


def test_encode_agrees_with_the_weight_generator():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(-500, 500, 20000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 1e-3, 5000)])
    np.testing.assert_array_equal(O.e4m3_encode(x), _e4m3_codes(x))


def test_row_quantization():
    rng = np.random.default_rng(5)
    h = O.round_bf16(rng.normal(0, 1, (40, 256)))
    h[3] = 0.0
    codes, s = O.quantize_rows_e4m3(h)
    assert s[3] == 0 and not codes[3].any()
    live = np.arange(40) != 3
    # the largest magnitude of every row lands on +-448
    big = np.abs(h).argmax(axis=1)
    assert np.all((codes[live, big[live]] & 0x7F) == 0x7E)
    back = O.decode_e4m3(codes) * s[:, None]
    # E4M3 keeps 3 mantissa bits: half a step is at most 2^-4 of the value, and the
    # subnormal half step is 2^-10 in code units (times the row scale)
    bound = np.abs(h) * 2.0 ** -4 + 2.0 ** -10 * s[:, None] + 1e-6 * np.abs(h)
    assert np.all(np.abs(back - h)[live] <= bound[live])


def test_w8a8_logits_formula():
    cfg = config(5, V=300, d=64, Hq=2, Hkv=1, hd=32, B=1, L=4, head="fp8a8")
    inp = make_inputs(cfg, seed=2)
    m = O.OracleModel(inp)
    rng = np.random.default_rng(6)
    h = O.round_bf16(rng.normal(0, 1, (3, 64)))
    z = O.head_logits_at(m, h, cols=[5, 7, 299])
    codes, s = O.quantize_rows_e4m3(h)
    for r in range(3):
        for i, v in enumerate([5, 7, 299]):
            want = s[r] * m.W_scale[v] * float(np.dot(O.decode_e4m3(codes[r]),
                                                      O.decode_e4m3(inp["W"][v])))
            assert abs(z[r, i] - want) <= 1e-12 * max(1.0, abs(want))


def test_w8a8_trie_pass_matches_sequence_scoring():
    """The whole trie pass with the W8A8 head equals per-label causal scoring, each
    answer position's hidden row quantized on its own."""
    cfg = config(5, V=400, d=64, Hq=4, Hkv=1, hd=32, B=2, L=30, head="fp8a8")
    inp = make_inputs(cfg, seed=3)
    res = O.classify(inp)
    for b in range(cfg.B):
        np.testing.assert_allclose(res["ll"][b], O.bruteforce_ll(inp, b), rtol=1e-10, atol=1e-12)
    # and it differs from the W8A16 head on the same weights
    ref = O.classify(dict(inp, cfg=cfg.replace(head="fp8")))
    assert np.abs(ref["ll"] - res["ll"]).max() > 1e-6
