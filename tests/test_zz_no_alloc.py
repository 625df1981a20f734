"""tcs_tree_attn_noalloc, the tree-attention entry point that allocates nothing:
its scratch (the per-(row, head) path partials) lives in the library's own per-GPU
device array.  It must give tcs_tree_attn's output bit for bit (same kernels), for
calls in a row that reuse the array: first at the largest size the array holds,
then on a smaller input; one row more than fits is refused before any launch."""
import ctypes as C

import numpy as np
import pytest

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, labels_to_csr, make_inputs
from tests.gpu_util import say, to_bf16_exact

pytestmark = pytest.mark.gpu


def _inputs(labels, Hq, Hkv, hd, lens, seed):
    cfg = config(2, V=5000, d=64, Hq=Hq, Hkv=Hkv, hd=hd, trie=("explicit", labels), doc_lens=lens)
    inp = make_inputs(cfg, seed=seed, weights=False)
    trie = O.build_trie(inp["labels"], inp["root_token"], cfg.V)
    rng = np.random.default_rng(seed)
    n = trie.n_int
    qn = O.round_bf16(rng.standard_normal((n, Hq, hd)))
    kn = O.round_bf16(rng.standard_normal((n, Hkv, hd)))
    vn = O.round_bf16(rng.standard_normal((n, Hkv, hd)))
    return cfg, inp, trie, qn, kn, vn


def _both(cfg, inp, qn, kn, vn):
    """(tcs_tree_attn output, tcs_tree_attn_noalloc output) on the same inputs."""
    import torch
    conv = lambda a: to_bf16_exact(a).cuda()
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(t)
    args = (conv(qn), conv(kn), conv(vn), conv(O.decode_bf16(inp["Kd"])), conv(O.decode_bf16(inp["Vd"])),
            torch.from_numpy(inp["doc_offsets"]).cuda(), td["qparent"], 1.0 / np.sqrt(cfg.hd))
    ref = tcs.tree_attn(*args)
    got = tcs.tree_attn_noalloc(*args)
    torch.cuda.synchronize()
    return ref.view(torch.int16).cpu().numpy(), got.view(torch.int16).cpu().numpy()


def _max_rows(Hq, hd):
    n = 1
    while tcs.tree_attn_workspace_bytes(n + 1, Hq, hd) <= tcs.NOALLOC_SCRATCH_BYTES:
        n += 1
    return n


def test_noalloc_equals_workspace_entry_point(dev):
    Hq, Hkv, hd = 32, 8, 128
    n_max = _max_rows(Hq, hd)
    # a root with n_max - 1 internal children, each with two leaf children: n_max rows
    labels = [[100 + a, b] for a in range(n_max - 1) for b in (1, 2)]
    cfg, inp, trie, qn, kn, vn = _inputs(labels, Hq, Hkv, hd, (0, 37, 130), seed=61)
    assert trie.n_int == n_max
    say(f"noalloc: call 1, n_int={trie.n_int} (the most the scratch holds), B=3")
    ref, got = _both(cfg, inp, qn, kn, vn)
    np.testing.assert_array_equal(got, ref)

    # one row more than fits: refused on the host, nothing launched
    big = labels + [[9, 1], [9, 2]]
    cfg2, inp2, trie2, *_ = _inputs(big, Hq, Hkv, hd, (5,), seed=62)
    assert trie2.n_int == n_max + 1
    lib = tcs.lib()
    fake = C.c_void_p(256)
    rc = lib.tcs_tree_attn_noalloc(None, tcs.TCS_BF16, 1, trie2.n_int, Hq, Hkv, hd, *([fake] * 7),
                                   1.0, fake)
    assert rc == tcs.TCS_ECAPACITY and b"scratch" in lib.tcs_last_error()

    # a smaller input on the same scratch: the running example, ragged documents
    cfg3 = config(2, V=5000, d=64, Hq=16, Hkv=4, hd=128, doc_lens=(3, 0, 300, 64))
    inp3 = make_inputs(cfg3, seed=63, weights=False)
    trie3 = O.build_trie(inp3["labels"], inp3["root_token"], cfg3.V)
    rng = np.random.default_rng(63)
    qn3 = O.round_bf16(rng.standard_normal((trie3.n_int, 16, 128)))
    kn3 = O.round_bf16(rng.standard_normal((trie3.n_int, 4, 128)))
    vn3 = O.round_bf16(rng.standard_normal((trie3.n_int, 4, 128)))
    say(f"noalloc: call 2, n_int={trie3.n_int}, B=4")
    ref3, got3 = _both(cfg3, inp3, qn3, kn3, vn3)
    np.testing.assert_array_equal(got3, ref3)
    # and the oracle on that input (one bf16 ulp, as the tree-attention tests)
    import torch
    want = O.round_bf16(O.tree_attention(qn3, kn3, vn3, trie3, O.decode_bf16(inp3["Kd"]),
                                         O.decode_bf16(inp3["Vd"]), inp3["doc_offsets"],
                                         1.0 / np.sqrt(128)))
    g = torch.from_numpy(got3).view(torch.bfloat16).to(torch.float64).numpy()
    ulp = np.ldexp(1.0, np.frexp(np.abs(want) + 1e-30)[1] - 8)
    assert (np.maximum(np.abs(g - want) - 4e-6, 0.0) / ulp).max() <= 1.0
    say("noalloc: both calls equal tcs_tree_attn bit for bit")
