"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host trie builder matches the oracle bit for bit."""
import ctypes as C
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O
import trie_constrained_scoring_amd as tcs
from synth import config, labels_to_csr, make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tcs.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tcs_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = tcs.lib()
    names = declared_functions()
    assert "tcs_classify" in names and "tcs_trie_build" in names
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert "gfx950" in tcs.version()


ARRAYS = ["parent", "token", "depth", "child_begin", "child_count", "node_label", "label_node",
          "qrow", "qnode", "qparent", "level_offsets", "e_tok", "e_qrow", "e_child"]


def assert_same_trie(t, o):
    assert (t.n_nodes, t.n_int, t.n_labels, t.max_depth) == (o.n_nodes, o.n_int, o.n_labels, o.max_depth)
    for n in ARRAYS:
        np.testing.assert_array_equal(t.arrays[n], getattr(o, n), err_msg=n)
    # derived arrays for the level-by-level path sums, from their definitions:
    # rows at depth < d, and the row a label's score starts from
    row_depth = o.depth[o.qnode]
    np.testing.assert_array_equal(
        t.arrays["row_level_offsets"], [int(np.sum(row_depth < d)) for d in range(o.max_depth + 2)])
    u = o.label_node
    np.testing.assert_array_equal(
        t.arrays["label_row"], np.where(o.child_count[u] > 0, o.qrow[u], o.qrow[o.parent[u]]))


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_trie_build_matches_oracle_on_configs(cid):
    inp = make_inputs(config(cid), weights=False) if cid != 5 else make_inputs(
        config(5, B=1, L=1), weights=False)
    V = config(cid).V
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], V)
    assert_same_trie(t, O.build_trie(inp["labels"], inp["root_token"], V))


@settings(max_examples=300, deadline=None)
@given(st.lists(st.lists(st.integers(0, 6), min_size=1, max_size=7), min_size=1, max_size=30),
       st.integers(0, 9))
def test_trie_build_matches_oracle_random(raw, root):
    V = 10
    try:
        o = O.build_trie(raw, root, V)
    except O.TrieError as e:
        offs, toks = labels_to_csr(raw)
        with pytest.raises(tcs.TcsError) as ei:
            tcs.trie_build(offs, toks, root, V)
        assert ei.value.code == e.code
        return
    offs, toks = labels_to_csr(raw)
    assert_same_trie(tcs.trie_build(offs, toks, root, V), o)


def test_trie_build_errors():
    def code(labels, root=0, V=10, offs=None, toks=None):
        if offs is None:
            offs, toks = labels_to_csr(labels)
        with pytest.raises(tcs.TcsError) as e:
            tcs.trie_build(offs, toks, root, V)
        return e.value.code
    assert code([[1, 2], [1, 2]]) == tcs.TCS_EDUPLICATE
    assert code([[1, 12]]) == tcs.TCS_EINVAL
    assert code([[1, -1]]) == tcs.TCS_EINVAL
    assert code([[1]], root=10) == tcs.TCS_EINVAL
    assert code(None, offs=np.array([0, 1, 1], np.int32), toks=np.array([3], np.int32)) == tcs.TCS_EINVAL
    assert code(None, offs=np.array([0], np.int32), toks=np.zeros(0, np.int32)) == tcs.TCS_EINVAL


def test_trie_build_capacity_report():
    lib = tcs.lib()
    offs, toks = labels_to_csr([[1, 2, 3], [1, 4], [5]])
    bufs = [np.zeros(3, np.int32) for _ in range(14)]
    t = tcs.tcs_trie(cap_nodes=3, cap_levels=2)
    for n, b in zip([f for f, _ in tcs.tcs_trie._fields_[6:]], bufs):
        setattr(t, n, b.ctypes.data_as(tcs.P32))
    rc = lib.tcs_trie_build(offs.ctypes.data_as(tcs.P32), toks.ctypes.data_as(tcs.P32), 3, 0, 8, C.byref(t))
    assert rc == tcs.TCS_ECAPACITY
    assert t.n_nodes == 6 and t.max_depth == 3 and t.n_int == 3


def test_null_pointer_errors_without_gpu():
    lib = tcs.lib()
    assert lib.tcs_trie_build(None, None, 1, 0, 10, None) == tcs.TCS_EINVAL
    assert b"null" in lib.tcs_last_error()
    assert lib.tcs_tree_attn(None, tcs.TCS_BF16, 1, 1, 4, 2, 96, *([None] * 7), 1.0, None, None, 0) == \
        tcs.TCS_EUNSUPPORTED
    assert lib.tcs_tree_attn(None, tcs.TCS_BF16, 1, 1, 4, 3, 128, *([None] * 7), 1.0, None, None, 0) == \
        tcs.TCS_EINVAL
    assert lib.tcs_lmhead_lse_gather(None, tcs.TCS_BF16, tcs.TCS_F32, 1, 1, 2, 64, 10, *([None] * 9), 0) == \
        tcs.TCS_EUNSUPPORTED
    assert lib.tcs_lmhead_lse_gather(None, tcs.TCS_BF16, tcs.TCS_BF16, 1, 1, 2, 100, 10, *([None] * 9), 0) == \
        tcs.TCS_EUNSUPPORTED
    assert lib.tcs_path_sum_softmax(None, 1, None, None, None, None, None) == tcs.TCS_EINVAL
    assert lib.tcs_classify(None, None, None, None, None, None, None, None, 0) == tcs.TCS_EINVAL


def test_path_sum_rejects_null_qparent_without_gpu():
    """A trie struct whose qparent is NULL is refused before any launch, also when the
    optional level-by-level arrays are set (that kernel reads qparent)."""
    lib = tcs.lib()
    labels = [[i, i + 1] for i in range(2, 1400, 2)]   # > 512 labels: level-by-level sums
    t = tcs.trie_build(*labels_to_csr(labels), 0, 2000)
    fake = 256   # never dereferenced: the call fails before launching
    dev = tcs.tcs_trie_dev(n_nodes=t.n_nodes, n_int=t.n_int, n_labels=t.n_labels,
                           max_depth=t.max_depth, **{n: fake for n in tcs.TRIE_DEV_ARRAYS})
    dev.qparent = None
    rc = lib.tcs_path_sum_softmax(None, 2, C.byref(dev), fake, fake, fake, fake)
    assert rc == tcs.TCS_EINVAL and b"null" in lib.tcs_last_error()


def test_lmhead_workspace_query_by_dtype_pair():
    """The head's workspace size depends on the (h, W) dtype pair: a W8A8 head also
    holds the hidden rows' E4M3 codes (1 byte each) and scales; unsupported pairs give 0."""
    lib = tcs.lib()
    B, n_int, n_nodes, d, V = 4, 8, 18, 256, 1000
    bf = lib.tcs_lmhead_workspace_bytes(tcs.TCS_BF16, tcs.TCS_BF16, B, n_int, n_nodes, d, V)
    w8 = lib.tcs_lmhead_workspace_bytes(tcs.TCS_BF16, tcs.TCS_FP8_E4M3, B, n_int, n_nodes, d, V)
    a8 = lib.tcs_lmhead_workspace_bytes(tcs.TCS_BF16, tcs.TCS_FP8_E4M3_A8, B, n_int, n_nodes, d, V)
    assert bf > 0 and w8 == bf and a8 >= bf + B * n_int * (d + 4)
    assert lib.tcs_lmhead_workspace_bytes(tcs.TCS_F32, tcs.TCS_FP8_E4M3, B, n_int, n_nodes, d, V) == 0
    assert lib.tcs_lmhead_workspace_bytes(tcs.TCS_F32, tcs.TCS_FP8_E4M3_A8, B, n_int, n_nodes, d, V) == 0
    assert lib.tcs_lmhead_lse_gather(None, tcs.TCS_F32, tcs.TCS_FP8_E4M3_A8, 1, 1, 2, 64, 10,
                                     *([None] * 9), 0) == tcs.TCS_EUNSUPPORTED
    # the W8A8 head steps over 128 codes of d at a time: d = 192 is refused before any
    # pointer is touched
    assert lib.tcs_lmhead_lse_gather(None, tcs.TCS_BF16, tcs.TCS_FP8_E4M3_A8, 1, 1, 2, 192, 10,
                                     *([None] * 9), 0) == tcs.TCS_EUNSUPPORTED
    assert b"128" in lib.tcs_last_error()


def test_tree_attn_noalloc_refuses_oversize_without_gpu():
    """tcs_tree_attn_noalloc checks its sizes before any HIP call: scratch beyond the
    built-in array is refused with TCS_ECAPACITY (pointers are never dereferenced)."""
    lib = tcs.lib()
    fake = C.c_void_p(256)
    n_ok = 1
    while tcs.tree_attn_workspace_bytes(n_ok + 1, 32, 128) <= tcs.NOALLOC_SCRATCH_BYTES:
        n_ok += 1
    assert n_ok >= 1000
    rc = lib.tcs_tree_attn_noalloc(None, tcs.TCS_BF16, 1, n_ok + 1, 32, 8, 128, *([fake] * 7), 1.0, fake)
    assert rc == tcs.TCS_ECAPACITY and b"scratch" in lib.tcs_last_error()
    assert lib.tcs_tree_attn_noalloc(None, tcs.TCS_BF16, 1, 4, 4, 2, 96, *([fake] * 7), 1.0, fake) == \
        tcs.TCS_EUNSUPPORTED
    assert lib.tcs_tree_attn_noalloc(None, tcs.TCS_BF16, 1, 4, 4, 2, 128, *([None] * 7), 1.0, None) == \
        tcs.TCS_EINVAL


def test_timing_api_without_launches():
    tcs.timing_enable(True)
    assert tcs.timing_read(tcs.TCS_TIMER_HEAD) == (0.0, 0)
    assert tcs.timing_read(tcs.TCS_TIMER_DOC_ATTN) == (0.0, 0)
    with pytest.raises(tcs.TcsError):
        tcs.timing_read(7)
    lib = tcs.lib()
    assert lib.tcs_timing_read(0, None, None) == tcs.TCS_EINVAL
    tcs.timing_enable(False)


# ------------------------------------------------------------ decision-word cut

def assert_same_cut(labels, flags, V):
    offs, toks = labels_to_csr(labels)
    c_offs, c_toks, c_depth = tcs.decision_truncate(offs, toks, V, flags)
    d = O.decision_depths(labels, flags)
    np.testing.assert_array_equal(c_depth, d)
    cut_o, cut_t = labels_to_csr(O.truncate_labels(labels, d))
    np.testing.assert_array_equal(c_offs, cut_o)
    np.testing.assert_array_equal(c_toks, cut_t)


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_decision_truncate_matches_oracle_on_configs(cid):
    inp = make_inputs(config(cid), weights=False)
    assert_same_cut(inp["labels"], inp["word_cont"], config(cid).V)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.lists(st.integers(0, 6), min_size=1, max_size=7), min_size=1, max_size=30),
       st.lists(st.integers(0, 1), min_size=10, max_size=10))
def test_decision_truncate_matches_oracle_random(raw, flags):
    V = 10
    flags = np.array(flags, dtype=np.uint8)
    try:
        O.decision_depths(raw, flags)
    except O.TrieError as e:
        offs, toks = labels_to_csr(raw)
        with pytest.raises(tcs.TcsError) as ei:
            tcs.decision_truncate(offs, toks, V, flags)
        assert ei.value.code == e.code
        return
    assert_same_cut(raw, flags, V)


def test_decision_truncate_errors():
    lib = tcs.lib()
    z = np.zeros(10, np.uint8)

    def code(labels, offs=None, toks=None, V=10):
        if offs is None:
            offs, toks = labels_to_csr(labels)
        with pytest.raises(tcs.TcsError) as e:
            tcs.decision_truncate(offs, toks, V, np.zeros(V, np.uint8))
        return e.value.code
    assert code([[1, 2], [3], [1, 2]]) == tcs.TCS_EDUPLICATE
    assert code([[1, 10]]) == tcs.TCS_EINVAL
    assert code(None, offs=np.array([0, 1, 1], np.int32), toks=np.array([3], np.int32)) == tcs.TCS_EINVAL
    assert code(None, offs=np.array([0], np.int32), toks=np.zeros(0, np.int32)) == tcs.TCS_EINVAL
    offs, toks = labels_to_csr([[1, 2]])
    out = np.zeros(3, np.int32)
    P = lambda a: a.ctypes.data_as(tcs.P32)
    assert lib.tcs_decision_truncate(P(offs), P(toks), 1, 10, None, P(out), P(out), None) == \
        tcs.TCS_EINVAL
    assert b"null" in lib.tcs_last_error()
    flags = z.ctypes.data_as(C.POINTER(C.c_uint8))
    assert lib.tcs_decision_truncate(P(offs), P(toks), 1, 10, flags, None, P(out), None) == \
        tcs.TCS_EINVAL
    # depth may be NULL
    o2, t2 = np.zeros(2, np.int32), np.zeros(2, np.int32)
    assert lib.tcs_decision_truncate(P(offs), P(toks), 1, 10, flags, P(o2), P(t2), None) == tcs.TCS_OK
    assert list(o2) == [0, 1] and t2[0] == 1


def test_letters_rejects_deeper_tries_without_gpu():
    """tcs_letters_run checks the trie before touching any device memory: a label of
    two tokens is refused (the pointers below are never dereferenced)."""
    lib = tcs.lib()
    assert lib.tcs_letters_run(None, None, None, None, None, None, None, None, None, 0) == tcs.TCS_EINVAL
    t = tcs.trie_build(*labels_to_csr([[3], [4, 5]]), 0, 16)
    fake = 256
    dev = tcs.tcs_trie_dev(n_nodes=t.n_nodes, n_int=t.n_int, n_labels=t.n_labels,
                           max_depth=t.max_depth,
                           **{n: fake for n in tcs.TRIE_DEV_ARRAYS})
    model = tcs.tcs_model(dtype=tcs.TCS_BF16, head_dtype=tcs.TCS_BF16, d=128, Hq=2, Hkv=1, hd=128,
                          V=16, eps=1e-6, E=fake, Wq=fake, Wk=fake, Wv=fake, Wo=fake, W=fake)
    docs = tcs.tcs_docs(B=1, total_tokens=4, doc_offsets=fake, Kd=fake, Vd=fake)
    rc = lib.tcs_letters_run(None, C.byref(model), C.byref(dev), C.byref(docs), None, None, None,
                             None, None, 0)
    assert rc == tcs.TCS_EINVAL and b"one-token" in lib.tcs_last_error()


# ------------------------------------------------------------ greedy-decoding tables

def assert_decode_tables(labels, t):
    """sub_label, dec_node and max_decode_steps against their definitions, with each
    node named by its token path."""
    labels = [tuple(l) for l in labels]
    below = {}
    for m, l in enumerate(labels):
        for k in range(len(l) + 1):
            below.setdefault(l[:k], []).append(m)
    path = [()] * t.n_nodes
    for u in range(1, t.n_nodes):
        path[u] = path[t.parent[u]] + (int(t.token[u]),)
    for u in range(t.n_nodes):
        ms = below[path[u]]
        assert t.sub_label[u] == (ms[0] if len(ms) == 1 else -1), u
        w = u
        while t.child_count[w] == 1 and len(below[path[w]]) > 1:
            w = t.child_begin[w]
        assert t.dec_node[u] == w, u
    most = 0
    for m, l in enumerate(labels):
        if any(l2[:len(l)] == l and len(l2) > len(l) for l2 in labels):
            continue  # never returned by greedy decoding
        most = max(most, O.greedy_walk(labels, lambda p, c, l=l: l[len(p)])[1])
    assert t.max_decode_steps == most
    assert t.max_children == max(int(c) for c in t.child_count)


@pytest.mark.parametrize("cid", [1, 2, 3, 4])
def test_decode_tables_on_configs(cid):
    inp = make_inputs(config(cid), weights=False)
    t = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], config(cid).V)
    assert_decode_tables(inp["labels"], t)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.lists(st.integers(0, 5), min_size=1, max_size=6), min_size=1, max_size=25,
                unique_by=tuple))
def test_decode_tables_random(raw):
    offs, toks = labels_to_csr(raw)
    assert_decode_tables(raw, tcs.trie_build(offs, toks, 0, 8))


def test_decode_run_errors_without_gpu():
    lib = tcs.lib()
    assert lib.tcs_decode_run(None, None, None, None, None, None, None, None, 0) == tcs.TCS_EINVAL
    t = tcs.trie_build(*labels_to_csr([[3], [4, 5]]), 0, 16)
    fake = 256
    arrays = {n: fake for n in tcs.TRIE_DEV_ARRAYS}
    arrays["dec_node"] = None
    dev = tcs.tcs_trie_dev(n_nodes=t.n_nodes, n_int=t.n_int, n_labels=t.n_labels,
                           max_depth=t.max_depth, max_decode_steps=t.max_decode_steps,
                           max_children=t.max_children, **arrays)
    model = tcs.tcs_model(dtype=tcs.TCS_BF16, head_dtype=tcs.TCS_BF16, d=128, Hq=2, Hkv=1, hd=128,
                          V=16, eps=1e-6, E=fake, Wq=fake, Wk=fake, Wv=fake, Wo=fake, W=fake)
    docs = tcs.tcs_docs(B=1, total_tokens=4, doc_offsets=fake, Kd=fake, Vd=fake)
    assert lib.tcs_decode_workspace_bytes(C.byref(model), C.byref(dev), C.byref(docs)) == 0
    rc = lib.tcs_decode_run(None, C.byref(model), C.byref(dev), C.byref(docs), None, None, None,
                            None, 0)
    assert rc == tcs.TCS_EINVAL and b"dec_node" in lib.tcs_last_error()
    dev.dec_node = fake
    model.hd, model.Hq = 64, 4
    assert lib.tcs_decode_run(None, C.byref(model), C.byref(dev), C.byref(docs), None, None, None,
                              None, 0) == tcs.TCS_EUNSUPPORTED
