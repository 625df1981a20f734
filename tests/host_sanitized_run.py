"""Body of the host sanitizer test (run in a child process that preloads the ASan
runtime; not collected by pytest).  Loads the host-only library built with ASan +
UBSan and drives tcs_trie_build and tcs_decision_truncate through the configs'
label sets, random label sets, every error path and short output capacities,
checking results against the oracle.  Any memory error or undefined behaviour
aborts the process; the last line printed is SANITIZED_OK."""
import ctypes as C
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import trie_constrained_scoring_amd as tcs  # noqa: E402
from synth import config, labels_to_csr, make_inputs  # noqa: E402

P32 = tcs.P32


def load(path):
    L = C.CDLL(path)
    L.tcs_last_error.restype = C.c_char_p
    L.tcs_version.restype = C.c_char_p
    L.tcs_trie_build.argtypes = [P32, P32, C.c_int32, C.c_int32, C.c_int32, C.POINTER(tcs.tcs_trie)]
    L.tcs_decision_truncate.argtypes = [P32, P32, C.c_int32, C.c_int32, C.POINTER(C.c_uint8), P32,
                                        P32, P32]
    return L


def same_trie(t, o):
    assert (t.n_nodes, t.n_int, t.n_labels, t.max_depth) == (o.n_nodes, o.n_int, o.n_labels, o.max_depth)
    for n in ("parent", "token", "depth", "child_begin", "child_count", "node_label", "label_node",
              "qrow", "qnode", "qparent", "level_offsets", "e_tok", "e_qrow", "e_child"):
        assert np.array_equal(t.arrays[n], getattr(o, n)), n


def check_build(labels, root, V):
    offs, toks = labels_to_csr(labels)
    # the library checks every token before looking for duplicates
    bad_token = any(t < 0 or t >= V for l in labels for t in l)
    try:
        o = O.build_trie(labels, root, V)
    except O.TrieError as e:
        try:
            tcs.trie_build(offs, toks, root, V)
        except tcs.TcsError as g:
            assert g.code == (tcs.TCS_EINVAL if bad_token else e.code), (g.code, e.code)
            return
        raise AssertionError("library accepted a label set the oracle refuses")
    same_trie(tcs.trie_build(offs, toks, root, V), o)


def check_cut(labels, flags, V):
    offs, toks = labels_to_csr(labels)
    if any(t < 0 or t >= V for l in labels for t in l):
        # the oracle's cut takes no vocabulary size; the library refuses such tokens
        try:
            tcs.decision_truncate(offs, toks, V, flags)
        except tcs.TcsError as g:
            assert g.code == tcs.TCS_EINVAL
            return
        raise AssertionError("library cut labels with tokens outside [0, V)")
    try:
        d = O.decision_depths(labels, flags)
    except O.TrieError as e:
        try:
            tcs.decision_truncate(offs, toks, V, flags)
        except tcs.TcsError as g:
            assert g.code == e.code
            return
        raise AssertionError("library cut a label set the oracle refuses")
    c_offs, c_toks, c_depth = tcs.decision_truncate(offs, toks, V, flags)
    assert np.array_equal(c_depth, d)
    o_offs, o_toks = labels_to_csr(O.truncate_labels(labels, d))
    assert np.array_equal(c_offs, o_offs) and np.array_equal(c_toks, o_toks)


def short_capacities(L):
    """Every capacity from 1 up to the needed one: the call must report the sizes and
    write nothing past the given arrays (ASan checks the writes)."""
    labels = [[1, 2, 3, 4], [1, 2, 5], [6], [6, 7, 8, 9, 2]]
    offs, toks = labels_to_csr(labels)
    o = O.build_trie(labels, 0, 10)
    names = [f for f, _ in tcs.tcs_trie._fields_[6:] if f not in ("max_decode_steps", "max_children")]
    for cap in range(1, o.n_nodes + 1):
        for levels in range(1, o.max_depth + 3):
            bufs = {n: np.zeros(cap if n not in ("level_offsets", "row_level_offsets") else levels,
                                np.int32) for n in names}
            bufs["label_node"] = np.zeros(len(labels), np.int32)
            bufs["label_row"] = np.zeros(len(labels), np.int32)
            t = tcs.tcs_trie(cap_nodes=cap, cap_levels=levels)
            for n, b in bufs.items():
                setattr(t, n, b.ctypes.data_as(P32))
            rc = L.tcs_trie_build(offs.ctypes.data_as(P32), toks.ctypes.data_as(P32), len(labels), 0,
                                  10, C.byref(t))
            if cap >= o.n_nodes and levels >= o.max_depth + 2:
                assert rc == tcs.TCS_OK
            else:
                assert rc == tcs.TCS_ECAPACITY, (cap, levels, rc)
                assert t.n_nodes == o.n_nodes and t.max_depth == o.max_depth


def main(path):
    L = load(path)
    tcs._lib_handle = L  # the binding's host calls now go to the sanitized library
    assert b"gfx950" in L.tcs_version()
    for cid in (1, 2, 3, 4):
        inp = make_inputs(config(cid), weights=False)
        check_build(inp["labels"], inp["root_token"], config(cid).V)
        check_cut(inp["labels"], inp["word_cont"], config(cid).V)
    rng = np.random.default_rng(2024)
    for _ in range(400):
        V = int(rng.integers(2, 12))
        M = int(rng.integers(1, 30))
        labels = [[int(t) for t in rng.integers(-1 if rng.random() < 0.02 else 0,
                                                V + (1 if rng.random() < 0.02 else 0),
                                                int(rng.integers(1, 8)))] for _ in range(M)]
        if rng.random() < 0.1:
            labels.append(list(labels[0]))       # a duplicate
        root = int(rng.integers(0, V))
        check_build(labels, root, V)
        check_cut(labels, (rng.random(V) < 0.3).astype(np.uint8), V)
    # empty label, M = 0, null pointers
    for offs, toks, M in ((np.array([0, 1, 1], np.int32), np.array([3], np.int32), 2),
                          (np.array([0], np.int32), np.zeros(1, np.int32), 0)):
        t = tcs.tcs_trie(cap_nodes=4, cap_levels=4)
        assert L.tcs_trie_build(offs.ctypes.data_as(P32), toks.ctypes.data_as(P32), M, 0, 10,
                                C.byref(t)) == tcs.TCS_EINVAL
    assert L.tcs_trie_build(None, None, 1, 0, 10, None) == tcs.TCS_EINVAL
    assert L.tcs_decision_truncate(None, None, 1, 10, None, None, None, None) == tcs.TCS_EINVAL
    short_capacities(L)
    print("SANITIZED_OK", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
