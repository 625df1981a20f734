"""Helpers for the GPU parity tests (not collected by pytest)."""
import json
import os
import sys

import numpy as np

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

LL_TOL = 2e-2      # label log-likelihood, absolute
PROB_TOL = 1e-3    # label probability, absolute
GAP = 1e-2         # labels compared only where the oracle's top-2 gap exceeds this


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_bf16_exact(x):
    """fp64 values already rounded to bf16 -> torch bf16 (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), np.asarray(x, dtype=np.float64)), "not bf16 values"
    return t


def check_labels(gpu_ll, gpu_prob, gpu_label, o_ll, o_prob, o_label, what=""):
    """The spec bar: ll within 2e-2, prob within 1e-3, labels exact where the
    oracle's top-2 gap exceeds 1e-2 (elsewhere the GPU's label must still be a
    label whose oracle ll is within the gap of the maximum)."""
    gpu_ll = np.asarray(gpu_ll, dtype=np.float64)
    fin = np.isfinite(o_ll)
    assert np.array_equal(fin, np.isfinite(gpu_ll)), f"{what}: -inf pattern differs"
    err_ll = np.abs(gpu_ll[fin] - o_ll[fin]).max() if fin.any() else 0.0
    assert err_ll <= LL_TOL, f"{what}: ll error {err_ll}"
    if gpu_prob is not None:
        err_p = np.abs(np.asarray(gpu_prob, dtype=np.float64) - o_prob).max()
        assert err_p <= PROB_TOL, f"{what}: prob error {err_p}"
    else:
        err_p = float("nan")
    srt = np.sort(o_ll, axis=1)
    gap = srt[:, -1] - srt[:, -2] if o_ll.shape[1] > 1 else np.full(o_ll.shape[0], np.inf)
    sure = gap > GAP
    assert np.array_equal(np.asarray(gpu_label)[sure], o_label[sure]), f"{what}: labels differ"
    rows = np.arange(o_ll.shape[0])
    lab = np.asarray(gpu_label)
    assert np.all((lab >= 0) & (lab < o_ll.shape[1]))
    assert np.all(o_ll.max(axis=1) - o_ll[rows, lab] <= GAP + LL_TOL)
    say(f"{what}: max |dll| {err_ll:.2e}  max |dP| {err_p:.2e}  labels compared {sure.sum()}/{len(sure)}")
    return err_ll, err_p


def load_golden(name):
    """A stored oracle result under tests/golden (JSON)."""
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def golden_fingerprint(inp, docs):
    """Fingerprint of regenerated inputs, as the golden writer computes it."""
    from tests.golden.make_full_size_goldens import fingerprint
    return fingerprint(inp, docs)
