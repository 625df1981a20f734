"""Write the full-size oracle goldens of the 255- and 5,000-label workloads.

    python tests/golden/make_full_size_goldens.py [--check]

For the seeded 255-label workload (B = 32 documents of 1,024 tokens, Qwen3-4B
shapes) and the 5,000-label workload (B = 8 documents of 256 tokens) this runs the
whole fp64 oracle pass (`oracle.classify`: tree attention, projection, the
full-vocabulary head and log-sum-exp, path sums, label softmax) on a few documents
of each batch and stores every label's log-likelihood and the chosen label.  The
255-label workload is also stored in the decision-word form ("To Classify, Try a
Trie Tree", section 3.2), scored on the oracle's own cut of the labels.

Only `oracle/` and the seeded input generator are called.  Each file records a
SHA-256 fingerprint of the inputs it was computed from (labels, weights and the
listed documents' keys/values), so a test that regenerates the inputs can first
check it has the same ones.  --check recomputes and compares instead of writing.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
from synth import config, make_inputs  # noqa: E402

# (file name, workload id, documents, form)
GOLDENS = [
    ("classify_max_label_set_255.json", 3, [0, 1, 16, 31], "full"),
    ("classify_max_label_set_255_decision_words.json", 3, [0, 1, 16, 31], "decision"),
    ("classify_large_finite_set_5000.json", 4, [0, 1, 4, 7], "full"),
]


def fingerprint(inp: dict, docs) -> str:
    """SHA-256 over the label set, the root token, every weight array and the listed
    documents' keys/values (or tokens)."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(inp["label_offsets"], dtype=np.int32).tobytes())
    h.update(np.ascontiguousarray(inp["label_tokens"], dtype=np.int32).tobytes())
    h.update(np.int64(inp["root_token"]).tobytes())
    h.update(np.ascontiguousarray(inp["word_cont"]).tobytes())
    for k in ("E", "Wq", "Wk", "Wv", "Wo", "W", "W_scale"):
        if inp.get(k) is not None:
            h.update(np.ascontiguousarray(inp[k]).tobytes())
    offs = inp["doc_offsets"]
    for b in docs:
        for k in ("Kd", "Vd", "doc_tokens"):
            if k in inp:
                h.update(np.ascontiguousarray(inp[k][offs[b]:offs[b + 1]]).tobytes())
    return h.hexdigest()


def oracle_trie(inp: dict, form: str):
    if form == "full":
        return O.build_trie(inp["labels"], inp["root_token"], inp["cfg"].V)
    d = O.decision_depths(inp["labels"], inp["word_cont"])
    return O.build_trie(O.truncate_labels(inp["labels"], d), inp["root_token"], inp["cfg"].V)


def compute(cid: int, docs, form: str, inp=None) -> dict:
    inp = inp if inp is not None else make_inputs(config(cid))
    trie = oracle_trie(inp, form)
    t0 = time.time()
    o = O.classify(inp, docs=docs, trie=trie)
    cfg = inp["cfg"]
    return {
        "source": "oracle.classify (fp64), written by tests/golden/make_full_size_goldens.py",
        "workload": cfg.name, "config_id": cid, "seed": inp["seed"],
        "form": "every label scored root to leaf" if form == "full" else
                "decision words: labels cut by oracle.decision_depths",
        "B": cfg.B, "L": cfg.L, "n_labels": trie.n_labels, "n_nodes": trie.n_nodes,
        "n_int": trie.n_int, "docs": list(docs), "fingerprint": fingerprint(inp, docs),
        "oracle_seconds": round(time.time() - t0, 1),
        # 12 significant digits: far below the 2e-2 log-likelihood bar
        "ll": [[float("%.12g" % x) for x in row] for row in o["ll"]],
        "label": [int(x) for x in o["label"]],
    }


def main(check: bool = False) -> int:
    cache = {}
    bad = 0
    for fname, cid, docs, form in GOLDENS:
        if cid not in cache:
            cache = {cid: make_inputs(config(cid))}
        g = compute(cid, docs, form, cache[cid])
        path = os.path.join(HERE, fname)
        if check:
            old = json.load(open(path))
            same = old["fingerprint"] == g["fingerprint"] and old["label"] == g["label"] and \
                np.allclose(old["ll"], g["ll"], rtol=0, atol=1e-9)
            print(f"{fname}: {'same' if same else 'DIFFERS'}", flush=True)
            bad += not same
        else:
            with open(path, "w") as f:
                json.dump(g, f, separators=(",", ":"))
                f.write("\n")
            print(f"{fname}: {g['n_labels']} labels x {len(docs)} docs, oracle {g['oracle_seconds']} s",
                  flush=True)
    return bad


if __name__ == "__main__":
    sys.exit(main(check="--check" in sys.argv))
