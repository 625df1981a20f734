"""Throughput of the trie_tree label-scoring pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--extra 3,4]
                    [--no-cpu-baseline] [--no-path-stress] [--no-decision-word] [--no-letters]
                    [--no-decode] [--no-long-document] [--no-shard] [--no-w8a8]
    python bench.py --copy-calibration     # plain copy of known size, for HBM counters
    python bench.py --head-probe --config 3 [--power]  # head alone: workload-like vs constant
                                                       # operands (+ socket power and clocks)

One step is one ``tcs_classify_run`` call over one batch of synthetic documents
(consecutive steps alternate over ``--streams`` HIP streams, default 3, each with its
own run workspace, so one batch's attention and projection can use the CUs the
previous batch's output head leaves idle in its last partial round of tiles):
ancestor-masked tree attention over the documents, output projection + RMSNorm,
the full-vocabulary output head with fused log-sum-exp and child gather, and the
path sums / label softmax / argmax.  Inputs are resident in HBM before timing.
What depends only on the label set is done once per label set and timed
separately: the trie, built on the host (``trie_build_ms``), and
``tcs_classify_prepare`` (node q/k/v, path partials, head gather lists;
``prepare_ms``).

Prints ONE JSON line.  ``value`` is documents classified per second at the
primary workload (default: the running-example shape, 10 labels); the 255- and
5000-label workloads are reported under ``at_labels``, and ``path_roofline`` times the
path-sum kernel alone on 4096 documents of the 5000-label trie (enough bytes to hold
it against HBM).  ``decision_word`` runs the same documents and weights with every
label cut after the word in which its prefix stops being shared (the decision-word form
of trie_tree: fewer query rows, same kernels); the headline scores every label over
its full root-to-leaf path.  ``letters`` runs them under the letters method (one
answer position per document, only the letter rows of the head), ``trie_decode`` under
greedy decoding in the trie (one answer position per undecided document per step).
``long_document`` runs the long-document workload as stated (B = 128 documents of 4,096
tokens, fp8 head weights with bf16 activations), where the document attention streams
2.1 GB of keys and values per batch.
``w8a8`` runs the long-document workload with the hidden rows quantized to E4M3 before
the head (fp8 x fp8 matrix cores; roofline against the 5.0 PFLOP/s fp8 peak).
``shard_of_8`` runs the long-document workload at one GPU's share of an 8-GPU run
(16 of its 128 documents; documents shard over GPUs with no collective).
``roofline`` is for the
dominant kernel (the output head): after the timed steps, the same steps run
again with the head launches bracketed by HIP events on the stream they run on
(the library's tcs_timing_enable hook), and achieved = algorithmic FLOP per
launch / mean launch duration.  ``traffic`` is the HBM bytes per launch measured by the FETCH_SIZE and
WRITE_SIZE counters (scaled by what they read for a plain copy of known size),
read from the profile summary under profiles/ while the kernel's sources still
hash to the value recorded there, else null.  ``cpu_baseline`` times the fp64
oracle on a bounded sample of the same workload on this host's cores.  Before the
``--warmup`` steps of the primary measurement, untimed steps run for ``prewarm_s``
seconds: the GPU runs its first ~10 ms of work after idling ~15% slower.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "documents classified/sec at 10/255/5000 labels; % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 matrix cores
PEAK_HBM_GBS = 8000.0
HEAD_SOURCES = ["gemm_core.h", "k_lmhead.hip", "tcs_device.h"]
HEAD_TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "lmhead_ring_bf16_running_example_B64_traffic.md")
COPY_BYTES = 1 << 30


def head_source_hash() -> str:
    """sha256 over the sources the output-head kernel is compiled from."""
    h = hashlib.sha256()
    for f in HEAD_SOURCES:
        with open(os.path.join(ROOT, "trie_constrained_scoring_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per head launch from the committed counter summary, or None when
    the summary is missing or was taken on other kernel sources."""
    try:
        text = open(HEAD_TRAFFIC_PROFILE).read()
    except OSError:
        return None
    m_hash = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_val or m_hash.group(1) != head_source_hash():
        return None
    return float(m_val.group(1))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(cid: int, streams: int = 1, inp=None, **overrides):
    """Inputs (generated, or `inp` when given: arrays drawn for this workload), the
    trie, device weights and documents, the prepared state and run buffers."""
    import torch
    import trie_constrained_scoring_amd as tcs
    from synth import config, make_inputs
    cfg = config(cid, **overrides)
    if inp is None:
        t0 = time.time()
        inp = make_inputs(cfg)
        log(f"[bench] config {cid} inputs generated in {time.time() - t0:.1f}s")
    else:
        inp = dict(inp, cfg=cfg)
    t0 = time.perf_counter()
    trie = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    trie_ms = (time.perf_counter() - t0) * 1e3
    td = tcs.TrieDevice(trie)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    prep = tcs.Prepared(model, td, docs.B)
    torch.cuda.synchronize()
    prep_ms = (time.perf_counter() - t0) * 1e3
    ws, out = run_buffers(model, td, docs, streams)
    return dict(cfg=cfg, inp=inp, trie=trie, td=td, model=model, docs=docs, ws=ws, out=out,
                trie_ms=trie_ms, prep=prep, prep_ms=prep_ms)


def run_buffers(model, td, docs, streams):
    """One run workspace and output set per batch in flight."""
    import torch
    import trie_constrained_scoring_amd as tcs
    B, M = docs.B, td.trie.n_labels
    ws, out = [], []
    for _ in range(max(1, streams)):
        ws.append(torch.empty(tcs.classify_run_workspace_bytes(model, td, docs), dtype=torch.uint8,
                              device="cuda"))
        out.append(dict(label=torch.empty(B, dtype=torch.int32, device="cuda"),
                        prob=torch.empty((B, M), dtype=torch.float32, device="cuda"),
                        ll=torch.empty((B, M), dtype=torch.float32, device="cuda")))
    torch.cuda.synchronize()
    return ws, out


def decision_word(S, steps, warmup, streams):
    """The same documents and weights scored in the decision-word form: every label
    cut after the word in which its prefix stops being shared (tcs_decision_truncate),
    then the unchanged classify pass on the cut trie."""
    import torch
    import trie_constrained_scoring_amd as tcs
    cfg, inp = S["cfg"], S["inp"]
    t0 = time.perf_counter()
    offs, toks, _ = tcs.decision_truncate(inp["label_offsets"], inp["label_tokens"], cfg.V,
                                          inp["word_cont"])
    trie = tcs.trie_build(offs, toks, inp["root_token"], cfg.V)
    cut_ms = (time.perf_counter() - t0) * 1e3
    td = tcs.TrieDevice(trie)
    prep = tcs.Prepared(S["model"], td, S["docs"].B)
    ws, out = run_buffers(S["model"], td, S["docs"], streams)
    C = dict(S, trie=trie, td=td, prep=prep, ws=ws, out=out)
    sec, kern = run_steps(C, *long_enough(C, steps, warmup))
    f, R = head_flops(C)
    tf = f / (kern["head"] * 1e-3) / 1e12
    B = S["docs"].B
    e = {"config": cfg.id, "docs_per_s": round(B / sec, 2), "ms_per_step": round(sec * 1e3, 4),
         "query_rows": trie.n_int, "query_rows_full_labels": S["trie"].n_int,
         "trie_nodes": trie.n_nodes, "cut_and_build_ms": round(cut_ms, 3),
         "head_tflops": round(tf, 2), "head_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
         "head_ms": round(kern["head"], 4)}
    del C, prep, ws, out, td
    torch.cuda.empty_cache()
    return e


def long_enough(S, steps, warmup, min_s=0.1):
    """(steps, warmup) for a secondary measurement: at least `steps` steps, and as
    many as fill about `min_s` seconds (judged from a short untimed trial), so that
    fast passes are not timed over a millisecond or two; the warmup fills as long
    (the GPU runs the first few milliseconds of work after idling ~15% slower)."""
    import time as _t
    import torch
    trial = S.copy()
    t0 = _t.perf_counter()
    for _ in range(3):
        _one_step(trial)
    torch.cuda.synchronize()
    per = max((_t.perf_counter() - t0) / 3, 1e-6)
    fill = int(min_s / per)
    return max(steps, fill), max(warmup, 10, fill)


def _one_step(S):
    import trie_constrained_scoring_amd as tcs
    if S.get("letters"):
        tcs.letters(S["model"], S["td"], S["docs"], S["prep"], ws=S["ws"][0], **S["out"][0])
    elif S.get("decode"):
        tcs.trie_decode(S["model"], S["td"], S["docs"], S["prep"], ws=S["ws"][0], **S["out"][0])
    else:
        tcs.classify(S["model"], S["td"], S["docs"], ws=S["ws"][0], prepared=S["prep"], **S["out"][0])


PREWARM_S = 0.1  # untimed steps before the warmup steps of the primary measurement


def run_steps(S, steps, warmup, prewarm_s=0.0):
    """Seconds per step over `steps` timed steps (after `warmup` untimed ones; step i
    runs on stream i mod len(S["ws"]) with workspace i mod len(S["ws"])), then the mean
    duration (ms) of the head and document-attention kernel launches over a second
    pass of `steps` identical steps, all on one stream, in which the library brackets
    those launches with HIP events on their stream (recording events costs host time
    per launch, so that pass is kept out of the throughput figure).  With prewarm_s,
    untimed steps run for that long first: after the host-side setup the GPU has
    been idle, and it runs its first ~10 ms of work ~15% slower, which a warmup of a
    few steps (a few ms) would leave inside the timed region."""
    import torch
    import trie_constrained_scoring_amd as tcs

    n = len(S["ws"])
    streams = [torch.cuda.current_stream()] if n == 1 else [torch.cuda.Stream() for _ in range(n)]

    def step(i, k=None):
        k = i % n if k is None else k
        if S.get("letters"):
            tcs.letters(S["model"], S["td"], S["docs"], S["prep"], ws=S["ws"][k], stream=streams[k],
                        **S["out"][k])
        elif S.get("decode"):
            tcs.trie_decode(S["model"], S["td"], S["docs"], S["prep"], ws=S["ws"][k],
                            stream=streams[k], **S["out"][k])
        else:
            tcs.classify(S["model"], S["td"], S["docs"], ws=S["ws"][k], prepared=S["prep"],
                         stream=streams[k], **S["out"][k])
    if prewarm_s > 0:
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < prewarm_s:
            step(i)
            i += 1
            if i % n == 0:
                torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    tcs.timing_enable(True)
    for i in range(steps):
        step(i, 0)
    torch.cuda.synchronize()
    kern = {}
    for name, timer in (("head", tcs.TCS_TIMER_HEAD), ("doc_attn", tcs.TCS_TIMER_DOC_ATTN)):
        ms, n = tcs.timing_read(timer)
        kern[name] = ms / n if n else None
    tcs.timing_enable(False)
    return sec, kern


def head_flops(S):
    """Algorithmic FLOP of one head launch: 2 * rows * d * V, rows = B * internal nodes."""
    R = S["docs"].B * S["td"].trie.n_int
    return 2.0 * R * S["cfg"].d * S["cfg"].V, R


def doc_attn_bytes(S):
    """Algorithmic HBM bytes of one document-attention launch: every document's K
    and V once, the node queries and the per-trie ancestor partials once, the node
    outputs once (bf16 storage, fp32 partials)."""
    cfg, td = S["cfg"], S["td"]
    B, n_int, T = S["docs"].B, td.trie.n_int, int(S["inp"]["doc_offsets"][-1])
    kv = 2 * T * cfg.Hkv * cfg.hd * 2
    q = n_int * cfg.Hq * cfg.hd * 2
    anc = n_int * cfg.Hq * (cfg.hd + 2) * 4
    o = B * n_int * cfg.Hq * cfg.hd * 2
    return kv + q + anc + o


def doc_attn_flops(S):
    """Algorithmic FLOP of one document-attention launch: q.k and p.v for every
    (document, internal node, query head) over the document's keys, 4 hd FLOP per key
    (the path keys are reduced once per label set, in the prepare step)."""
    cfg, td = S["cfg"], S["td"]
    B, n_int, T = S["docs"].B, td.trie.n_int, int(S["inp"]["doc_offsets"][-1])
    return 4.0 * n_int * cfg.Hq * cfg.hd * T


def doc_attn_roofline(S, ms):
    """Roofline of the document attention: HBM-bound below the bf16 ridge
    (2.5 PFLOP/s / 8 TB/s = 312 FLOP/B), matrix-core-bound above it."""
    by, fl = doc_attn_bytes(S), doc_attn_flops(S)
    if fl / by > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
        tf = fl / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_launch": fl, "bytes_per_launch": by,
                "ms_per_launch": round(ms, 4)}
    gbs = by / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": by, "flops_per_launch": fl,
            "ms_per_launch": round(ms, 4)}


def classify_roofline(S, step_ms):
    """Roofline of the whole classify step: the sum over its kernels of each one's
    bound, max(algorithmic FLOP / matrix-core peak, algorithmic bytes / HBM peak),
    against the measured time per batch.  Kernels: document attention, output
    projection (+ residual), RMSNorm, output head (bf16 matrix cores for bf16 and
    fp8 weights, fp8 ones for W8A8, after the rows' quantization), log-sum-exp merge
    of its partials, path sums."""
    cfg, td = S["cfg"], S["td"]
    B, n_int, N, M = S["docs"].B, td.trie.n_int, td.trie.n_nodes, td.trie.n_labels
    R, qd, d, V = B * n_int, cfg.Hq * cfg.hd, cfg.d, cfg.V
    hbm = PEAK_HBM_GBS * 1e9
    def bound_us(flops, nbytes, peak_tflops=PEAK_BF16_TFLOPS):
        return max(flops / (peak_tflops * 1e12), nbytes / hbm) * 1e6
    wbytes = 1 if cfg.head in ("fp8", "fp8a8") else 2
    parts = {
        "doc_attn": bound_us(doc_attn_flops(S), doc_attn_bytes(S)),
        "o_proj": bound_us(2.0 * R * qd * d, R * qd * 2 + d * qd * 2 + R * d * 4),
        "rownorm": bound_us(0, R * d * 4 + R * d * 2),
        "head": bound_us(2.0 * R * d * V, V * d * wbytes + R * d * 2,
                         PEAK_FP8_TFLOPS if cfg.head == "fp8a8" else PEAK_BF16_TFLOPS),
        "lse_merge": bound_us(0, R * 2 * ((V + 255) // 256) * 8 + R * 4),
        "path_sums": bound_us(0, B * (4 * N + 8 * M)),
    }
    if cfg.head == "fp8a8":  # the hidden rows' E4M3 quantization before the head
        parts["quant_rows"] = bound_us(0, R * d * 2 + R * d + R * 4)
    total = sum(parts.values())
    return {"bound_ms": round(total / 1e3, 4), "ms_per_step": round(step_ms, 4),
            "frac": round(total / 1e3 / step_ms, 4),
            "parts_us": {k: round(v, 2) for k, v in parts.items()}}


def letters_measure(S, steps, warmup, streams):
    """The same documents and weights under the letters method (tcs_letters_run): one
    answer position per document and the M letter rows of the head; the document
    attention is then the dominant kernel."""
    import torch
    import trie_constrained_scoring_amd as tcs
    cfg, inp = S["cfg"], S["inp"]
    letters = np.asarray(inp["letters"], dtype=np.int32)
    trie = tcs.trie_build(np.arange(len(letters) + 1, dtype=np.int32), letters, inp["root_token"],
                          cfg.V)
    td = tcs.TrieDevice(trie)
    prep = tcs.Prepared(S["model"], td, S["docs"].B)
    ws, out = run_buffers(S["model"], td, S["docs"], streams)
    C = dict(S, trie=trie, td=td, prep=prep, ws=ws, out=out, letters=True)
    sec, kern = run_steps(C, *long_enough(C, steps, warmup))
    B = S["docs"].B
    e = {"config": cfg.id, "letters": len(letters), "docs_per_s": round(B / sec, 2),
         "ms_per_step": round(sec * 1e3, 4)}
    if kern["doc_attn"]:
        e["doc_attn_roofline"] = doc_attn_roofline(C, kern["doc_attn"])
        e["doc_attn_share_of_step"] = round(kern["doc_attn"] / (sec * 1e3), 4)
    del C, prep, ws, out, td
    torch.cuda.empty_cache()
    return e


def decode_measure(S, steps, warmup, streams):
    """The same documents, weights and trie under trie_decode (tcs_decode_run): greedy
    generation, one answer position per undecided document per step.  The document
    attention re-reads a document's K/V at every step it takes part in; its HBM
    figure counts those bytes (sum over documents of runs x K/V bytes) against the
    summed duration of the step launches."""
    import torch
    import trie_constrained_scoring_amd as tcs
    cfg, inp, docs = S["cfg"], S["inp"], S["docs"]
    B = docs.B
    nbytes = tcs.decode_workspace_bytes(S["model"], S["td"], docs)
    ws = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(max(1, streams))]
    out = [dict(label=torch.empty(B, dtype=torch.int32, device="cuda"),
                runs=torch.empty(B, dtype=torch.int32, device="cuda")) for _ in ws]
    C = dict(S, ws=ws, out=out, decode=True)
    sec, kern = run_steps(C, *long_enough(C, steps, warmup))
    runs = out[0]["runs"].cpu().numpy().astype(np.int64)
    n_steps = S["td"].trie.max_decode_steps
    e = {"config": cfg.id, "docs_per_s": round(B / sec, 2), "ms_per_step": round(sec * 1e3, 4),
         "mean_model_runs_per_doc": round(float(runs.mean()), 4), "decode_steps": n_steps}
    if kern["doc_attn"] and n_steps:
        lens = np.diff(np.asarray(inp["doc_offsets"], dtype=np.int64))
        by = int((runs * lens).sum()) * 2 * cfg.Hkv * cfg.hd * 2
        ms = kern["doc_attn"] * n_steps
        gbs = by / (ms * 1e-3) / 1e9
        e["doc_attn_roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                  "bytes_per_call": by, "ms_per_call": round(ms, 4)}
    del C, ws, out
    torch.cuda.empty_cache()
    return e


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def first_docs(inp, n):
    """The first n documents of a key/value batch (a view of the same arrays)."""
    offs = inp["doc_offsets"][:n + 1]
    return dict(inp, doc_offsets=offs, Kd=inp["Kd"][:offs[-1]], Vd=inp["Vd"][:offs[-1]])


def cpu_baseline(S, budget_s=15.0):
    """The fp64 oracle, as it stands, on a bounded sample of documents."""
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    inp = S["inp"]
    t0 = time.time()
    model = O.OracleModel(inp)
    trie = O.build_trie(inp["labels"], inp["root_token"], S["cfg"].V)
    log(f"[bench] oracle weights decoded in {time.time() - t0:.1f}s")
    t0 = time.perf_counter()
    O.classify(inp, docs=[0], model=model, trie=trie)
    one = time.perf_counter() - t0
    n = int(max(1, min(S["docs"].B, budget_s // max(one, 1e-3))))
    # a whole batch that takes well under the budget is scored again, so that the
    # timed sample is ~10 s or more of CPU work
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.classify(inp, docs=list(range(n)), model=model, trie=trie)
        reps += 1
        dt = time.perf_counter() - t0
        if n < S["docs"].B or dt >= 0.6 * budget_s:
            break
    return {"value": n * reps / dt, "unit": "docs/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{n} of {S['docs'].B} documents of the same batch x {reps} passes, every label, "
                      f"fp64 numpy (BLAS threads = visible cores), {dt:.1f}s"}


def path_stress(cid: int = 4, B: int = 4096, reps: int = 10):
    """tcs_path_sum_softmax alone on many documents of one label set (the 5,000-label
    trie by default), so that the path kernel streams enough bytes to be measured
    against HBM: it reads lp [B, n_nodes] once and writes ll and prob [B, M] and
    label [B].  lp holds edge log-probs drawn in [-12, -2] (the root's is 0)."""
    import torch
    import trie_constrained_scoring_amd as tcs
    from synth import config, make_inputs
    cfg = config(cid)
    inp = make_inputs(cfg, weights=False)
    trie = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(trie)
    N, M = trie.n_nodes, trie.n_labels
    g = torch.Generator(device="cuda").manual_seed(cid)
    lp = torch.rand(B, N, device="cuda", generator=g) * -10.0 - 2.0
    lp[:, 0] = 0.0
    ll = torch.empty(B, M, device="cuda")
    prob = torch.empty(B, M, device="cuda")
    label = torch.empty(B, dtype=torch.int32, device="cuda")
    tcs.path_sum_softmax(lp, td, ll, prob, label)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tcs.path_sum_softmax(lp, td, ll, prob, label)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    nbytes = B * (N * 4 + 2 * M * 4 + 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": "path_levels_kernel",
            "workload": f"{B} documents on the {M}-label trie of config {cid} ({N} nodes)",
            "bytes_per_launch": nbytes, "ms_per_launch": round(ms, 4),
            "timing": "torch.cuda.Event around 10 launches on the current stream"}


def smi_sample(stop, samples, period=0.3):
    """Append (socket power W, mean GFX clock MHz) read by `amd-smi metric` (a child
    process) until `stop` is set."""
    import subprocess
    while not stop.is_set():
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c"], capture_output=True,
                               text=True, timeout=20)
        except (OSError, subprocess.TimeoutExpired):
            return
        pw = re.findall(r"SOCKET_POWER: (\d+) W", r.stdout)
        clk = [float(x) for x in re.findall(r"GFX_\d+:\s+CLK: (\d+) MHz", r.stdout)]
        if pw and clk:
            samples.append((float(pw[0]), sum(clk) / len(clk)))
        stop.wait(period)


def head_probe(cid: int, reps: int = 5, power: bool = False):
    """The output head alone (tcs_lmhead_lse_gather) at a workload's shape, on operands
    drawn like the workload's (unit-RMS rows h, W ~ N(0, 0.02), bf16) and on constant
    operands of the same shape: the gap between the two is the part of the head's
    time that depends on the operand values (matrix-core power), not on the schedule.
    With `power`, the head then runs back to back for ~4 s per operand kind while
    amd-smi samples the socket power and the GFX clocks."""
    import torch
    import trie_constrained_scoring_amd as tcs
    from synth import config, make_inputs
    cfg = config(cid)
    inp = make_inputs(cfg, weights=False)
    trie = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    td = tcs.TrieDevice(trie)
    B, R = cfg.B, cfg.B * trie.n_int
    g = torch.Generator(device="cuda").manual_seed(cid)
    out = {}
    for kind in ("random", "constant"):
        if kind == "random":
            h = torch.randn(R, cfg.d, device="cuda", generator=g).to(torch.bfloat16)
            W = (torch.randn(cfg.V, cfg.d, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
        else:
            h = torch.ones(R, cfg.d, device="cuda", dtype=torch.bfloat16)
            W = torch.full((cfg.V, cfg.d), 0.02, device="cuda", dtype=torch.bfloat16)
        ws = torch.empty(tcs.lmhead_workspace_bytes(B, trie.n_int, trie.n_nodes, cfg.d, cfg.V),
                         dtype=torch.uint8, device="cuda")
        tcs.lmhead_lse_gather(h, W, td, B, ws=ws)
        torch.cuda.synchronize()
        tcs.timing_enable(True)
        for _ in range(reps):
            tcs.lmhead_lse_gather(h, W, td, B, ws=ws)
        torch.cuda.synchronize()
        ms, n = tcs.timing_read(tcs.TCS_TIMER_HEAD)
        tcs.timing_enable(False)
        ms /= n
        tf = 2.0 * R * cfg.d * cfg.V / (ms * 1e-3) / 1e12
        out[kind] = {"ms_per_launch": round(ms, 4), "tflops": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if power:
            import threading
            n_launch = max(20, int(4.0 / (ms * 1e-3)))
            samples, stop = [], threading.Event()
            for _ in range(n_launch):
                tcs.lmhead_lse_gather(h, W, td, B, ws=ws)
            time.sleep(0.5)  # past the ramp
            th = threading.Thread(target=smi_sample, args=(stop, samples))
            th.start()
            torch.cuda.synchronize()
            stop.set()
            th.join()
            if samples:
                out[kind]["socket_power_w"] = round(statistics.mean(p for p, _ in samples), 1)
                out[kind]["gfx_clock_mhz"] = round(statistics.mean(c for _, c in samples), 1)
                out[kind]["power_samples"] = len(samples)
        del h, W, ws
        torch.cuda.empty_cache()
    print(json.dumps({"head_probe": {"config": cid, "rows": R, "d": cfg.d, "V": cfg.V, **out}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # ~0.1 s of timed steps after ~40 ms of warmup on the running example: 20 steps
    # after 3 (9 ms after 1.4 ms) measured ~15% below the steady rate on MI355X
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--batch", type=int, default=None,
                    help="documents per batch (default: the workload's own batch)")
    ap.add_argument("--extra", default="3,4", help="other label-set sizes to report (config ids)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=3,
                    help="batches in flight: consecutive steps alternate over this many HIP streams, "
                         "each with its own run workspace")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (3 launches) and exit")
    ap.add_argument("--head-probe", action="store_true",
                    help="only time the output head alone on workload-like vs constant operands")
    ap.add_argument("--path-stress", action="store_true",
                    help="only time tcs_path_sum_softmax on 4096 documents of the 5000-label trie")
    ap.add_argument("--no-path-stress", action="store_true",
                    help="leave the path-sum stress measurement (path_roofline) out")
    ap.add_argument("--no-decision-word", action="store_true",
                    help="leave the decision-word measurements (labels cut to their deciding word) out")
    ap.add_argument("--head", default=None, choices=["same", "fp8", "fp8a8"],
                    help="output-head kind for the primary workload (default: the workload's own)")
    ap.add_argument("--no-w8a8", action="store_true",
                    help="leave out the long-document workload with the W8A8 head (fp8 activations)")
    ap.add_argument("--no-long-document", action="store_true",
                    help="leave out the long-document workload (B = 128 x 4096, W8A16 head)")
    ap.add_argument("--no-shard", action="store_true",
                    help="leave out the long-document workload at one GPU's share of 8 (B = 16)")
    ap.add_argument("--no-decode", action="store_true",
                    help="leave the trie_decode measurements (greedy decoding in the trie) out")
    ap.add_argument("--no-letters", action="store_true",
                    help="leave the letters measurements (one answer position, letter rows only) out")
    ap.add_argument("--power", action="store_true",
                    help="with --head-probe: also sample socket power and GFX clocks (amd-smi)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); documents shard across GPUs "
              "with no collective, so a multi-GPU figure is not measured here.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)
        return

    if args.head_probe:
        head_probe(args.config, power=args.power)
        return
    if args.path_stress:
        print(json.dumps({"path_roofline": path_stress()}), flush=True)
        return

    over = {"head": args.head} if args.head else {}
    if args.batch:
        over["B"] = args.batch
    S = setup(args.config, args.streams, **over)
    cfg, trie = S["cfg"], S["trie"]
    sec, kern = run_steps(S, args.steps, args.warmup, prewarm_s=PREWARM_S)
    few = max(3, min(args.steps, 20) // 2)  # steps of the slow secondary passes
    B = S["docs"].B
    value = B / sec
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "docs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "prewarm_s": PREWARM_S,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"same": cfg.dtype, "fp8": f"{cfg.dtype} (head weights fp8 e4m3)",
                  "fp8a8": f"{cfg.dtype} (head fp8 e4m3 weights and activations)"}[cfg.head],
        "data": "synthetic (seeded; random weights N(0,0.02), random doc KV N(0,1))",
        "config": {"workload": f"{cfg.name} (config {cfg.id}): B={B} docs x {cfg.L} tokens, "
                               f"{trie.n_labels} labels, {trie.n_nodes} trie nodes "
                               f"({trie.n_int} internal), d={cfg.d}, Hq/Hkv/hd={cfg.Hq}/{cfg.Hkv}/{cfg.hd}, "
                               f"V={cfg.V}",
                   "labels": trie.n_labels, "trie_nodes": trie.n_nodes, "global_batch": B,
                   "seq_len": cfg.L, "parallelism": "none (1 GPU)",
                   "batches_in_flight": len(S["ws"])},
        "trie_nodes_per_s": round(B * trie.n_nodes / sec, 1),
        "trie_build_ms": round(S["trie_ms"], 3),
        "prepare_ms": round(S["prep_ms"], 3),
    }
    flops, R = head_flops(S)
    ach = flops / (kern["head"] * 1e-3) / 1e12
    kname = {"fp8": "lmhead_ring_kernel<true> (fp8 W)",
             "fp8a8": "quant_rows_e4m3_kernel + lmhead_ring_kernel<fp8 W, fp8 h>"}.get(
                 cfg.head, "lmhead_ring_kernel<false> (bf16 W)")
    peak = PEAK_FP8_TFLOPS if cfg.head == "fp8a8" else PEAK_BF16_TFLOPS
    traffic = recorded_traffic() if cfg.id == 2 and cfg.head == "same" else None
    res["roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak,
                       "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                       "traffic": traffic, "kernel": kname, "rows": R,
                       "flops_per_launch": flops, "ms_per_launch": round(kern["head"], 4),
                       "timing": "HIP events around each head launch of a second pass of the same steps"}
    res["head_share_of_step"] = round(kern["head"] / (sec * 1e3), 4)
    if kern["doc_attn"]:
        res["doc_attn_roofline"] = doc_attn_roofline(S, kern["doc_attn"])
    res["classify_roofline"] = classify_roofline(S, sec * 1e3)
    decision, letters, decode = {}, {}, {}
    if not args.no_decision_word:
        decision[cfg.name] = decision_word(S, args.steps, args.warmup, args.streams)
    if not args.no_letters:
        letters[cfg.name] = letters_measure(S, args.steps, args.warmup, args.streams)
    if not args.no_decode:
        decode[cfg.name] = decode_measure(S, args.steps, args.warmup, args.streams)
    extra = {}
    for c in [int(x) for x in args.extra.split(",") if x.strip()]:
        if c == args.config:
            continue
        del S
        torch.cuda.empty_cache()
        S2 = setup(c, args.streams)
        s2, k2 = run_steps(S2, few, 2)
        f2, _ = head_flops(S2)
        tf = f2 / (k2["head"] * 1e-3) / 1e12
        e = {"config": c, "docs_per_s": round(S2["docs"].B / s2, 2), "ms_per_step": round(s2 * 1e3, 3),
             "labels": S2["trie"].n_labels, "trie_nodes": S2["trie"].n_nodes,
             "trie_nodes_per_s": round(S2["docs"].B * S2["trie"].n_nodes / s2, 1),
             "head_tflops": round(tf, 2), "head_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
             "head_ms": round(k2["head"], 4), "prepare_ms": round(S2["prep_ms"], 3)}
        if k2["doc_attn"]:
            e["doc_attn_ms"] = round(k2["doc_attn"], 4)
            e["doc_attn_roofline"] = doc_attn_roofline(S2, k2["doc_attn"])
        e["classify_roofline"] = classify_roofline(S2, s2 * 1e3)
        extra[str(S2["trie"].n_labels)] = e
        if not args.no_decision_word:
            decision[S2["cfg"].name] = decision_word(S2, few, 2, args.streams)
        if not args.no_letters:
            letters[S2["cfg"].name] = letters_measure(S2, few, 2, args.streams)
        if not args.no_decode:
            decode[S2["cfg"].name] = decode_measure(S2, few, 2, args.streams)
        S = S2
    if extra:
        res["at_labels"] = extra
    # the long-document workload (B = 128 x 4,096 tokens) as stated: bf16 activations,
    # fp8 head weights (W8A16); its inputs are drawn once and serve the W8A8 and
    # one-GPU-share passes below as well
    inp5 = None
    if args.config != 5 and not (args.no_long_document and args.no_w8a8 and args.no_shard):
        from synth import config as _config, make_inputs
        del S
        torch.cuda.empty_cache()
        t0 = time.time()
        inp5 = make_inputs(_config(5))
        log(f"[bench] config 5 inputs generated in {time.time() - t0:.1f}s")
        S = None
    if inp5 is not None and not args.no_long_document:
        del S
        torch.cuda.empty_cache()
        S = setup(5, args.streams, inp=inp5)
        sl, kl = run_steps(S, *long_enough(S, few, 10))
        fl, Rl = head_flops(S)
        tf = fl / (kl["head"] * 1e-3) / 1e12
        t5 = S["trie"]
        res["long_document"] = {
            "config": 5, "workload": f"long-document-kv: B={S['docs'].B} docs x {S['cfg'].L} tokens, "
                                     f"{t5.n_labels} labels, fp8 e4m3 head weights + fp32 row scales, "
                                     "bf16 activations (W8A16)",
            "docs_per_s": round(S["docs"].B / sl, 2), "ms_per_step": round(sl * 1e3, 4),
            "trie_nodes_per_s": round(S["docs"].B * t5.n_nodes / sl, 1),
            "head_ms": round(kl["head"], 4), "head_rows": Rl, "head_tflops": round(tf, 2),
            "head_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "head_share_of_step": round(kl["head"] / (sl * 1e3), 4)}
        if kl["doc_attn"]:
            res["long_document"]["doc_attn_roofline"] = doc_attn_roofline(S, kl["doc_attn"])
        res["long_document"]["classify_roofline"] = classify_roofline(S, sl * 1e3)
    if not args.no_w8a8 and cfg.head != "fp8a8":
        # the long-document workload with its hidden rows quantized to E4M3 before
        # the head (fp8 x fp8 matrix cores); a precision change, so reported apart
        del S
        torch.cuda.empty_cache()
        S = setup(5, args.streams, inp=inp5, head="fp8a8")
        s8, k8 = run_steps(S, *long_enough(S, few, 10))
        f8, R8 = head_flops(S)
        tf = f8 / (k8["head"] * 1e-3) / 1e12
        res["w8a8"] = {"config": 5, "docs_per_s": round(S["docs"].B / s8, 2),
                       "ms_per_step": round(s8 * 1e3, 4), "dtype": "fp8 e4m3 x fp8 e4m3 (head only)",
                       "head_ms": round(k8["head"], 4), "rows": R8,
                       "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(tf / PEAK_FP8_TFLOPS, 4),
                                    "kernel": "quant_rows_e4m3_kernel + lmhead_ring_kernel<fp8 W, fp8 h>"},
                       "classify_roofline": classify_roofline(S, s8 * 1e3)}
    if not args.no_shard:
        # documents shard over GPUs with no collective: one GPU's share of the
        # 128-document long-document batch over 8 GPUs is 16 documents
        del S
        torch.cuda.empty_cache()
        S = setup(5, args.streams, inp=first_docs(inp5, 16) if inp5 is not None else None, B=16)
        s5, k5 = run_steps(S, *long_enough(S, few, 10))
        f5, _ = head_flops(S)
        tf = f5 / (k5["head"] * 1e-3) / 1e12
        res["shard_of_8"] = {"config": 5, "global_batch": 128, "per_gpu_batch": 16,
                             "docs_per_s": round(16 / s5, 2), "ms_per_step": round(s5 * 1e3, 4),
                             "head_ms": round(k5["head"], 4), "head_tflops": round(tf, 2),
                             "head_frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        if k5["doc_attn"]:
            res["shard_of_8"]["doc_attn_roofline"] = doc_attn_roofline(S, k5["doc_attn"])
    del inp5
    if decision:
        res["decision_word"] = decision
    if letters:
        res["letters"] = letters
    if decode:
        res["trie_decode"] = decode
    if not args.no_path_stress:
        del S
        torch.cuda.empty_cache()
        res["path_roofline"] = path_stress()
        S = None
    if not args.no_cpu_baseline:
        del S
        torch.cuda.empty_cache()
        S0 = setup(args.config)
        res["cpu_baseline"] = cpu_baseline(S0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
