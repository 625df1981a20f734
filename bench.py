"""Throughput of the trie_tree label-scoring pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2] [--extra 3,4]
                    [--no-cpu-baseline] [--no-lmhead-timing]

One step is one ``tcs_classify`` call over one batch of synthetic documents: the
node input block, ancestor-masked tree attention, output projection + RMSNorm,
the full-vocabulary output head with fused log-sum-exp and child gather, and the
path sums / label softmax / argmax.  Inputs are resident in HBM before timing.
The trie itself is built once per label set on the host (timed separately).

Prints ONE JSON line.  ``value`` is documents classified per second at the
primary workload (default: the running-example shape, 10 labels); the 255- and
5000-label workloads are reported under ``at_labels``.  ``roofline`` is for the
dominant kernel (the output head), timed with HIP events on the stream it runs
on; ``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "documents classified/sec at 10/255/5000 labels; % of HBM/MFMA roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def setup(cid: int):
    import torch
    import trie_constrained_scoring_amd as tcs
    from synth import config, make_inputs
    cfg = config(cid)
    t0 = time.time()
    inp = make_inputs(cfg)
    log(f"[bench] config {cid} inputs generated in {time.time() - t0:.1f}s")
    t0 = time.perf_counter()
    trie = tcs.trie_build(inp["label_offsets"], inp["label_tokens"], inp["root_token"], cfg.V)
    trie_ms = (time.perf_counter() - t0) * 1e3
    td = tcs.TrieDevice(trie)
    model = tcs.Model(cfg, inp)
    docs = tcs.Docs(cfg, inp)
    ws = torch.empty(tcs.classify_workspace_bytes(model, td, docs), dtype=torch.uint8, device="cuda")
    B, M = docs.B, trie.n_labels
    out = dict(label=torch.empty(B, dtype=torch.int32, device="cuda"),
               prob=torch.empty((B, M), dtype=torch.float32, device="cuda"),
               ll=torch.empty((B, M), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    return dict(cfg=cfg, inp=inp, trie=trie, td=td, model=model, docs=docs, ws=ws, out=out,
                trie_ms=trie_ms)


def run_steps(S, steps, warmup):
    import torch
    import trie_constrained_scoring_amd as tcs

    def step():
        tcs.classify(S["model"], S["td"], S["docs"], ws=S["ws"], **S["out"])
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_lmhead(S, reps):
    """Average duration of the output-head entry point (MFMA GEMM + LSE/gather
    epilogue + finalize) with HIP events on the stream it is launched on, fed the
    hidden states of the same workload's shape."""
    import torch
    import trie_constrained_scoring_amd as tcs
    cfg, td = S["cfg"], S["td"]
    R = S["docs"].B * td.trie.n_int
    g = torch.Generator(device="cuda").manual_seed(0)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    h = torch.randn((R, cfg.d), device="cuda", generator=g).to(dt)
    W, Ws = S["model"].t["W"], S["model"].t["W_scale"]
    lse = torch.empty(R, dtype=torch.float32, device="cuda")
    lp = torch.empty((S["docs"].B, td.trie.n_nodes), dtype=torch.float32, device="cuda")
    ws = torch.empty(tcs.lmhead_workspace_bytes(R, cfg.V), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        tcs.lmhead_lse_gather(h, W, td, S["docs"].B, w_scale=Ws, lse=lse, lp=lp, ws=ws, stream=stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        tcs.lmhead_lse_gather(h, W, td, S["docs"].B, w_scale=Ws, lse=lse, lp=lp, ws=ws, stream=stream)
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 2.0 * R * cfg.d * cfg.V
    return ms, flops, R


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
    t0 = time.perf_counter()
    O.classify(inp, docs=list(range(n)), model=model, trie=trie)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "docs/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of {S['docs'].B} documents of the same batch, every label, fp64 numpy "
                      f"(BLAS threads = visible cores), {dt:.1f}s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--extra", default="3,4", help="other label-set sizes to report (config ids)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lmhead-timing", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); documents shard across GPUs "
              "with no collective, so a multi-GPU figure is not measured here.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    S = setup(args.config)
    cfg, trie = S["cfg"], S["trie"]
    sec = run_steps(S, args.steps, args.warmup)
    B = S["docs"].B
    value = B / sec
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "docs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype if cfg.head == "same" else f"{cfg.dtype} (head weights fp8 e4m3)",
        "data": "synthetic (seeded; random weights N(0,0.02), random doc KV N(0,1))",
        "config": {"workload": f"{cfg.name} (config {cfg.id}): B={B} docs x {cfg.L} tokens, "
                               f"{trie.n_labels} labels, {trie.n_nodes} trie nodes "
                               f"({trie.n_int} internal), d={cfg.d}, Hq/Hkv/hd={cfg.Hq}/{cfg.Hkv}/{cfg.hd}, "
                               f"V={cfg.V}",
                   "labels": trie.n_labels, "trie_nodes": trie.n_nodes, "global_batch": B,
                   "seq_len": cfg.L, "parallelism": "none (1 GPU)"},
        "trie_nodes_per_s": round(B * trie.n_nodes / sec, 1),
        "trie_build_ms": round(S["trie_ms"], 3),
    }
    if not args.no_lmhead_timing:
        ms, flops, R = time_lmhead(S, reps=max(3, args.steps))
        ach = flops / (ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": "lmhead_lse_gather (bf16 MFMA GEMM + LSE/gather epilogue + finalize)",
                           "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": None, "rows": R, "flops_per_launch": flops,
                           "ms_per_launch": round(ms, 4)}
        res["lmhead_share_of_step"] = round(ms / (sec * 1e3), 4)
    extra = {}
    for c in [int(x) for x in args.extra.split(",") if x.strip()]:
        if c == args.config:
            continue
        del S
        torch.cuda.empty_cache()
        S2 = setup(c)
        s2 = run_steps(S2, max(3, args.steps // 2), 2)
        e = {"docs_per_s": round(S2["docs"].B / s2, 2), "ms_per_step": round(s2 * 1e3, 3),
             "labels": S2["trie"].n_labels, "trie_nodes": S2["trie"].n_nodes,
             "trie_nodes_per_s": round(S2["docs"].B * S2["trie"].n_nodes / s2, 1)}
        if not args.no_lmhead_timing:
            ms, flops, R = time_lmhead(S2, reps=5)
            e["lmhead_tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            e["lmhead_frac_bf16_peak"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        extra[str(S2["trie"].n_labels)] = e
        S = S2
    if extra:
        res["at_labels"] = extra
    if not args.no_cpu_baseline:
        del S
        torch.cuda.empty_cache()
        S0 = setup(args.config)
        res["cpu_baseline"] = cpu_baseline(S0)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
