"""Seeded synthetic workloads for trie_tree label scoring.

The workloads stand in for the ones the pages describe: the 10-topic support
query of "To Classify, Try a Trie Tree" (section 2, section 3.1 running example),
classification operators with up to 255 labels (section 2, categories argument), and
tool-registry / taxonomy label sets of thousands of labels ("Trie Automata for
Constrained Decoding over Large Finite Sets", introduction).  No dataset from the
pages is available here, so every label set, weight and document KV is drawn from
a seeded numpy PCG64 generator.

Storage formats produced here:
  * bf16 tensors are numpy ``uint16`` bit patterns, rounded to nearest-even from fp32;
  * fp32 tensors are numpy ``float32``;
  * the fp8 LM head is OCP ``E4M3FN`` bytes (``uint8``) plus one fp32 scale per
    vocabulary row, ``s_v = max|W_v| / 448``, codes rounded to nearest-even and
    saturated at +-448.

Random sub-streams, in spawn order: trie, root token, E, Wq, Wk, Wv, Wo, W, doc,
word (the word-continuation flags), letters (the letter token ids); streams are
only ever appended, so the earlier ones do not change.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

STREAMS = ("trie", "root", "E", "Wq", "Wk", "Wv", "Wo", "W", "doc", "word", "letters")


@dataclass(frozen=True)
class Config:
    """One workload: model dims, label-set recipe and document batch."""
    id: int
    name: str
    B: int                       # documents per batch
    L: int                       # tokens per document (uniform unless doc_lens given)
    V: int                       # vocabulary rows of E and of the LM head
    d: int                       # model width
    Hq: int
    Hkv: int
    hd: int
    dtype: str                   # "f32" or "bf16": storage of weights and activations
    head: str                    # "same" (LM head in `dtype`), "fp8" (E4M3FN + fp32 row scale) or
                                 # "fp8a8" (the same weights; activations quantized to E4M3 too)
    trie: tuple                  # ("running",) or ("zipf", M, lo, hi, s)
    doc_mode: str                # "kv": doc K/V given; "tokens": doc token ids given
    doc_lens: tuple | None = None  # ragged lengths (overrides B and L)
    std: float = 0.02            # weight init std

    def lens(self):
        return list(self.doc_lens) if self.doc_lens is not None else [self.L] * self.B

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


QWEN3_4B = dict(V=151936, d=2560, Hq=32, Hkv=8, hd=128)

CONFIGS = {
    1: Config(1, "tiny", B=4, L=32, V=1000, d=64, Hq=1, Hkv=1, hd=64, dtype="f32", head="same",
              trie=("running",), doc_mode="tokens"),
    2: Config(2, "running-example", B=64, L=512, dtype="bf16", head="same", trie=("running",),
              doc_mode="kv", **QWEN3_4B),
    3: Config(3, "max-label-set-255", B=32, L=1024, dtype="bf16", head="same",
              trie=("zipf", 255, 2, 40, 1.2), doc_mode="kv", **QWEN3_4B),
    4: Config(4, "large-finite-set-5000", B=8, L=256, dtype="bf16", head="same",
              trie=("zipf", 5000, 3, 10, 1.1), doc_mode="kv", **QWEN3_4B),
    5: Config(5, "long-document-kv", B=128, L=4096, dtype="bf16", head="fp8", trie=("running",),
              doc_mode="kv", **QWEN3_4B),
}


def config(cid: int, **overrides) -> Config:
    """A named workload, optionally with some fields replaced (for smaller test shapes)."""
    return CONFIGS[cid].replace(**overrides)


# --------------------------------------------------------------------------- labels

# Shape of the running example: 10 labels, 17 distinct word tokens.  Token symbols
# 0..16 are mapped to distinct seeded ids.  Lengths [1,2,2,2,2,3,2,4,1,1]; the root
# forks 7 ways, "refund" 2 ways, "shipping" 3 ways; "two" starts a 4-token chain.
_RUNNING_SHAPE = [
    [0],               # billing
    [1, 2],            # refund request
    [1, 3],            # refund status
    [4, 5],            # shipping delay
    [4, 6],            # shipping damage
    [4, 7, 8],         # shipping address change
    [9, 10],           # product defect
    [11, 12, 13, 14],  # two -factor authentication issue
    [15],              # praise
    [16],              # other
]
# "-factor" carries no leading space: it continues the word "two".
_RUNNING_CONTINUATION = {12}

# Share of vocabulary tokens that continue the previous token's word (no leading
# space) in the synthetic tokenizer.
WORD_CONT_P = 0.25


def running_example_labels(rng: np.random.Generator, V: int):
    ids = rng.choice(V, size=17, replace=False)
    return [[int(ids[s]) for s in lab] for lab in _RUNNING_SHAPE]


def word_continuation_flags(cfg: "Config", labels, rng: np.random.Generator):
    """uint8 [V]: 1 where a vocabulary token continues the previous token's word.

    Words decide how far a label is scored in the decision-word form of trie_tree
    ("To Classify, Try a Trie Tree", section 3.2: a label is scored through the
    last token of the word in which no other label shares its prefix any more).
    Each token is a continuation with probability WORD_CONT_P; in the running
    example the label tokens are set by hand so that only "-factor" continues a word.
    """
    flags = (rng.random(cfg.V) < WORD_CONT_P).astype(np.uint8)
    if cfg.trie[0] == "running":
        for lab, shape in zip(labels, _RUNNING_SHAPE):
            for t, sym in zip(lab, shape):
                flags[t] = 1 if sym in _RUNNING_CONTINUATION else 0
    return flags


def zipf_copy_prefix_labels(rng: np.random.Generator, V: int, M: int, lo: int, hi: int, s: float):
    """Prefix-free, duplicate-free label set with Zipf-distributed prefix sharing.

    Label i draws a length L ~ U{lo..hi}, picks an earlier label j with probability
    proportional to (j+1)^-s, copies a prefix of length p ~ U{0..min(L, L_j)-1} and
    fills the rest uniformly from [0, V).  Candidates that duplicate a label, or are
    a prefix of one or have one as a prefix, are redrawn.
    """
    labels: list[list[int]] = []
    full: set[tuple] = set()
    proper_prefixes: set[tuple] = set()
    cw = np.cumsum((np.arange(M) + 1.0) ** (-s))
    tries = 0
    while len(labels) < M:
        tries += 1
        if tries > 1000 * M:
            raise RuntimeError("label generator could not find enough prefix-free labels")
        L = int(rng.integers(lo, hi + 1))
        if labels:
            n = len(labels)
            j = int(np.searchsorted(cw[:n], rng.random() * cw[n - 1], side="right"))
            j = min(j, n - 1)
            p = int(rng.integers(0, min(L, len(labels[j]))))
            prefix = labels[j][:p]
        else:
            prefix = []
        cand = prefix + [int(t) for t in rng.integers(0, V, L - len(prefix))]
        tc = tuple(cand)
        if tc in full or tc in proper_prefixes:
            continue
        if any(tc[:k] in full for k in range(1, len(tc))):
            continue
        labels.append(cand)
        full.add(tc)
        for k in range(1, len(tc)):
            proper_prefixes.add(tc[:k])
    return labels


def make_labels(cfg: Config, rng: np.random.Generator):
    kind = cfg.trie[0]
    if kind == "running":
        return running_example_labels(rng, cfg.V)
    if kind == "zipf":
        _, M, lo, hi, s = cfg.trie
        return zipf_copy_prefix_labels(rng, cfg.V, M, lo, hi, s)
    if kind == "explicit":
        return [list(l) for l in cfg.trie[1]]
    raise ValueError(f"unknown trie recipe {cfg.trie!r}")


def labels_to_csr(labels):
    offsets = np.zeros(len(labels) + 1, dtype=np.int32)
    offsets[1:] = np.cumsum([len(l) for l in labels])
    tokens = np.array([t for l in labels for t in l], dtype=np.int32)
    return offsets, tokens


def csr_to_labels(offsets, tokens):
    return [list(map(int, tokens[offsets[i]:offsets[i + 1]])) for i in range(len(offsets) - 1)]


# --------------------------------------------------------------------------- storage formats

def _bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _e4m3_grid():
    """Non-negative finite OCP E4M3FN values indexed by their 7-bit code (0..126)."""
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3_GRID = _e4m3_grid()


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round |x| <= 448 to the nearest E4M3FN code (ties to even code), keep the sign."""
    a = np.minimum(np.abs(x), 448.0)
    hi = np.searchsorted(_E4M3_GRID, a, side="left").clip(1, 126)
    lo = hi - 1
    dlo = a - _E4M3_GRID[lo]
    dhi = _E4M3_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 448.0, 126, code)
    sign = (np.signbit(x)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _normal_f32(rng, shape, std, chunk_rows=8192):
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32) * np.float32(std)
    return out


def _weight(rng, shape, std, dtype, chunk_rows=8192):
    if dtype == "f32":
        return _normal_f32(rng, shape, std, chunk_rows)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32) * np.float32(std)
        flat[r0:r1] = _bf16_bits_from_f32(x)
    return out


def _fp8_head(rng, V, d, std, chunk_rows=8192):
    codes = np.empty((V, d), dtype=np.uint8)
    scale = np.empty(V, dtype=np.float32)
    for r0 in range(0, V, chunk_rows):
        r1 = min(V, r0 + chunk_rows)
        w = rng.standard_normal((r1 - r0, d), dtype=np.float32) * np.float32(std)
        s = (np.abs(w).max(axis=1) / np.float32(448.0)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        scale[r0:r1] = s
        codes[r0:r1] = _e4m3_codes(w.astype(np.float64) / s[:, None].astype(np.float64))
    return codes, scale


# --------------------------------------------------------------------------- full input set

def make_inputs(cfg: Config, seed: int | None = None, *, weights: bool = True):
    """Draw one workload.  Returns a dict of numpy arrays plus the label lists.

    Keys: labels (list of lists), label_offsets, label_tokens, root_token, word_cont
    (uint8 [V] word-continuation flags), letters (int32 [M] letter token ids), E, Wq, Wk,
    Wv, Wo, W, W_scale (fp8 head only, else None), doc_offsets, and either Kd/Vd
    ([sum L, Hkv, hd]) or doc_tokens ([sum L]).
    """
    seed = cfg.id if seed is None else seed
    ss = np.random.SeedSequence(seed)
    rngs = dict(zip(STREAMS, (np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(len(STREAMS)))))
    out: dict = {"cfg": cfg, "seed": seed}
    labels = make_labels(cfg, rngs["trie"])
    out["labels"] = labels
    out["label_offsets"], out["label_tokens"] = labels_to_csr(labels)
    out["root_token"] = int(rngs["root"].integers(0, cfg.V))
    out["word_cont"] = word_continuation_flags(cfg, labels, rngs["word"])
    # letters ("To Classify, Try a Trie Tree", section 3.3): one answer token per
    # label, M distinct vocabulary ids standing in for "A", "B", ...
    out["letters"] = rngs["letters"].choice(cfg.V, size=len(labels), replace=False).astype(np.int32)
    d, Hq, Hkv, hd, V = cfg.d, cfg.Hq, cfg.Hkv, cfg.hd, cfg.V
    if weights:
        out["E"] = _weight(rngs["E"], (V, d), cfg.std, cfg.dtype)
        out["Wq"] = _weight(rngs["Wq"], (Hq * hd, d), cfg.std, cfg.dtype)
        out["Wk"] = _weight(rngs["Wk"], (Hkv * hd, d), cfg.std, cfg.dtype)
        out["Wv"] = _weight(rngs["Wv"], (Hkv * hd, d), cfg.std, cfg.dtype)
        out["Wo"] = _weight(rngs["Wo"], (d, Hq * hd), cfg.std, cfg.dtype)
        if cfg.head in ("fp8", "fp8a8"):
            out["W"], out["W_scale"] = _fp8_head(rngs["W"], V, d, cfg.std)
        else:
            out["W"] = _weight(rngs["W"], (V, d), cfg.std, cfg.dtype)
            out["W_scale"] = None
    lens = cfg.lens()
    offs = np.zeros(len(lens) + 1, dtype=np.int32)
    offs[1:] = np.cumsum(lens)
    out["doc_offsets"] = offs
    T = int(offs[-1])
    if cfg.doc_mode == "tokens":
        out["doc_tokens"] = rngs["doc"].integers(0, V, T).astype(np.int32)
    else:
        kv = _weight(rngs["doc"], (2 * T, Hkv, hd), 1.0, cfg.dtype, chunk_rows=65536)
        out["Kd"] = kv[:T]
        out["Vd"] = kv[T:]
    return out
