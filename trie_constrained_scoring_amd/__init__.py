"""Python binding of libtcs, the gfx950 trie_tree label scorer.

Argument marshalling only: every computation runs in the HIP kernels of
``libtcs.so``.  Torch provides device memory and the stream; tensors are passed
by ``data_ptr()`` on ``torch.cuda.current_stream()``.  If the library is not
built, every call raises ``RuntimeError`` -- there is no fallback.

Entry points (same names as the C ABI in ``include/tcs.h``):
  trie_build, tree_attn, lmhead_lse_gather, path_sum_softmax, classify
plus the workspace-size queries and small holders (TrieDevice, Model, Docs).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtcs.so")

TCS_OK, TCS_EINVAL, TCS_EDUPLICATE, TCS_ECAPACITY, TCS_EUNSUPPORTED, TCS_EHIP, TCS_ENOTIMPL = \
    0, -1, -2, -3, -4, -5, -6
TCS_F32, TCS_BF16, TCS_FP8_E4M3, TCS_FP8_E4M3_A8 = 0, 1, 2, 3
DTYPES = {"f32": TCS_F32, "bf16": TCS_BF16, "fp8": TCS_FP8_E4M3}

P32 = C.POINTER(C.c_int32)
PF = C.POINTER(C.c_float)


class TcsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"tcs error {code}: {msg}")
        self.code = code


class tcs_trie(C.Structure):
    _fields_ = [("cap_nodes", C.c_int32), ("cap_levels", C.c_int32),
                ("n_nodes", C.c_int32), ("n_int", C.c_int32), ("n_labels", C.c_int32),
                ("max_depth", C.c_int32)] + [(n, P32) for n in (
                    "parent", "token", "depth", "child_begin", "child_count", "node_label", "qrow",
                    "qnode", "qparent", "label_node", "level_offsets", "e_tok", "e_qrow", "e_child",
                    "row_level_offsets", "label_row", "sub_label", "dec_node")] + [
                ("max_decode_steps", C.c_int32), ("max_children", C.c_int32)]


TRIE_DEV_ARRAYS = ("parent", "token", "child_begin", "child_count", "qnode", "qparent", "label_node",
                   "e_tok", "e_qrow", "e_child", "qrow", "row_level_offsets", "label_row", "sub_label",
                   "dec_node")


class tcs_trie_dev(C.Structure):
    _fields_ = [("n_nodes", C.c_int32), ("n_int", C.c_int32), ("n_labels", C.c_int32),
                ("max_depth", C.c_int32)] + [(n, C.c_void_p) for n in TRIE_DEV_ARRAYS] + [
                ("max_decode_steps", C.c_int32), ("max_children", C.c_int32)]


class tcs_model(C.Structure):
    _fields_ = [("dtype", C.c_int), ("head_dtype", C.c_int), ("d", C.c_int32), ("Hq", C.c_int32),
                ("Hkv", C.c_int32), ("hd", C.c_int32), ("V", C.c_int32), ("eps", C.c_float),
                ("E", C.c_void_p), ("Wq", C.c_void_p), ("Wk", C.c_void_p), ("Wv", C.c_void_p),
                ("Wo", C.c_void_p), ("W", C.c_void_p), ("W_scale", C.c_void_p)]


class tcs_docs(C.Structure):
    _fields_ = [("B", C.c_int32), ("total_tokens", C.c_int32), ("doc_offsets", C.c_void_p),
                ("Kd", C.c_void_p), ("Vd", C.c_void_p), ("doc_tokens", C.c_void_p)]


class tcs_prepared(C.Structure):
    _fields_ = [("B", C.c_int32), ("buf", C.c_void_p), ("bytes", C.c_size_t)]


_lib_handle = None


def lib():
    """The loaded libtcs.so; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libtcs.so not found at {LIB_PATH}: build it first "
                               "(python -m trie_constrained_scoring_amd.build)")
        L = C.CDLL(LIB_PATH)
        vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
        L.tcs_last_error.restype = C.c_char_p
        L.tcs_version.restype = C.c_char_p
        L.tcs_trie_build.argtypes = [P32, P32, i32, i32, i32, C.POINTER(tcs_trie)]
        L.tcs_decision_truncate.argtypes = [P32, P32, i32, i32, C.POINTER(C.c_uint8), P32, P32,
                                            P32]
        L.tcs_tree_attn_workspace_bytes.restype = sz
        L.tcs_tree_attn_workspace_bytes.argtypes = [i32, i32, i32]
        L.tcs_tree_attn.argtypes = [vp, C.c_int, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                    C.c_float, vp, vp, sz]
        L.tcs_tree_attn_noalloc.argtypes = [vp, C.c_int, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                            vp, vp, C.c_float, vp]
        L.tcs_lmhead_workspace_bytes.restype = sz
        L.tcs_lmhead_workspace_bytes.argtypes = [C.c_int, C.c_int, i32, i32, i32, i32, i32]
        L.tcs_lmhead_lse_gather.argtypes = [vp, C.c_int, C.c_int, i32, i32, i32, i32, i32, vp, vp,
                                            vp, vp, vp, vp, vp, vp, vp, sz]
        L.tcs_path_sum_softmax.argtypes = [vp, i32, C.POINTER(tcs_trie_dev), vp, vp, vp, vp]
        L.tcs_classify_workspace_bytes.restype = sz
        L.tcs_classify_workspace_bytes.argtypes = [C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                                   C.POINTER(tcs_docs)]
        L.tcs_classify.argtypes = [vp, C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                   C.POINTER(tcs_docs), vp, vp, vp, vp, sz]
        L.tcs_classify_prepared_bytes.restype = sz
        L.tcs_classify_prepared_bytes.argtypes = [C.POINTER(tcs_model), C.POINTER(tcs_trie_dev), i32]
        L.tcs_classify_prepare.argtypes = [vp, C.POINTER(tcs_model), C.POINTER(tcs_trie_dev), i32,
                                           C.POINTER(tcs_prepared)]
        L.tcs_classify_run_workspace_bytes.restype = sz
        L.tcs_classify_run_workspace_bytes.argtypes = [C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                                       C.POINTER(tcs_docs)]
        L.tcs_classify_run.argtypes = [vp, C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                       C.POINTER(tcs_docs), C.POINTER(tcs_prepared), vp, vp, vp, vp, sz]
        L.tcs_letters_run.argtypes = list(L.tcs_classify_run.argtypes)
        L.tcs_decode_workspace_bytes.restype = sz
        L.tcs_decode_workspace_bytes.argtypes = [C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                                 C.POINTER(tcs_docs)]
        L.tcs_decode_run.argtypes = [vp, C.POINTER(tcs_model), C.POINTER(tcs_trie_dev),
                                     C.POINTER(tcs_docs), C.POINTER(tcs_prepared), vp, vp, vp, sz]
        L.tcs_timing_enable.argtypes = [C.c_int]
        L.tcs_timing_read.argtypes = [C.c_int, C.POINTER(C.c_double), C.POINTER(i32)]
        _lib_handle = L
    return _lib_handle


def _check(rc):
    if rc != TCS_OK:
        raise TcsError(rc, lib().tcs_last_error().decode())


def version() -> str:
    return lib().tcs_version().decode()


TCS_TIMER_HEAD, TCS_TIMER_DOC_ATTN = 0, 1


def timing_enable(on: bool = True) -> None:
    """Start (or stop and reset) HIP-event timing of the head and document-attention
    kernels inside the library (tcs_timing_enable)."""
    _check(lib().tcs_timing_enable(1 if on else 0))


def timing_read(timer: int):
    """(total milliseconds, launches) recorded for `timer` since the last read
    (tcs_timing_read); waits for the recorded events."""
    ms, n = C.c_double(), C.c_int32()
    _check(lib().tcs_timing_read(int(timer), C.byref(ms), C.byref(n)))
    return ms.value, n.value


# ------------------------------------------------------------------ torch glue

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def to_device(arr: np.ndarray, kind: str, device="cuda"):
    """Upload a host array: kind 'bf16' takes uint16 bit patterns, 'fp8' uint8 codes."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    if kind == "fp8":
        return torch.from_numpy(a.view(np.uint8)).to(device)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
    if kind == "i32":
        return torch.from_numpy(a.astype(np.int32, copy=False)).to(device)
    raise ValueError(kind)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return TCS_F32
    if t.dtype in (torch.bfloat16, torch.int16):
        return TCS_BF16
    if t.dtype in (torch.uint8, getattr(torch, "float8_e4m3fn", None)):
        return TCS_FP8_E4M3
    raise ValueError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------------------------ trie

@dataclass
class Trie:
    """Host trie arrays from tcs_trie_build (numpy int32)."""
    n_nodes: int
    n_int: int
    n_labels: int
    max_depth: int
    arrays: dict
    max_decode_steps: int = 0
    max_children: int = 0

    def __getattr__(self, k):
        a = self.__dict__.get("arrays")
        if a is not None and k in a:
            return a[k]
        raise AttributeError(k)


def trie_build(label_offsets, label_tokens, root_token: int, V: int) -> Trie:
    """Canonical token trie of the labels (host library call, no GPU needed)."""
    L = lib()
    offs = np.ascontiguousarray(label_offsets, dtype=np.int32)
    toks = np.ascontiguousarray(label_tokens, dtype=np.int32)
    M = len(offs) - 1
    cap = max(2, int(offs[-1]) + 1 if M > 0 else 2)
    for _ in range(2):
        arrays = {n: np.zeros(cap, dtype=np.int32) for n in (
            "parent", "token", "depth", "child_begin", "child_count", "node_label", "qrow", "qnode",
            "qparent", "e_tok", "e_qrow", "e_child", "sub_label", "dec_node")}
        arrays["label_node"] = np.zeros(max(M, 1), dtype=np.int32)
        arrays["label_row"] = np.zeros(max(M, 1), dtype=np.int32)
        arrays["level_offsets"] = np.zeros(cap + 1, dtype=np.int32)
        arrays["row_level_offsets"] = np.zeros(cap + 1, dtype=np.int32)
        t = tcs_trie(cap_nodes=cap, cap_levels=cap + 1)
        for n, a in arrays.items():
            setattr(t, n, a.ctypes.data_as(P32))
        rc = L.tcs_trie_build(offs.ctypes.data_as(P32), toks.ctypes.data_as(P32), M, root_token, V,
                              C.byref(t))
        if rc == TCS_ECAPACITY:
            cap = max(t.n_nodes, t.max_depth + 2)
            continue
        _check(rc)
        N, n_int, D = t.n_nodes, t.n_int, t.max_depth
        cut = {"qnode": n_int, "qparent": n_int, "e_tok": N - 1, "e_qrow": N - 1, "e_child": N - 1,
               "label_node": M, "label_row": M, "level_offsets": D + 2, "row_level_offsets": D + 2}
        out = {n: a[:cut.get(n, N)].copy() for n, a in arrays.items()}
        return Trie(N, n_int, M, D, out, int(t.max_decode_steps), int(t.max_children))
    raise TcsError(TCS_ECAPACITY, "trie capacity")


def decision_truncate(label_offsets, label_tokens, V: int, word_cont):
    """Decision-word cut of the labels (tcs_decision_truncate, host library call).

    Returns (offsets [M+1], tokens, depth [M]) as numpy int32: label m cut to its
    first depth[m] tokens.  Feed the result to trie_build to score labels in the
    decision-word form."""
    L = lib()
    offs = np.ascontiguousarray(label_offsets, dtype=np.int32)
    toks = np.ascontiguousarray(label_tokens, dtype=np.int32)
    flags = np.ascontiguousarray(word_cont, dtype=np.uint8)
    M = len(offs) - 1
    if flags.shape != (V,):
        raise TcsError(TCS_EINVAL, f"decision_truncate: word_cont has shape {flags.shape}, need ({V},)")
    out_offs = np.zeros(max(M, 0) + 1, dtype=np.int32)
    out_toks = np.zeros(max(len(toks), 1), dtype=np.int32)
    depth = np.zeros(max(M, 1), dtype=np.int32)
    _check(L.tcs_decision_truncate(offs.ctypes.data_as(P32), toks.ctypes.data_as(P32), M, V,
                                   flags.ctypes.data_as(C.POINTER(C.c_uint8)),
                                   out_offs.ctypes.data_as(P32), out_toks.ctypes.data_as(P32),
                                   depth.ctypes.data_as(P32)))
    return out_offs, out_toks[:out_offs[-1]].copy(), depth[:M].copy()


class TrieDevice:
    """Device copy of the trie arrays the kernels read (tcs_trie_dev)."""

    def __init__(self, trie: Trie, device="cuda"):
        torch = _torch()
        self.trie = trie
        self.tensors = {n: torch.from_numpy(np.ascontiguousarray(trie.arrays[n])).to(device)
                        for n in TRIE_DEV_ARRAYS}
        self.struct = tcs_trie_dev(n_nodes=trie.n_nodes, n_int=trie.n_int, n_labels=trie.n_labels,
                                   max_depth=trie.max_depth, max_decode_steps=trie.max_decode_steps,
                                   max_children=trie.max_children,
                                   **{n: self.tensors[n].data_ptr() for n in TRIE_DEV_ARRAYS})

    def __getitem__(self, k):
        return self.tensors[k]


# ------------------------------------------------------------------ kernels

def tree_attn_workspace_bytes(n_int, Hq, hd) -> int:
    return int(lib().tcs_tree_attn_workspace_bytes(n_int, Hq, hd))


def tree_attn(Qn, Kn, Vn, Kd, Vd, doc_offsets, qparent, scale, O=None, ws=None, stream=None):
    """Ancestor-masked tree attention (tcs_tree_attn).

    Qn [n_int, Hq, hd]; Kn, Vn [n_int, Hkv, hd]; Kd, Vd [sum L, Hkv, hd];
    doc_offsets [B+1] int32; qparent [n_int] int32.  Returns O [B, n_int, Hq, hd].
    """
    torch = _torch()
    n_int, Hq, hd = Qn.shape
    Hkv = Kn.shape[1]
    B = doc_offsets.shape[0] - 1
    if O is None:
        O = torch.empty((B, n_int, Hq, hd), dtype=Qn.dtype, device=Qn.device)
    need = tree_attn_workspace_bytes(n_int, Hq, hd)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=Qn.device)
    _need_cuda(Qn, Kn, Vn, Kd, Vd, doc_offsets, qparent, O, ws)
    _check(lib().tcs_tree_attn(_stream(stream), _dtype_code(Qn), B, n_int, Hq, Hkv, hd, _ptr(Qn),
                               _ptr(Kn), _ptr(Vn), _ptr(Kd), _ptr(Vd), _ptr(doc_offsets),
                               _ptr(qparent), float(scale), _ptr(O), _ptr(ws), ws.numel()))
    return O


NOALLOC_SCRATCH_BYTES = 16 << 20   # TCS_NOALLOC_SCRATCH_BYTES in include/tcs.h


def tree_attn_noalloc(Qn, Kn, Vn, Kd, Vd, doc_offsets, qparent, scale, O=None, stream=None):
    """tcs_tree_attn_noalloc: tcs_tree_attn with its scratch in the library's own
    per-GPU device array (no workspace argument, nothing allocated by the call).
    Calls that overlap on one GPU race on that array."""
    torch = _torch()
    n_int, Hq, hd = Qn.shape
    Hkv = Kn.shape[1]
    B = doc_offsets.shape[0] - 1
    if O is None:
        O = torch.empty((B, n_int, Hq, hd), dtype=Qn.dtype, device=Qn.device)
    _need_cuda(Qn, Kn, Vn, Kd, Vd, doc_offsets, qparent, O)
    _check(lib().tcs_tree_attn_noalloc(_stream(stream), _dtype_code(Qn), B, n_int, Hq, Hkv, hd,
                                       _ptr(Qn), _ptr(Kn), _ptr(Vn), _ptr(Kd), _ptr(Vd),
                                       _ptr(doc_offsets), _ptr(qparent), float(scale), _ptr(O)))
    return O


def lmhead_workspace_bytes(B, n_int, n_nodes, d, V, h_dtype=TCS_BF16, w_dtype=None) -> int:
    w_dtype = h_dtype if w_dtype is None else w_dtype
    n = int(lib().tcs_lmhead_workspace_bytes(h_dtype, w_dtype, B, n_int, n_nodes, d, V))
    if n == 0:
        _check(TCS_EINVAL)
    return n


def lmhead_lse_gather(h, W, trie_dev: TrieDevice, B, w_scale=None, lse=None, lp=None, ws=None,
                      stream=None, act8=False):
    """Output head with fused log-sum-exp and child gather (tcs_lmhead_lse_gather).

    h [B * n_int, d]; W [V, d] (bf16/f32, or uint8 E4M3 codes with w_scale [V]);
    act8 (fp8 W only): quantize each row of h to E4M3 first (the W8A8 head).
    Returns (lse [B * n_int], lp [B, n_nodes]).
    """
    torch = _torch()
    t = trie_dev.trie
    R, d = h.shape
    V = W.shape[0]
    if R != B * t.n_int:
        raise ValueError("h rows must be B * n_int")
    if lse is None:
        lse = torch.empty(R, dtype=torch.float32, device=h.device)
    if lp is None:
        lp = torch.empty((B, t.n_nodes), dtype=torch.float32, device=h.device)
    w_code = _dtype_code(W)
    if act8:
        if w_code != TCS_FP8_E4M3:
            raise ValueError("act8 needs E4M3 weights")
        w_code = TCS_FP8_E4M3_A8
    need = lmhead_workspace_bytes(B, t.n_int, t.n_nodes, d, V, _dtype_code(h), w_code)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=h.device)
    _need_cuda(h, W, w_scale, lse, lp, ws)
    _check(lib().tcs_lmhead_lse_gather(
        _stream(stream), _dtype_code(h), w_code, B, t.n_int, t.n_nodes, d, V, _ptr(h),
        _ptr(W), _ptr(w_scale), _ptr(trie_dev["e_tok"]), _ptr(trie_dev["e_qrow"]),
        _ptr(trie_dev["e_child"]), _ptr(lse), _ptr(lp), _ptr(ws), ws.numel()))
    return lse, lp


def path_sum_softmax(lp, trie_dev: TrieDevice, ll=None, prob=None, label=None, with_prob=True,
                     stream=None):
    """Label log-likelihoods, softmax and argmax (tcs_path_sum_softmax)."""
    torch = _torch()
    B = lp.shape[0]
    M = trie_dev.trie.n_labels
    if ll is None:
        ll = torch.empty((B, M), dtype=torch.float32, device=lp.device)
    if prob is None and with_prob:
        prob = torch.empty((B, M), dtype=torch.float32, device=lp.device)
    if label is None:
        label = torch.empty(B, dtype=torch.int32, device=lp.device)
    _need_cuda(lp, ll, prob, label)
    _check(lib().tcs_path_sum_softmax(_stream(stream), B, C.byref(trie_dev.struct), _ptr(lp),
                                      _ptr(ll), _ptr(prob), _ptr(label)))
    return ll, prob, label


# ------------------------------------------------------------------ classify

class Model:
    """Device weights of the scoring layer + output head (tcs_model)."""

    def __init__(self, cfg, inp: dict, device="cuda", eps=1e-6):
        kind = cfg.dtype
        self.cfg = cfg
        self.t = {k: to_device(inp[k], kind, device) for k in ("E", "Wq", "Wk", "Wv", "Wo")}
        if cfg.head in ("fp8", "fp8a8"):
            self.t["W"] = to_device(inp["W"], "fp8", device)
            self.t["W_scale"] = to_device(inp["W_scale"], "f32", device)
        else:
            self.t["W"] = to_device(inp["W"], kind, device)
            self.t["W_scale"] = None
        head = {"fp8": TCS_FP8_E4M3, "fp8a8": TCS_FP8_E4M3_A8}.get(cfg.head, DTYPES[kind])
        self.struct = tcs_model(
            dtype=DTYPES[kind], head_dtype=head,
            d=cfg.d, Hq=cfg.Hq, Hkv=cfg.Hkv, hd=cfg.hd, V=cfg.V, eps=eps,
            E=self.t["E"].data_ptr(), Wq=self.t["Wq"].data_ptr(), Wk=self.t["Wk"].data_ptr(),
            Wv=self.t["Wv"].data_ptr(), Wo=self.t["Wo"].data_ptr(), W=self.t["W"].data_ptr(),
            W_scale=self.t["W_scale"].data_ptr() if self.t["W_scale"] is not None else None)


class Docs:
    """A document batch on the device (tcs_docs): doc K/V, or token ids."""

    def __init__(self, cfg, inp: dict, device="cuda"):
        offs = inp["doc_offsets"]
        self.B = len(offs) - 1
        self.offsets = to_device(offs, "i32", device)
        self.Kd = self.Vd = self.tokens = None
        if "Kd" in inp:
            self.Kd = to_device(inp["Kd"], cfg.dtype, device)
            self.Vd = to_device(inp["Vd"], cfg.dtype, device)
        else:
            self.tokens = to_device(inp["doc_tokens"], "i32", device)
        self.struct = tcs_docs(
            B=self.B, total_tokens=int(offs[-1]), doc_offsets=self.offsets.data_ptr(),
            Kd=self.Kd.data_ptr() if self.Kd is not None else None,
            Vd=self.Vd.data_ptr() if self.Vd is not None else None,
            doc_tokens=self.tokens.data_ptr() if self.tokens is not None else None)


def classify_workspace_bytes(model: Model, trie_dev: TrieDevice, docs: Docs) -> int:
    n = int(lib().tcs_classify_workspace_bytes(C.byref(model.struct), C.byref(trie_dev.struct),
                                               C.byref(docs.struct)))
    if n == 0:
        _check(TCS_EINVAL)
    return n


class Prepared:
    """Per-label-set state of classify for batches of B documents (tcs_classify_prepare):
    a device buffer owned here, valid while the model and trie stay unchanged."""

    def __init__(self, model: Model, trie_dev: TrieDevice, B: int, stream=None):
        torch = _torch()
        n = int(lib().tcs_classify_prepared_bytes(C.byref(model.struct), C.byref(trie_dev.struct), B))
        if n == 0:
            _check(TCS_EINVAL)
        self.buf = torch.empty(n, dtype=torch.uint8, device=trie_dev["parent"].device)
        _need_cuda(self.buf)
        self.struct = tcs_prepared(B=0, buf=self.buf.data_ptr(), bytes=n)
        _check(lib().tcs_classify_prepare(_stream(stream), C.byref(model.struct),
                                          C.byref(trie_dev.struct), B, C.byref(self.struct)))
        self.B = B


def classify_run_workspace_bytes(model: Model, trie_dev: TrieDevice, docs: Docs) -> int:
    n = int(lib().tcs_classify_run_workspace_bytes(C.byref(model.struct), C.byref(trie_dev.struct),
                                                   C.byref(docs.struct)))
    if n == 0:
        _check(TCS_EINVAL)
    return n


def classify(model: Model, trie_dev: TrieDevice, docs: Docs, label=None, prob=None, ll=None,
             with_prob=True, ws=None, stream=None, prepared: Prepared = None):
    """The whole trie_tree pass (tcs_classify), or with `prepared` one batch on
    per-label-set state (tcs_classify_run).  Returns (label [B], prob [B, M], ll [B, M]).
    With `stream`, the work is queued on that torch stream; the results are ready once
    it has finished.  Runs on different streams need their own `ws`."""
    torch = _torch()
    B, M = docs.B, trie_dev.trie.n_labels
    dev = docs.offsets.device
    if label is None:
        label = torch.empty(B, dtype=torch.int32, device=dev)
    if prob is None and with_prob:
        prob = torch.empty((B, M), dtype=torch.float32, device=dev)
    if ll is None:
        ll = torch.empty((B, M), dtype=torch.float32, device=dev)
    if prepared is None:
        need = classify_workspace_bytes(model, trie_dev, docs)
    else:
        need = classify_run_workspace_bytes(model, trie_dev, docs)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _need_cuda(label, prob, ll, ws)
    if stream is not None:
        # the kernels use these on `stream`: keep the caching allocator from handing
        # their memory to other work before that stream is done with it
        for x in (label, prob, ll, ws):
            if x is not None:
                x.record_stream(stream)
    if prepared is None:
        _check(lib().tcs_classify(_stream(stream), C.byref(model.struct), C.byref(trie_dev.struct),
                                  C.byref(docs.struct), _ptr(label), _ptr(prob), _ptr(ll), _ptr(ws),
                                  ws.numel()))
    else:
        _check(lib().tcs_classify_run(_stream(stream), C.byref(model.struct),
                                      C.byref(trie_dev.struct), C.byref(docs.struct),
                                      C.byref(prepared.struct), _ptr(label), _ptr(prob), _ptr(ll),
                                      _ptr(ws), ws.numel()))
    return label, prob, ll


def letters(model: Model, trie_dev: TrieDevice, docs: Docs, prepared: Prepared, label=None,
            prob=None, ll=None, with_prob=True, ws=None, stream=None):
    """letters (tcs_letters_run): one answer position per document, the M letter rows
    of the head only, probabilities rescaled over the letters.  `trie_dev` holds the
    letter tokens as one-token labels; `prepared` is its tcs_classify_prepare state.
    Returns (label [B], prob [B, M], ll [B, M] letter logits)."""
    torch = _torch()
    B, M = docs.B, trie_dev.trie.n_labels
    dev = docs.offsets.device
    if label is None:
        label = torch.empty(B, dtype=torch.int32, device=dev)
    if prob is None and with_prob:
        prob = torch.empty((B, M), dtype=torch.float32, device=dev)
    if ll is None:
        ll = torch.empty((B, M), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty(classify_run_workspace_bytes(model, trie_dev, docs), dtype=torch.uint8,
                         device=dev)
    _need_cuda(label, prob, ll, ws)
    if stream is not None:
        for x in (label, prob, ll, ws):
            if x is not None:
                x.record_stream(stream)
    _check(lib().tcs_letters_run(_stream(stream), C.byref(model.struct), C.byref(trie_dev.struct),
                                 C.byref(docs.struct), C.byref(prepared.struct), _ptr(label),
                                 _ptr(prob), _ptr(ll), _ptr(ws), ws.numel()))
    return label, prob, ll


def decode_workspace_bytes(model: Model, trie_dev: TrieDevice, docs: Docs) -> int:
    n = int(lib().tcs_decode_workspace_bytes(C.byref(model.struct), C.byref(trie_dev.struct),
                                             C.byref(docs.struct)))
    if n == 0:
        _check(TCS_EINVAL)
    return n


def trie_decode(model: Model, trie_dev: TrieDevice, docs: Docs, prepared: Prepared, label=None,
                runs=None, ws=None, stream=None):
    """trie_decode (tcs_decode_run): greedy generation inside the label trie, the
    model run only where labels branch.  Returns (label [B], runs [B])."""
    torch = _torch()
    B = docs.B
    dev = docs.offsets.device
    if label is None:
        label = torch.empty(B, dtype=torch.int32, device=dev)
    if runs is None:
        runs = torch.empty(B, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty(decode_workspace_bytes(model, trie_dev, docs), dtype=torch.uint8, device=dev)
    _need_cuda(label, runs, ws)
    if stream is not None:
        for x in (label, runs, ws):
            x.record_stream(stream)
    _check(lib().tcs_decode_run(_stream(stream), C.byref(model.struct), C.byref(trie_dev.struct),
                                C.byref(docs.struct), C.byref(prepared.struct), _ptr(label),
                                _ptr(runs), _ptr(ws), ws.numel()))
    return label, runs
