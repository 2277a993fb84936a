"""Plain CPU oracle of one top-k Mixture-of-Experts layer (ctypes over ``moe_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only code that may import this module.  The GPU library never
imports it and shares no code with it.

The steps follow "Event Tensor: A Unified Abstraction for Compiling Dynamic Megakernel"
(MLSys 2026), sections "Problem" and "Core method": routing by the runtime top-k, the
per-expert histogram and its exp_indptr prefix sum, token grouping, the expert
GroupGEMM, and the weighted combine.  The arithmetic of each step is written out in
``moe_oracle.c``.

Array conventions: bf16 arrays are ``numpy.uint16`` holding the bit pattern; all arrays
are C-contiguous.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32p, u16p = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p
    f32p, f64p = ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_router_logits.argtypes = [u16p, f32p, f32p, i64, i64, i64, f32p]
    lib.oracle_topk.argtypes = [f32p, i64, i64, i64, ctypes.c_void_p]
    lib.oracle_softmax_topk.argtypes = [f32p, ctypes.c_void_p, i64, i64, i64, f64p]
    lib.oracle_histogram.argtypes = [ctypes.c_void_p, i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_permutation.argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64, i64, i64,
                                       ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_expert_row.argtypes = [u16p, u16p, u16p, u16p, i64, i64, f64p]
    lib.oracle_moe_token.argtypes = [u16p, i64, ctypes.c_void_p, f64p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, i64, i64, f64p]
    lib.oracle_moe_tokens.argtypes = [u16p, i64, ctypes.c_void_p, i64, i64, ctypes.c_void_p, f64p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, i64, f64p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    del i32p
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def router_logits(x: np.ndarray, Wr: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """fp32 logits [B, E] in the fixed summation order (64 interleaved fma chains, halves fold, bias last)."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    B, d = x.shape
    d2, E = Wr.shape
    assert d == d2
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
    out = np.empty((B, E), dtype=np.float32)
    _check(_load().oracle_router_logits(_ptr(x), _ptr(Wr), _ptr(bias), B, d, E, _ptr(out)), "router")
    return out


def topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert indices [B, k] (descending logit, ties to the lower index)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    B, E = logits.shape
    idx = np.empty((B, k), dtype=np.int32)
    _check(_load().oracle_topk(_ptr(logits), B, E, k, _ptr(idx)), "topk")
    return idx


def softmax_topk(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """fp64 softmax over the selected logits, [B, k]."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, E = logits.shape
    k = idx.shape[1]
    w = np.empty((B, k), dtype=np.float64)
    _check(_load().oracle_softmax_topk(_ptr(logits), _ptr(idx), B, E, k, _ptr(w)), "softmax")
    return w


def histogram(idx: np.ndarray, E: int):
    """(hist [E], exp_indptr [E+1]) int32."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B, k = idx.shape
    hist = np.empty(E, dtype=np.int32)
    indptr = np.empty(E + 1, dtype=np.int32)
    _check(_load().oracle_histogram(_ptr(idx), B, k, E, _ptr(hist), _ptr(indptr)), "histogram")
    return hist, indptr


def permutation(idx: np.ndarray, exp_indptr: np.ndarray, E: int):
    """(perm, inv) int32 [B*k]: stable counting sort of assignments b*k+i by expert."""
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    exp_indptr = np.ascontiguousarray(exp_indptr, dtype=np.int32)
    B, k = idx.shape
    perm = np.empty(B * k, dtype=np.int32)
    inv = np.empty(B * k, dtype=np.int32)
    _check(_load().oracle_permutation(_ptr(idx), _ptr(exp_indptr), B, k, E, _ptr(perm), _ptr(inv)),
           "permutation")
    return perm, inv


def routing(x, Wr, bias, k):
    """All routing outputs of the layer for every token."""
    E = Wr.shape[1]
    logits = router_logits(x, Wr, bias)
    idx = topk(logits, k)
    w = softmax_topk(logits, idx)
    hist, indptr = histogram(idx, E)
    perm, inv = permutation(idx, indptr, E)
    return {"logits": logits, "topk_idx": idx, "topk_w": w, "hist": hist,
            "exp_indptr": indptr, "perm": perm, "inv": inv}


def expert_row(xrow, W1e, W3e, W2e) -> np.ndarray:
    """One expert's SwiGLU FFN on one bf16 row, fp64 [d]."""
    xrow = np.ascontiguousarray(xrow, dtype=np.uint16)
    W1e = np.ascontiguousarray(W1e, dtype=np.uint16)
    W3e = np.ascontiguousarray(W3e, dtype=np.uint16)
    W2e = np.ascontiguousarray(W2e, dtype=np.uint16)
    d, f = W1e.shape
    y = np.empty(d, dtype=np.float64)
    _check(_load().oracle_expert_row(_ptr(xrow), _ptr(W1e), _ptr(W3e), _ptr(W2e), d, f, _ptr(y)), "expert_row")
    return y


def moe_tokens(x, tokens, idx, w, experts, d: int, f: int) -> np.ndarray:
    """Layer output (fp64 [len(tokens), d]) for the listed tokens, computed token-parallel.

    ``experts`` is either a tuple of full arrays (W1 [E,d,f], W3 [E,d,f], W2 [E,f,d]) or a
    callable ``e -> (W1e, W3e, W2e)`` that returns one expert's arrays.  Each token's values
    are the same whatever the thread count (``oracle_moe_tokens``).
    """
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.uint16)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    k = idx.shape[1]
    toks = np.ascontiguousarray(np.asarray([int(t) for t in tokens], dtype=np.int64))
    assert toks.size == 0 or (toks.min() >= 0 and toks.max() < min(x.shape[0], idx.shape[0]))
    used = sorted({int(e) for e in idx[toks].reshape(-1)}) if toks.size else []
    E = int(max(used)) + 1 if used else 1
    keep = {}
    if callable(experts):
        for e in used:
            keep[e] = tuple(np.ascontiguousarray(a, dtype=np.uint16) for a in experts(e))
    else:
        W1, W3, W2 = experts
        for e in used:
            keep[e] = tuple(np.ascontiguousarray(a, dtype=np.uint16) for a in (W1[e], W3[e], W2[e]))
    for e, (a1, a3, a2) in keep.items():
        assert a1.shape == (d, f) and a3.shape == (d, f) and a2.shape == (f, d)
    P = ctypes.c_void_p * E
    t1, t3, t2 = P(), P(), P()
    for e, (a1, a3, a2) in keep.items():
        t1[e], t3[e], t2[e] = a1.ctypes.data, a3.ctypes.data, a2.ctypes.data
    out = np.empty((toks.size, d), dtype=np.float64)
    _check(lib.oracle_moe_tokens(_ptr(x), d, _ptr(toks), toks.size, k, _ptr(idx), _ptr(w), t1, t3, t2, f,
                                 _ptr(out)), "moe_tokens")
    return out


def moe_token(xrow, idx_row, w_row, experts, d: int, f: int) -> np.ndarray:
    """One token's layer output (fp64 [d]) with the expert columns shared over threads
    (``oracle_moe_token``)."""
    lib = _load()
    xrow = np.ascontiguousarray(xrow, dtype=np.uint16)
    ib = np.ascontiguousarray(idx_row, dtype=np.int32)
    wb = np.ascontiguousarray(w_row, dtype=np.float64)
    W1, W3, W2 = experts
    E = W1.shape[0]
    keep = [tuple(np.ascontiguousarray(a, dtype=np.uint16) for a in (W1[e], W3[e], W2[e])) for e in range(E)]
    P = ctypes.c_void_p * E
    t1, t3, t2 = P(*[a[0].ctypes.data for a in keep]), P(*[a[1].ctypes.data for a in keep]), \
        P(*[a[2].ctypes.data for a in keep])
    o = np.empty(d, dtype=np.float64)
    _check(lib.oracle_moe_token(_ptr(xrow), ib.size, _ptr(ib), _ptr(wb), t1, t3, t2, d, f, _ptr(o)), "moe_token")
    return o


def forward(x, Wr, bias, W1, W3, W2, k):
    """Whole layer for every token (small sizes): routing dict plus ``out`` fp64 [B, d]."""
    r = routing(x, Wr, bias, k)
    B, d = x.shape
    f = W1.shape[2]
    r["out"] = moe_tokens(x, range(B), r["topk_idx"], r["topk_w"], (W1, W3, W2), d, f) if B else \
        np.zeros((0, d), dtype=np.float64)
    return r
