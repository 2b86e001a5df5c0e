"""Python access to the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the bench's CPU-baseline
leg, never by the product library.  It does not import the GPU package, and the GPU package does not
import it.  Arguments are numpy arrays (weights as float32 or as uint16 bf16 bits); outputs are numpy
arrays.  See ``oracle.c`` for the definitions and their sources on the pages.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB_PATH lets the mutation tests load a deliberately broken copy in a child process
_LIB_PATH = os.environ.get("ORACLE_LIB_PATH") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
W2_RV, W2_VR = 0, 1
GREEDY, SAMPLE = 0, 1


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first (__graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, u32, u64, dbl, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64,
                                       ctypes.c_double, ctypes.c_void_p)
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_num_threads.argtypes = [i32]
        lib.oracle_fmix32.argtypes = [u32]
        lib.oracle_fmix32.restype = u32
        lib.oracle_noise_bits.argtypes = [u64, u32, u32, u32]
        lib.oracle_noise_bits.restype = u32
        lib.oracle_noise_uniform.argtypes = [u64, u32, u32, u32]
        lib.oracle_noise_uniform.restype = dbl
        lib.oracle_gumbel.argtypes = [u64, u32, u32, u32]
        lib.oracle_gumbel.restype = dbl
        lib.oracle_noise_fill.argtypes = [u64, u32, u32, u32, i64, vp, vp]
        lib.oracle_gate.argtypes = [vp, vp, i32, i32, i32, vp]
        lib.oracle_confidence.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp, i32, i32, vp, vp]
        lib.oracle_schedule_greedy.argtypes = [vp, vp, i32, i32, vp]
        lib.oracle_schedule_greedy.restype = dbl
        lib.oracle_schedule_best.argtypes = [vp, vp, i32, i32, vp]
        lib.oracle_schedule_best.restype = dbl
        lib.oracle_markov_draft.argtypes = [vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, dbl,
                                            vp, vp, i32, vp, vp, vp, vp, vp, vp, dbl]
        lib.oracle_markov_logits.argtypes = [vp, i64, vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, i32, vp]
        lib.oracle_topk.argtypes = [vp, i64, i32, i32, i32, vp, vp]
        lib.oracle_markov_restricted.argtypes = [vp, vp, vp, i32, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 u64, dbl, vp, vp, i32, vp, vp, vp, vp, vp, dbl]
        lib.oracle_selector_draft.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, u64, dbl,
                                              vp, i32, vp, vp, vp, vp, vp]
        lib.oracle_enumerate_paths.argtypes = [vp, vp, vp, i32, i32, i32, vp, i32, i32, i32, dbl, vp]
        lib.oracle_enumerate_paths.restype = i32
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _w(a):
    """Weights as stored: float32 (F32) or uint16 bf16 bits (BF16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"weights must be float32 or uint16 bf16 bits, got {a.dtype}")


def _rows(rows: Optional[Sequence[int]]):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    return r, int(r.size)


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int):
    """Threads for the oracle's later parallel loops."""
    _load().oracle_set_num_threads(int(n))


# --------------------------------------------------------------------------------------------- noise

def fmix32(h: int) -> int:
    return int(_load().oracle_fmix32(h & 0xFFFFFFFF))


def noise_bits(seed: int, row: int, pos: int, v: int) -> int:
    return int(_load().oracle_noise_bits(seed, row, pos, v))


def noise_uniform(seed: int, row: int, pos: int, v: int) -> float:
    return float(_load().oracle_noise_uniform(seed, row, pos, v))


def gumbel(seed: int, row: int, pos: int, v: int) -> float:
    return float(_load().oracle_gumbel(seed, row, pos, v))


def noise_fill(seed: int, row: int, pos: int, v0: int, n: int):
    """(uniforms, gumbels) of ids v0 .. v0+n-1 at (row, pos), float64 arrays."""
    u = np.empty(n, np.float64)
    g = np.empty(n, np.float64)
    _load().oracle_noise_fill(seed, row, pos, v0, n, _ptr(u), _ptr(g))
    return u, g


# ---------------------------------------------------------------------------------------------- gate

def gate(h: np.ndarray, Wg: np.ndarray) -> np.ndarray:
    """H = sigmoid(h Wg) in fp64; h [..., D] bf16 bits, Wg [D, r] bf16 bits -> [..., r] float64."""
    h = _c(h, np.uint16)
    Wg = _c(Wg, np.uint16)
    D, r = Wg.shape
    rows = h.size // D
    H = np.empty(h.shape[:-1] + (r,), dtype=np.float64)
    _load().oracle_gate(_ptr(h), _ptr(Wg), rows, D, r, _ptr(H))
    return H


# ---------------------------------------------------------------------------------------- confidence

def confidence(h, w, W1, anchor, tokens):
    """c_k = sigmoid(w_h . h_k + w_m . W1[x_{k-1}]) and the prefix survival a_k = prod_{i<=k} c_i, fp64.
    h [B, K, D] bf16 bits; w [D + r] float32 (h part, then W1 part); W1 [V, r] float32 or bf16 bits;
    anchor [B]; tokens [B, K] (x_{-1} is the anchor).  Returns (conf, survival), each [B, K] float64."""
    h = _c(h, np.uint16)
    B, K, D = h.shape
    W1, wd = _w(W1)
    r = W1.shape[1]
    w = _c(w, np.float32)
    assert w.shape == (D + r,)
    anchor = _c(anchor, np.int32)
    tokens = _c(tokens, np.int32)
    conf = np.empty((B, K), np.float64)
    surv = np.empty((B, K), np.float64)
    _load().oracle_confidence(_ptr(h), D, _ptr(w), _ptr(W1), wd, r, _ptr(anchor), _ptr(tokens), B, K, _ptr(conf),
                              _ptr(surv))
    return conf, surv


# ---------------------------------------------------------------------------------------- scheduling

def schedule_greedy(a, sps):
    """Greedy load-aware prefix scheduling: a [R, K] prefix survival (float32), sps [R (K + 1) + 1] steps per
    second by target batch size.  Returns (lengths [R] int32, Theta)."""
    a = _c(a, np.float32)
    R, K = a.shape
    sps = _c(sps, np.float32)
    assert sps.shape == (R * (K + 1) + 1,)
    lengths = np.empty(R, np.int32)
    theta = _load().oracle_schedule_greedy(_ptr(a), _ptr(sps), R, K, _ptr(lengths))
    return lengths, theta


def schedule_best(a, sps):
    """Brute force over all prefix-length vectors ((K + 1)^R <= 2^22): (lengths [R], best Theta)."""
    a = _c(a, np.float32)
    R, K = a.shape
    sps = _c(sps, np.float32)
    lengths = np.empty(R, np.int32)
    theta = _load().oracle_schedule_best(_ptr(a), _ptr(sps), R, K, _ptr(lengths))
    return lengths, theta


# -------------------------------------------------------------------------------------------- markov

REACH_EPS = 1e-2  # perturbation of every key / log-mass under which a differing token is still accepted


def markov_draft(U, W1, W2, anchor, *, w2_layout=W2_RV, H=None, mode=GREEDY, seed=0, temperature=1.0,
                 follow=None, rows=None, eps=REACH_EPS):
    """Full-vocabulary Markov head over K positions (fp64).  Returns a dict of [B,K] arrays:
    tokens, logprobs, margins, best_logit, and lp_follow and reach when ``follow`` is given (reach: the
    follow token is the pick, or a perturbation of at most ``eps`` of every key selects it).  Rows not
    listed in ``rows`` are left as -1 / nan."""
    U = _c(U, np.float32)
    B, K, V = U.shape
    W1, wd = _w(W1)
    W2, wd2 = _w(W2)
    assert wd == wd2
    r = W1.shape[1]
    anchor = _c(anchor, np.int32)
    H = _c(H, np.float64)
    follow = _c(follow, np.int32)
    rr, nr = _rows(rows)
    tokens = np.full((B, K), -1, np.int32)
    lp = np.full((B, K), np.nan)
    mg = np.full((B, K), np.nan)
    bl = np.full((B, K), np.nan)
    lpf = np.full((B, K), np.nan) if follow is not None else None
    reach = np.full((B, K), -1, np.int32) if follow is not None else None
    _load().oracle_markov_draft(_ptr(U), _ptr(W1), _ptr(W2), wd, w2_layout, _ptr(anchor), _ptr(H), B, K, V, r,
                                mode, seed, float(temperature), _ptr(follow), _ptr(rr), nr, _ptr(tokens), _ptr(lp),
                                _ptr(mg), _ptr(lpf), _ptr(bl), _ptr(reach), float(eps))
    out = dict(tokens=tokens, logprobs=lp, margins=mg, best_logit=bl)
    if lpf is not None:
        out["lp_follow"] = lpf
        out["reach"] = reach
    return out


def markov_logits(Uk, W1, W2, prev, *, w2_layout=W2_RV, Hk=None, rows=None):
    """Calibrated logits of one position, [B, V] float64: Uk [B, V] + (W1[prev] (.) Hk) W2."""
    Uk = _c(Uk, np.float32)
    B, V = Uk.shape
    W1, wd = _w(W1)
    W2, _ = _w(W2)
    r = W1.shape[1]
    prev = _c(prev, np.int32)
    Hk = _c(Hk, np.float64)
    rr, nr = _rows(rows)
    out = np.full((B, V), np.nan)
    _load().oracle_markov_logits(_ptr(Uk), V, _ptr(W1), _ptr(W2), wd, w2_layout, _ptr(prev), _ptr(Hk), B, V, r,
                                 _ptr(rr), nr, _ptr(out))
    return out


def markov_restricted(U, W1, W2, anchor, cand, *, w2_layout=W2_RV, H=None, mode=GREEDY, seed=0,
                      temperature=1.0, follow=None, rows=None, eps=REACH_EPS):
    """The head restricted to the candidate sets cand [B, K, topk] (fp64); outputs as markov_draft."""
    U = _c(U, np.float32)
    B, K, V = U.shape
    W1, wd = _w(W1)
    W2, _ = _w(W2)
    r = W1.shape[1]
    cand = _c(cand, np.int32)
    topk = cand.shape[-1]
    anchor = _c(anchor, np.int32)
    H = _c(H, np.float64)
    follow = _c(follow, np.int32)
    rr, nr = _rows(rows)
    tokens = np.full((B, K), -1, np.int32)
    lp = np.full((B, K), np.nan)
    mg = np.full((B, K), np.nan)
    lpf = np.full((B, K), np.nan) if follow is not None else None
    reach = np.full((B, K), -1, np.int32) if follow is not None else None
    _load().oracle_markov_restricted(_ptr(U), _ptr(W1), _ptr(W2), wd, w2_layout, _ptr(anchor), _ptr(H), _ptr(cand),
                                     B, K, V, r, topk, mode, seed, float(temperature), _ptr(follow), _ptr(rr), nr,
                                     _ptr(tokens), _ptr(lp), _ptr(mg), _ptr(lpf), _ptr(reach), float(eps))
    out = dict(tokens=tokens, logprobs=lp, margins=mg)
    if lpf is not None:
        out["lp_follow"] = lpf
        out["reach"] = reach
    return out


# ----------------------------------------------------------------------------------------- selector

def topk(U, k):
    """Top-k ids (value desc, id asc) of every row of U [..., V]: (idx int32, val float32)."""
    U = _c(U, np.float32)
    V = U.shape[-1]
    rows = U.size // V
    idx = np.empty(U.shape[:-1] + (k,), np.int32)
    val = np.empty(U.shape[:-1] + (k,), np.float32)
    _load().oracle_topk(_ptr(U), V, rows, V, k, _ptr(idx), _ptr(val))
    return idx, val


def selector_draft(U, A, Bemb, anchor, *, H=None, topk=16, mode=GREEDY, seed=0, temperature=1.0, rows=None):
    """Selector step by step: candidates, all pair tables, walk.  Returns tokens/logprobs/margins [B,K],
    cand [B,K,topk] and tables [B, topk + (K-1)*topk*topk] (float64)."""
    U = _c(U, np.float32)
    B, K, V = U.shape
    A, wd = _w(A)
    Bemb, _ = _w(Bemb)
    r = A.shape[1]
    anchor = _c(anchor, np.int32)
    H = _c(H, np.float64)
    rr, nr = _rows(rows)
    tokens = np.full((B, K), -1, np.int32)
    lp = np.full((B, K), np.nan)
    mg = np.full((B, K), np.nan)
    cand = np.full((B, K, topk), -1, np.int32)
    tables = np.full((B, topk + (K - 1) * topk * topk), np.nan)
    _load().oracle_selector_draft(_ptr(U), _ptr(A), _ptr(Bemb), wd, _ptr(anchor), _ptr(H), B, K, V, r, topk, mode,
                                  seed, float(temperature), _ptr(rr), nr, _ptr(tokens), _ptr(lp), _ptr(mg),
                                  _ptr(cand), _ptr(tables))
    return dict(tokens=tokens, logprobs=lp, margins=mg, cand=cand, tables=tables)


def enumerate_paths(U_row, W1, W2, anchor, *, w2_layout=W2_RV, H_row=None, temperature=1.0):
    """log q of every path of one row (U_row [K, V]); returns float64 [V]*K array indexed by the path."""
    U_row = _c(U_row, np.float32)
    K, V = U_row.shape
    W1, wd = _w(W1)
    W2, _ = _w(W2)
    r = W1.shape[1]
    H_row = _c(H_row, np.float64)
    out = np.empty((V,) * K, np.float64)
    rc = _load().oracle_enumerate_paths(_ptr(U_row), _ptr(W1), _ptr(W2), wd, w2_layout, int(anchor), _ptr(H_row),
                                        K, V, r, float(temperature), _ptr(out))
    if rc != 0:
        raise ValueError("enumeration needs V <= 64, K <= 32 and V**K <= 2**20")
    return out
