"""Python binding of libdspark (C ABI in include/dspark.h).

Thin marshalling only: every function takes torch tensors on the GPU, checks dtypes and shapes, and
passes raw device pointers, sizes and the current HIP stream to the library function of the same
name.  All computation happens in the library's HIP kernels.  Outputs and workspaces that the caller
does not supply are allocated with torch (device memory plumbing).

The library is loaded at import; if it is missing or cannot be loaded, the import fails.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libdspark.so")

DSPARK_OK, DSPARK_EINVAL, DSPARK_EUNSUPPORTED, DSPARK_EWORKSPACE, DSPARK_EDEVICE = 0, 1, 2, 3, 4
DSPARK_F32, DSPARK_BF16 = 0, 1
DSPARK_W2_RV, DSPARK_W2_VR = 0, 1
DSPARK_GREEDY, DSPARK_SAMPLE = 0, 1


class DsparkError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {_status_name(status)} ({detail})")
        self.status = status


def _load_lib():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libdspark is not built: {LIB_PATH} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, u64, f32, sz, vp, cp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_char_p)
    sig = {
        "dspark_abi_version": ([], i32),
        "dspark_status_str": ([i32], cp),
        "dspark_last_error": ([], cp),
        "dspark_markov_workspace_bytes": ([i32, i32, i32, i32, i32, i32], sz),
        "dspark_markov_draft": ([vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp, sz, vp], i32),
        "dspark_markov_draft_timed": ([vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp, sz,
                                       vp, vp, vp, vp], i32),
        "dspark_markov_draft_logits": ([vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp, vp,
                                        sz, vp], i32),
        "dspark_markov_status": ([vp, sz, i32, i32, vp], i32),
        "dspark_markov_noalloc_max_bytes": ([], sz),
        "dspark_markov_draft_noalloc": ([vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp],
                                        i32),
        "dspark_set_spin_limit": ([ctypes.c_uint32], None),
        "dspark_set_cooperative_launch": ([i32], None),
        "dspark_markov_draft_confidence": ([vp, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, i32, vp,
                                            vp, vp, vp, vp, vp, sz, vp], i32),
        "dspark_markov_step": ([vp, i64, vp, vp, i32, i32, vp, vp, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp, vp, sz,
                                vp], i32),
        "dspark_markov_logits": ([vp, i64, vp, vp, i32, i32, vp, vp, i32, i32, i32, vp, vp, sz, vp], i32),
        "dspark_pack_w2": ([vp, i32, i32, i32, vp, vp], i32),
        "dspark_stream_read": ([vp, sz, vp, sz, vp, vp], i32),
        "dspark_gate": ([vp, vp, i32, i32, i32, vp, vp, sz, vp], i32),
        "dspark_gate_workspace_bytes": ([i32, i32, i32], sz),
        "dspark_topk_workspace_bytes": ([i32, i32, i32], sz),
        "dspark_topk": ([vp, i64, i32, i32, i32, vp, vp, vp, sz, vp], i32),
        "dspark_selector_workspace_bytes": ([i32, i32, i32, i32, i32], sz),
        "dspark_schedule_prefixes": ([vp, vp, i32, i32, vp, vp, vp], i32),
        "dspark_selector_draft": ([vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32, i32, u64, f32, vp, vp, vp, vp, vp, sz,
                                   vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


_lib = _load_lib()


def _status_name(status: int) -> str:
    return _lib.dspark_status_str(status).decode()


def _check(status: int, where: str):
    if status != DSPARK_OK:
        raise DsparkError(status, where, _lib.dspark_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, has {t.dim()}")
    return t


def _wdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise TypeError(f"weights must be bfloat16 or float32, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Allocations of a call that enqueues on ``stream`` are made with that stream current, so the caching
    allocator orders their reuse after the call's kernels (a temporary workspace is freed on return)."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def dspark_abi_version() -> int:
    return int(_lib.dspark_abi_version())


def dspark_markov_workspace_bytes(B: int, K: int, V: int, r: int, wdtype: int, w2_layout: int) -> int:
    return int(_lib.dspark_markov_workspace_bytes(B, K, V, r, wdtype, w2_layout))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device), nbytes


def dspark_markov_draft(U, W1, W2, anchor, *, w2_layout=DSPARK_W2_VR, H=None, mode=DSPARK_GREEDY, seed=0,
                        temperature=1.0, tokens=None, logprobs=None, want_logprobs=True, workspace=None, stream=None):
    """K-position Markov-head draft.  U [B,K,V] fp32; W1 [V,r]; W2 [V,r] (DSPARK_W2_VR) or [r,V] (DSPARK_W2_RV);
    anchor [B] int32; H [B,K,r] fp32 or None.  Returns (tokens [B,K] int32, logprobs [B,K] fp32 or None)."""
    with _on(stream):
        _dev(U, "U", torch.float32, 3)
        B, K, V = U.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(anchor, "anchor", torch.int32, 1)
        if H is not None:
            _dev(H, "H", torch.float32, 3)
        wd = _wdtype(W1)
        if tokens is None:
            tokens = torch.empty((B, K), dtype=torch.int32, device=U.device)
        if logprobs is None and want_logprobs:
            logprobs = torch.empty((B, K), dtype=torch.float32, device=U.device)
        ws, wsb = _workspace(dspark_markov_workspace_bytes(B, K, V, r, wd, w2_layout), U.device, workspace)
        _check(_lib.dspark_markov_draft(_p(U), _p(W1), _p(W2), wd, w2_layout, _p(anchor), _p(H), B, K, V, r, mode, seed,
                                        float(temperature), _p(tokens), _p(logprobs), _p(ws), wsb, _stream(stream)),
               "dspark_markov_draft")
        return tokens, logprobs


def dspark_markov_draft_logits(U, W1, W2, anchor, *, w2_layout=DSPARK_W2_VR, H=None, mode=DSPARK_GREEDY, seed=0,
                               temperature=1.0, workspace=None, stream=None):
    """Validation: dspark_markov_draft that also returns the calibrated logits [B, K, V] fp32 of every position
    along the drafted path, written by the whole-round kernel.  Returns (tokens, logprobs, logits)."""
    with _on(stream):
        _dev(U, "U", torch.float32, 3)
        B, K, V = U.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(anchor, "anchor", torch.int32, 1)
        if H is not None:
            _dev(H, "H", torch.float32, 3)
        wd = _wdtype(W1)
        tokens = torch.empty((B, K), dtype=torch.int32, device=U.device)
        logprobs = torch.empty((B, K), dtype=torch.float32, device=U.device)
        logits = torch.empty((B, K, V), dtype=torch.float32, device=U.device)
        ws, wsb = _workspace(dspark_markov_workspace_bytes(B, K, V, r, wd, w2_layout), U.device, workspace)
        _check(_lib.dspark_markov_draft_logits(_p(U), _p(W1), _p(W2), wd, w2_layout, _p(anchor), _p(H), B, K, V, r,
                                               mode, seed, float(temperature), _p(tokens), _p(logprobs), _p(logits),
                                               _p(ws), wsb, _stream(stream)), "dspark_markov_draft_logits")
        return tokens, logprobs, logits


def dspark_markov_draft_noalloc(U, W1, W2, anchor, tokens, logprobs, *, w2_layout=DSPARK_W2_VR, H=None,
                                mode=DSPARK_GREEDY, seed=0, temperature=1.0, stream=None):
    """dspark_markov_draft with the library's own scratch array instead of a workspace: the caller passes the
    outputs (tokens [B,K] int32, logprobs [B,K] fp32 or None); nothing is allocated."""
    _dev(U, "U", torch.float32, 3)
    B, K, V = U.shape
    _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
    _dev(W2, "W2", W1.dtype, 2)
    r = W1.shape[1]
    _dev(anchor, "anchor", torch.int32, 1)
    _dev(tokens, "tokens", torch.int32, 2)
    if logprobs is not None:
        _dev(logprobs, "logprobs", torch.float32, 2)
    if H is not None:
        _dev(H, "H", torch.float32, 3)
    _check(_lib.dspark_markov_draft_noalloc(_p(U), _p(W1), _p(W2), _wdtype(W1), w2_layout, _p(anchor), _p(H), B, K, V,
                                            r, mode, seed, float(temperature), _p(tokens), _p(logprobs),
                                            _stream(stream)), "dspark_markov_draft_noalloc")
    return tokens, logprobs


def dspark_markov_status(workspace, B, K, *, stream=None):
    """Device-side status of the last draft made with ``workspace`` (a uint8 device tensor): DSPARK_OK, or
    DSPARK_EDEVICE if a bounded wait of the whole-round kernel gave up.  Synchronises with the stream."""
    with _on(stream):
        return int(_lib.dspark_markov_status(_p(workspace), workspace.numel() * workspace.element_size(), B, K,
                                             _stream(stream)))


def dspark_set_cooperative_launch(on: bool):
    """Whole-round kernel launch for later calls: ordinary (default) or cooperative (guaranteed co-residency)."""
    _lib.dspark_set_cooperative_launch(1 if on else 0)


def dspark_set_spin_limit(sleeps: int):
    """Testing hook: bound of the round kernel's waits for later calls (0 restores the default)."""
    _lib.dspark_set_spin_limit(int(sleeps))


def dspark_markov_draft_confidence(U, W1, W2, anchor, h, conf_w, *, w2_layout=DSPARK_W2_VR, H=None, mode=DSPARK_GREEDY,
                                   seed=0, temperature=1.0, want_logprobs=True, workspace=None, stream=None):
    """Draft plus the confidence head: h [B,K,D] bf16, conf_w [D+r] fp32 (h part, then W1 part).  Returns
    (tokens, logprobs or None, conf [B,K] fp32, survival [B,K] fp32)."""
    with _on(stream):
        _dev(U, "U", torch.float32, 3)
        B, K, V = U.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(anchor, "anchor", torch.int32, 1)
        _dev(h, "h", torch.bfloat16, 3)
        _dev(conf_w, "conf_w", torch.float32, 1)
        if H is not None:
            _dev(H, "H", torch.float32, 3)
        D = h.shape[2]
        if tuple(h.shape[:2]) != (B, K) or conf_w.shape[0] != D + r:
            raise ValueError("h must be [B, K, D] and conf_w [D + r]")
        wd = _wdtype(W1)
        tokens = torch.empty((B, K), dtype=torch.int32, device=U.device)
        logprobs = torch.empty((B, K), dtype=torch.float32, device=U.device) if want_logprobs else None
        conf = torch.empty((B, K), dtype=torch.float32, device=U.device)
        surv = torch.empty((B, K), dtype=torch.float32, device=U.device)
        ws, wsb = _workspace(dspark_markov_workspace_bytes(B, K, V, r, wd, w2_layout), U.device, workspace)
        _check(_lib.dspark_markov_draft_confidence(_p(U), _p(W1), _p(W2), wd, w2_layout, _p(anchor), _p(H), B, K, V, r,
                                                   mode, seed, float(temperature), _p(h), D, _p(conf_w), _p(tokens),
                                                   _p(logprobs), _p(conf), _p(surv), _p(ws), wsb, _stream(stream)),
               "dspark_markov_draft_confidence")
        return tokens, logprobs, conf, surv


def dspark_markov_draft_timed(U, W1, W2, anchor, *, w2_layout=DSPARK_W2_VR, H=None, mode=DSPARK_GREEDY, seed=0,
                              temperature=1.0, tokens=None, logprobs=None, workspace=None, stream=None):
    """dspark_markov_draft plus contraction-kernel timing (HIP events on the same stream).
    Returns (tokens, logprobs, kernel_ms summed over the contraction launches, number of launches, round_ms)."""
    with _on(stream):
        _dev(U, "U", torch.float32, 3)
        B, K, V = U.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(anchor, "anchor", torch.int32, 1)
        if H is not None:
            _dev(H, "H", torch.float32, 3)
        wd = _wdtype(W1)
        if tokens is None:
            tokens = torch.empty((B, K), dtype=torch.int32, device=U.device)
        if logprobs is None:
            logprobs = torch.empty((B, K), dtype=torch.float32, device=U.device)
        ws, wsb = _workspace(dspark_markov_workspace_bytes(B, K, V, r, wd, w2_layout), U.device, workspace)
        kernel_ms = ctypes.c_float()
        launches = ctypes.c_int()
        round_ms = ctypes.c_float()
        _check(_lib.dspark_markov_draft_timed(_p(U), _p(W1), _p(W2), wd, w2_layout, _p(anchor), _p(H), B, K, V, r, mode,
                                              seed, float(temperature), _p(tokens), _p(logprobs), _p(ws), wsb,
                                              _stream(stream), ctypes.byref(kernel_ms), ctypes.byref(launches),
                                              ctypes.byref(round_ms)), "dspark_markov_draft_timed")
        return tokens, logprobs, float(kernel_ms.value), int(launches.value), float(round_ms.value)


def dspark_markov_step(U_k, W1, W2, prev, k, *, w2_layout=DSPARK_W2_VR, H_k=None, mode=DSPARK_GREEDY, seed=0,
                       temperature=1.0, workspace=None, stream=None):
    """One position with supplied predecessors.  U_k [B,V] fp32 (rows may be strided); prev [B] int32.
    Returns (tok [B], logprob [B], best_logit [B])."""
    with _on(stream):
        if not U_k.is_cuda or U_k.dtype != torch.float32 or U_k.dim() != 2 or U_k.stride(1) != 1:
            raise ValueError("U_k must be a GPU float32 [B, V] tensor with unit column stride")
        B, V = U_k.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(prev, "prev", torch.int32, 1)
        if H_k is not None:
            _dev(H_k, "H_k", torch.float32, 2)
        wd = _wdtype(W1)
        tok = torch.empty(B, dtype=torch.int32, device=U_k.device)
        lp = torch.empty(B, dtype=torch.float32, device=U_k.device)
        bl = torch.empty(B, dtype=torch.float32, device=U_k.device)
        ws, wsb = _workspace(dspark_markov_workspace_bytes(B, 1, V, r, wd, w2_layout), U_k.device, workspace)
        _check(_lib.dspark_markov_step(_p(U_k), U_k.stride(0), _p(W1), _p(W2), wd, w2_layout, _p(prev), _p(H_k), B, V, r,
                                       int(k), mode, seed, float(temperature), _p(tok), _p(lp), _p(bl), _p(ws), wsb,
                                       _stream(stream)), "dspark_markov_step")
        return tok, lp, bl


def dspark_markov_logits(U_k, W1, W2, prev, *, w2_layout=DSPARK_W2_VR, H_k=None, out=None, stream=None):
    """Calibrated logits of one position, [B, V] fp32 (validation path)."""
    with _on(stream):
        if not U_k.is_cuda or U_k.dtype != torch.float32 or U_k.dim() != 2 or U_k.stride(1) != 1:
            raise ValueError("U_k must be a GPU float32 [B, V] tensor with unit column stride")
        B, V = U_k.shape
        _dev(W1, "W1", (torch.bfloat16, torch.float32), 2)
        _dev(W2, "W2", W1.dtype, 2)
        r = W1.shape[1]
        _dev(prev, "prev", torch.int32, 1)
        if H_k is not None:
            _dev(H_k, "H_k", torch.float32, 2)
        wd = _wdtype(W1)
        if out is None:
            out = torch.empty((B, V), dtype=torch.float32, device=U_k.device)
        need = V * r * W1.element_size() if w2_layout == DSPARK_W2_RV else 0
        ws, wsb = _workspace(need, U_k.device, None)
        _check(_lib.dspark_markov_logits(_p(U_k), U_k.stride(0), _p(W1), _p(W2), wd, w2_layout, _p(prev), _p(H_k), B, V, r,
                                         _p(out), _p(ws), wsb, _stream(stream)), "dspark_markov_logits")
        return out


def dspark_pack_w2(W2_rv, *, out=None, stream=None):
    """[r, V] -> [V, r] copy of W2."""
    with _on(stream):
        _dev(W2_rv, "W2", (torch.bfloat16, torch.float32), 2)
        r, V = W2_rv.shape
        if out is None:
            out = torch.empty((V, r), dtype=W2_rv.dtype, device=W2_rv.device)
        _check(_lib.dspark_pack_w2(_p(W2_rv), V, r, _wdtype(W2_rv), _p(out), _stream(stream)), "dspark_pack_w2")
        return out


def dspark_stream_read(a, b, sink, *, stream=None):
    """Reads the contiguous device tensors a and b once (measurement utility); sink: a 1-element int32 tensor."""
    with _on(stream):
        for t, n in ((a, "a"), (b, "b"), (sink, "sink")):
            if not (t.is_cuda and t.is_contiguous()):
                raise ValueError(f"{n} must be a contiguous device tensor")
        _check(_lib.dspark_stream_read(_p(a), a.numel() * a.element_size(), _p(b), b.numel() * b.element_size(), _p(sink),
                                       _stream(stream)), "dspark_stream_read")


def dspark_gate_workspace_bytes(rows: int, D: int, r: int) -> int:
    return int(_lib.dspark_gate_workspace_bytes(rows, D, r))


def dspark_gate(h, Wg, *, out=None, workspace=None, split_k=True, stream=None):
    """H = sigmoid(h Wg): h [..., D] bf16, Wg [D, r] bf16 -> [..., r] fp32.  split_k=False (or sizes the split
    form does not take) runs the single-launch form without a workspace."""
    with _on(stream):
        _dev(h, "h", torch.bfloat16)
        _dev(Wg, "Wg", torch.bfloat16, 2)
        D, r = Wg.shape
        if h.shape[-1] != D:
            raise ValueError("h's last dim must equal Wg's first")
        rows = h.numel() // D
        if out is None:
            out = torch.empty(tuple(h.shape[:-1]) + (r,), dtype=torch.float32, device=h.device)
        nbytes = int(_lib.dspark_gate_workspace_bytes(rows, D, r)) if split_k else 0
        ws, wsb = (_workspace(nbytes, h.device, workspace) if nbytes > 0 else (None, 0))
        _check(_lib.dspark_gate(_p(h), _p(Wg), rows, D, r, _p(out), _p(ws), wsb, _stream(stream)), "dspark_gate")
        return out


def dspark_topk(U, topk, *, want_values=True, stream=None):
    """Top-k ids (value desc, id asc) of every row of U [..., V] fp32 -> (idx int32, val fp32 or None)."""
    with _on(stream):
        _dev(U, "U", torch.float32)
        V = U.shape[-1]
        rows = U.numel() // V
        idx = torch.empty(tuple(U.shape[:-1]) + (topk,), dtype=torch.int32, device=U.device)
        val = torch.empty(tuple(U.shape[:-1]) + (topk,), dtype=torch.float32, device=U.device) if want_values else None
        nbytes = int(_lib.dspark_topk_workspace_bytes(rows, V, topk))
        ws, wsb = _workspace(nbytes, U.device, None)
        _check(_lib.dspark_topk(_p(U), V, rows, V, topk, _p(idx), _p(val), _p(ws), wsb, _stream(stream)), "dspark_topk")
        return idx, val


def dspark_selector_workspace_bytes(B, K, V, r, topk) -> int:
    return int(_lib.dspark_selector_workspace_bytes(B, K, V, r, topk))


def dspark_schedule_prefixes(survival, sps, *, stream=None):
    """Greedy load-aware prefix scheduling.  survival [R, K] fp32, sps [R (K + 1) + 1] fp32 (steps per second by
    target batch size).  Returns (lengths [R] int32, theta [1] fp32)."""
    with _on(stream):
        _dev(survival, "survival", torch.float32, 2)
        R, K = survival.shape
        _dev(sps, "sps", torch.float32, 1)
        if sps.shape[0] != R * (K + 1) + 1:
            raise ValueError("sps must have R (K + 1) + 1 entries")
        lengths = torch.empty((R,), dtype=torch.int32, device=survival.device)
        theta = torch.empty((1,), dtype=torch.float32, device=survival.device)
        _check(_lib.dspark_schedule_prefixes(_p(survival), _p(sps), R, K, _p(lengths), _p(theta), _stream(stream)),
               "dspark_schedule_prefixes")
        return lengths, theta


def dspark_selector_draft(U, A, Bemb, anchor, *, H=None, topk=16, mode=DSPARK_GREEDY, seed=0, temperature=1.0,
                          want_logprobs=True, want_cand=False, want_scores=False, workspace=None, stream=None):
    """Selector execution.  Returns dict(tokens, logprobs, cand, scores) (absent items are None)."""
    with _on(stream):
        _dev(U, "U", torch.float32, 3)
        B, K, V = U.shape
        _dev(A, "A", (torch.bfloat16, torch.float32), 2)
        _dev(Bemb, "Bemb", A.dtype, 2)
        r = A.shape[1]
        _dev(anchor, "anchor", torch.int32, 1)
        if H is not None:
            _dev(H, "H", torch.float32, 3)
        dev = U.device
        tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
        lp = torch.empty((B, K), dtype=torch.float32, device=dev) if want_logprobs else None
        cand = torch.empty((B, K, topk), dtype=torch.int32, device=dev) if want_cand else None
        scores = torch.empty((B, topk + (K - 1) * topk * topk), dtype=torch.float32, device=dev) if want_scores else None
        ws, wsb = _workspace(dspark_selector_workspace_bytes(B, K, V, r, topk), dev, workspace)
        _check(_lib.dspark_selector_draft(_p(U), _p(A), _p(Bemb), _wdtype(A), _p(anchor), _p(H), B, K, V, r, topk, mode,
                                          seed, float(temperature), _p(tokens), _p(lp), _p(cand), _p(scores), _p(ws), wsb,
                                          _stream(stream)), "dspark_selector_draft")
        return dict(tokens=tokens, logprobs=lp, cand=cand, scores=scores)


def library():
    """The loaded ctypes handle (for ABI-level tests)."""
    return _lib
