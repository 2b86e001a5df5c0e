"""Seeded synthetic inputs for the draft-calibration workloads.

Holds no arithmetic of the method: it only maps (seed, tensor tag, flat index) to numbers, through
the C generator in ``synth.c`` (SplitMix64 counter streams, Box-Muller normals in fp64, round to
nearest even to fp32 then to bf16).  The GPU tests, the bench and the CPU oracle all draw their
inputs from here; nothing here imports either side.

Workload recipes follow the shapes the pages pin for the Markov head and the Selector:
vocabulary 151936 with rank 256 (the 77.8 M-parameter count of W1 + W2 in the DSpark overview,
"DSpark vs DFlash 2"), draft block K = 16 and batch 128 (the DSpark overview, "The Markov head").
The values themselves are synthetic stand-ins for trained weights and real draft logits.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

TAG = dict(U=1, W1=2, W2=3, A=4, Bemb=5, h=6, Wg=7, anchor=8, hot=9, Hd=10, conf=11)

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first (__graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, i32, dbl, vp = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int,
                                       ctypes.c_double, ctypes.c_void_p)
        lib.synth_splitmix.argtypes = [u64, u32, u64]
        lib.synth_splitmix.restype = u64
        lib.synth_normal.argtypes = [u64, u32, u64]
        lib.synth_normal.restype = dbl
        lib.synth_normal_f32.argtypes = [u64, u32, i64, dbl, vp]
        lib.synth_normal_bf16.argtypes = [u64, u32, i64, dbl, vp]
        lib.synth_logits.argtypes = [u64, u32, u32, i64, i32, i32, dbl, dbl, vp]
        lib.synth_tokens.argtypes = [u64, u32, i64, i32, vp]
        lib.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.synth_f32_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def splitmix(seed: int, tag: int, i: int) -> int:
    return int(_load().synth_splitmix(seed, tag, i))


def normal_f32(seed: int, tag: int, shape, sigma: float) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tag, out.size, sigma, out.ctypes.data)
    return out


def normal_bf16(seed: int, tag: int, shape, sigma: float) -> np.ndarray:
    """bf16 values as raw uint16 bit patterns."""
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tag, out.size, sigma, out.ctypes.data)
    return out


def logits(seed: int, rows_shape, V: int, n_hot: int, scale: float = 4.0, boost: float = 8.0) -> np.ndarray:
    """Base logits: scale * N(0,1) + boost on n_hot distinct ids per row, fp32, shape rows_shape + (V,)."""
    shape = tuple(rows_shape) + (V,)
    out = np.empty(shape, dtype=np.float32)
    rows = int(np.prod(rows_shape)) if len(rows_shape) else 1
    _load().synth_logits(seed, TAG["U"], TAG["hot"], rows, V, n_hot, scale, boost, out.ctypes.data)
    return out


def tokens(seed: int, tag: int, n: int, V: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_tokens(seed, tag, n, V, out.ctypes.data)
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bits (vectorised copy of the generator's rounding)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------------------------------------
# workloads
# ------------------------------------------------------------------------------------------------

F32, BF16 = 0, 1
GREEDY, SAMPLE = 0, 1


@dataclass
class Workload:
    """One seeded input set.  Arrays are host numpy arrays:

    U [B,K,V] f32; W1 [V,r]; W2 [r,V] (pages' orientation); W2T = W2 transposed [V,r];
    weights are float32 (wdtype F32) or uint16 bf16 bits (wdtype BF16); anchor [B] int32;
    h [B,K,D] bf16 bits and Wg [D,r] bf16 bits when gated; A/Bemb [V,r] for the Selector.
    """
    name: str
    B: int
    K: int
    V: int
    r: int
    wdtype: int
    mode: int
    seed: int
    noise_seed: int
    temperature: float
    U: np.ndarray
    W1: np.ndarray
    W2: np.ndarray
    anchor: np.ndarray
    h: Optional[np.ndarray] = None
    Wg: Optional[np.ndarray] = None
    D: int = 0
    topk: int = 16
    extra: dict = field(default_factory=dict)

    @property
    def W2T(self) -> np.ndarray:
        if "W2T" not in self.extra:
            self.extra["W2T"] = np.ascontiguousarray(self.W2.T)
        return self.extra["W2T"]


def _weights(seed, tag, shape, sigma, wdtype):
    return normal_f32(seed, tag, shape, sigma) if wdtype == F32 else normal_bf16(seed, tag, shape, sigma)


def make(B: int, K: int, V: int, r: int, *, wdtype: int = BF16, sigma_w: float = 0.02, n_hot: int = 16,
         u_scale: float = 4.0, u_boost: float = 8.0, mode: int = GREEDY, seed: int = 0xD5A10000,
         noise_seed: int = 0x5EED, temperature: float = 1.0, anchor_zero: bool = False, D: int = 0,
         sigma_h: float = 1.0, sigma_g: float = 0.02, name: str = "custom") -> Workload:
    """Generic recipe: U = u_scale*z + u_boost*[n_hot hot ids per row]; W1 [V,r] and W2 [r,V] ~ N(0, sigma_w)
    (sigma is the standard deviation); anchors uniform in [0,V) unless anchor_zero; with D > 0 also
    hidden states h [B,K,D] ~ N(0, sigma_h) and gate weights Wg [D,r] ~ N(0, sigma_g), both bf16."""
    U = logits(seed, (B, K), V, min(n_hot, V), u_scale, u_boost)
    W1 = _weights(seed, TAG["W1"], (V, r), sigma_w, wdtype)
    W2 = _weights(seed, TAG["W2"], (r, V), sigma_w, wdtype)
    anchor = np.zeros(B, np.int32) if anchor_zero else tokens(seed, TAG["anchor"], B, V)
    h = Wg = None
    if D > 0:
        h = normal_bf16(seed, TAG["h"], (B, K, D), sigma_h)
        Wg = normal_bf16(seed, TAG["Wg"], (D, r), sigma_g)
    return Workload(name=name, B=B, K=K, V=V, r=r, wdtype=wdtype, mode=mode, seed=seed, noise_seed=noise_seed,
                    temperature=temperature, U=U, W1=W1, W2=W2, anchor=anchor, h=h, Wg=Wg, D=D)


# The five measured shapes.  Seeds are 0xD5A10000 + index.
WORKLOADS = {
    # B=1, K=4, V=512, r=16, all fp32, 8 hot ids per row, anchor 0, greedy
    "tiny": dict(B=1, K=4, V=512, r=16, wdtype=F32, sigma_w=0.1, n_hot=8, anchor_zero=True, mode=GREEDY,
                 seed=0xD5A10001),
    # B=1, K=16, V=151936, r=256, bf16 weights, greedy (GEMV-shaped step)
    "batch1": dict(B=1, K=16, V=151936, r=256, wdtype=BF16, sigma_w=0.02, n_hot=16, mode=GREEDY,
                   seed=0xD5A10002),
    # B=128, K=16, V=151936, r=256, sampling at T=1 (the serving batch)
    "serving": dict(B=128, K=16, V=151936, r=256, wdtype=BF16, sigma_w=0.02, n_hot=16, mode=SAMPLE,
                    seed=0xD5A10003),
    # top-16 Selector, ungated, greedy walk (A := W1, Bemb := W2^T of this seed)
    "selector": dict(B=128, K=16, V=151936, r=256, wdtype=BF16, sigma_w=0.02, n_hot=16, mode=GREEDY,
                     seed=0xD5A10004),
    # gated: B=64, K=16, V=129280, r=256, D=4096
    "gated": dict(B=64, K=16, V=129280, r=256, wdtype=BF16, sigma_w=0.02, n_hot=16, mode=GREEDY,
                  seed=0xD5A10005, D=4096, sigma_h=1.0, sigma_g=0.02),
}


def workload(name: str, **overrides) -> Workload:
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return make(name=name, **cfg)


def strong(name: str, **overrides) -> Workload:
    """Parity-only strong-bias variant of a workload: weights ~ N(0, 0.25) at r = 256 (N(0, 0.5) at
    r = 16), so the bias has standard deviation about 1, and U = z + 2*[hot]."""
    cfg = dict(WORKLOADS[name])
    r = overrides.get("r", cfg["r"])
    cfg.update(sigma_w=(1.0 / np.sqrt(np.sqrt(r))), u_scale=1.0, u_boost=2.0)
    cfg.update(overrides)
    return make(name=name + "-strong", **cfg)
