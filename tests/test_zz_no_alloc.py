"""The allocation-free draft (dspark_markov_draft_noalloc), called through the C ABI, against dspark_markov_draft.

Both run the same kernels on the same inputs, the first with the library's own scratch array and the second
with a caller workspace, so tokens and log-probabilities must be bit-identical.  Two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents), and the host-side refusals."""
import ctypes

import numpy as np
import pytest
import torch

import synth as S
from helpers import host, t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


def _noalloc_abi(D, w, mode, seed, T, tokens, logprobs):
    """The C-ABI call with raw device pointers (no binding logic in between)."""
    lib = D.library()
    U, W1, W2T, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    wd = D.DSPARK_BF16 if w.W1.dtype == np.uint16 else D.DSPARK_F32
    vp = ctypes.c_void_p
    rc = lib.dspark_markov_draft_noalloc(vp(U.data_ptr()), vp(W1.data_ptr()), vp(W2T.data_ptr()), wd, D.DSPARK_W2_VR,
                                         vp(anc.data_ptr()), None, w.B, w.K, w.V, w.r, mode, seed, float(T),
                                         vp(tokens.data_ptr()), vp(logprobs.data_ptr()),
                                         vp(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return rc


CASES = [  # (workload, B, K, V, r, mode, weight dtype): the full serving round, then smaller ones
    ("serving", None, None, None, None, S.SAMPLE, S.BF16),
    ("serving", 40, 3, 2000, 128, S.SAMPLE, S.BF16),  # the half-block form
    ("serving", 1, 3, 3000, 256, S.GREEDY, S.BF16),   # one row at r = 256: the resident round
    ("serving", 16, 3, 3000, 256, S.GREEDY, S.BF16),  # up to 64 rows at r = 256: the matrix-core resident round
    ("serving", 5, 3, 3000, 64, S.GREEDY, S.BF16),
    ("serving", 3, 2, 1001, 24, S.SAMPLE, S.F32),
]


def test_noalloc_equals_workspace_draft_on_consecutive_calls(D):
    for cfg, B, K, V, r, mode, wd in CASES:
        kw = {} if B is None else dict(B=B, K=K, V=V, r=r, wdtype=wd, mode=mode)
        w = S.workload(cfg, **kw)
        print(f"[no-alloc] B={w.B} K={w.K} V={w.V} r={w.r} mode={mode}", flush=True)
        T = 0.9 if mode == S.SAMPLE else 1.0
        tokens = torch.full((w.B, w.K), -7, dtype=torch.int32, device="cuda")
        logprobs = torch.full((w.B, w.K), 7.0, dtype=torch.float32, device="cuda")
        rc = _noalloc_abi(D, w, mode, w.noise_seed, T, tokens, logprobs)
        assert rc == D.DSPARK_OK, D.library().dspark_last_error()
        ref_tok, ref_lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), mode=mode,
                                                seed=w.noise_seed, temperature=T)
        assert np.array_equal(host(tokens), host(ref_tok))
        assert np.array_equal(host(logprobs), host(ref_lp))


def test_noalloc_refusals(D):
    lib = D.library()
    assert lib.dspark_markov_noalloc_max_bytes() == 16 << 20
    w = S.workload("serving", B=4, K=2, V=512, r=32, mode=S.GREEDY)
    U, W1, W2, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2), t_i32(w.anchor)
    tok = torch.empty((w.B, w.K), dtype=torch.int32, device="cuda")
    vp = ctypes.c_void_p
    args = [vp(U.data_ptr()), vp(W1.data_ptr()), vp(W2.data_ptr()), D.DSPARK_BF16]
    tail = [vp(anc.data_ptr()), None, w.B, w.K, w.V, w.r, 0, 0, 1.0, vp(tok.data_ptr()), None, None]
    # a bf16 W2 stored [r, V] would need its transposed copy in the scratch
    assert lib.dspark_markov_draft_noalloc(*args, D.DSPARK_W2_RV, *tail) == D.DSPARK_EUNSUPPORTED
    # a batch whose workspace exceeds the scratch array
    big = list(tail)
    big[2], big[3] = 4096, 16
    assert lib.dspark_markov_draft_noalloc(*args, D.DSPARK_W2_VR, *big) == D.DSPARK_EUNSUPPORTED
