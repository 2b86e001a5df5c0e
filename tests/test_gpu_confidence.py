"""GPU parity of the confidence head and prefix survival (dspark_markov_draft_confidence) against the oracle
(DSpark overview, "Confidence-scheduled verification"): conf[b, k] = sigmoid(w_h . h_k + w_m . W1[x_{k-1}]) and
survival = the running product.  The oracle drafts its own tokens; rows whose GPU draft equals the oracle's
are compared (the others differ only at flagged near-ties and are covered by the draft parity tests)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S
from helpers import host, t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu

CONF_TOL = 1e-4  # fp32 dot products of D + r terms against fp64


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


def _h_and_w(B, K, Dm, r, seed, scale=0.05):
    rng = np.random.default_rng(seed)
    h = S.f32_to_bf16(rng.standard_normal((B, K, Dm)).astype(np.float32))
    w = (rng.standard_normal(Dm + r) * scale).astype(np.float32)
    return h, w


def _t_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


# (B, K, V, r, wdtype, D): bf16 [V, r] weights take the whole-round launch (the finalizer computes the head);
# fp32 weights and r = 512 go position by position, followed by the separate confidence launch
SHAPES = [(5, 4, 1000, 64, S.BF16, 256), (130, 3, 776, 32, S.BF16, 64), (3, 3, 300, 24, S.F32, 128),
          (2, 3, 600, 512, S.BF16, 512), (16, 6, 4096, 256, S.BF16, 4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d-K%d-V%d-r%d-%s-D%d" % (s[0], s[1], s[2], s[3],
                                                                                  "bf16" if s[4] == S.BF16 else "f32", s[5]))
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_confidence_parity(D, shape, mode):
    B, K, V, r, wd, Dm = shape
    w = S.strong("serving", B=B, K=K, V=V, r=r, wdtype=wd, mode=mode)
    h, cw = _h_and_w(B, K, Dm, r, seed=B * 7 + K)
    W2T = w.W2T
    tok, lp, conf, surv = D.dspark_markov_draft_confidence(t_f32(w.U), t_w(w.W1), t_w(W2T), t_i32(w.anchor), _t_bf16(h),
                                                           t_f32(cw), w2_layout=D.DSPARK_W2_VR, mode=mode,
                                                           seed=w.noise_seed, temperature=w.temperature)
    tok, conf, surv = host(tok), host(conf), host(surv)
    ref = O.markov_draft(w.U, w.W1, W2T, w.anchor, w2_layout=O.W2_VR, mode=mode, seed=w.noise_seed,
                         temperature=w.temperature)
    rconf, rsurv = O.confidence(h, cw, w.W1, w.anchor, ref["tokens"])
    same = np.all(tok == ref["tokens"], axis=1)
    assert same.mean() >= 0.75, same.mean()
    np.testing.assert_allclose(conf[same], rconf[same], rtol=0, atol=CONF_TOL)
    np.testing.assert_allclose(surv[same], rsurv[same], rtol=0, atol=CONF_TOL)
    np.testing.assert_allclose(surv, np.cumprod(conf, axis=1), rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("wd", [S.BF16, S.F32], ids=["whole-round", "per-position"])
def test_confidence_zero_weights(D, wd):
    """w = 0: every confidence is exactly 1/2 and survival 2^-(k+1) (fp32 represents these exactly)."""
    B, K, V, r, Dm = 4, 5, 512, 32, 64
    w = S.strong("serving", B=B, K=K, V=V, r=r, wdtype=wd)
    h, _ = _h_and_w(B, K, Dm, r, seed=1)
    cw = np.zeros(Dm + r, np.float32)
    _, _, conf, surv = D.dspark_markov_draft_confidence(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), _t_bf16(h),
                                                        t_f32(cw), w2_layout=D.DSPARK_W2_VR)
    assert np.all(host(conf) == 0.5)
    assert np.array_equal(host(surv), np.broadcast_to((0.5 ** np.arange(1, K + 1)).astype(np.float32), (B, K)))
