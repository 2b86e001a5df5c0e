"""GPU parity of the greedy load-aware prefix scheduler (dspark_schedule_prefixes) against the oracle (DSpark
overview, "Hardware-aware prefix scheduling"): the admitted prefix lengths are integers decided by fp64
comparisons on both sides, so they must be equal; Theta within fp32 output rounding."""
import numpy as np
import pytest
import torch

import oracle as O
from helpers import host, t_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


def _survival(R, K, seed):
    rng = np.random.default_rng(seed)
    return np.cumprod(rng.uniform(0.2, 0.999, (R, K)), axis=1).astype(np.float32)


def _curves(R, K, seed):
    B = np.arange(R * (K + 1) + 1, dtype=np.float64)
    n = R * (K + 1)
    yield "flat", np.full(n + 1, 3.0, np.float32)
    yield "linear", (100.0 - 90.0 * B / n).astype(np.float32)
    yield "knee", np.where(B <= R + n // 3, 50.0, 50.0 * (R + n // 3) / np.maximum(B, 1)).astype(np.float32)
    yield "bumpy", (60.0 - 40.0 * B / n + 4.0 * np.sin(B * 0.7 + seed)).clip(0.5).astype(np.float32)
    cliff = np.zeros(n + 1, np.float32)
    cliff[: R + 1] = 1.0
    yield "cliff", cliff


@pytest.mark.parametrize("R,K", [(1, 1), (3, 7), (4, 4), (128, 16), (64, 64), (4096, 1), (37, 13)])
def test_schedule_parity(D, R, K):
    a = _survival(R, K, seed=R * 31 + K)
    a[0, 0] = np.nan if R * K > 4 else a[0, 0]  # counts as 0 on both sides
    for name, sps in _curves(R, K, seed=R + K):
        lengths, theta = D.dspark_schedule_prefixes(t_f32(a), t_f32(sps))
        rl, rt = O.schedule_greedy(a, sps)
        assert np.array_equal(host(lengths), rl), name
        assert host(theta)[0] == pytest.approx(rt, rel=1e-6, abs=1e-6), name


def test_schedule_after_confidence(D):
    """End to end on the device: survival from the draft's confidence head feeds the scheduler.  Checked
    without an oracle (its parity is covered above on oracle inputs): lengths lie in [0, K], Theta recomputed
    on the host from the admitted prefixes matches the reported one, and admitting the next extension in the
    greedy order would not increase Theta."""
    import synth as S
    from helpers import t_i32, t_w
    B, K = 16, 8
    w = S.strong("serving", B=B, K=K, V=2048, r=64)
    rng = np.random.default_rng(5)
    h = torch.from_numpy(S.f32_to_bf16(rng.standard_normal((B, K, 256)).astype(np.float32)).view(np.int16)).cuda()
    cw = t_f32((rng.standard_normal(256 + 64) * 0.1).astype(np.float32))
    _, _, conf, surv = D.dspark_markov_draft_confidence(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor),
                                                        h.view(torch.bfloat16), cw, w2_layout=D.DSPARK_W2_VR)
    sps = (100.0 - 0.5 * np.arange(B * (K + 1) + 1)).astype(np.float32)
    lengths, theta = D.dspark_schedule_prefixes(surv, t_f32(sps))
    ln, a, th = host(lengths), host(surv).astype(np.float64), float(host(theta)[0])
    assert np.all((ln >= 0) & (ln <= K))
    n = int(ln.sum())
    tokens = B + sum(a[r, :ln[r]].sum() for r in range(B))
    assert th == pytest.approx(tokens * sps[B + n], rel=1e-5)
    nxt = [a[r, ln[r]] for r in range(B) if ln[r] < K]
    if nxt and n < B * K:
        assert (tokens + max(nxt)) * sps[B + n + 1] <= tokens * sps[B + n] * (1 + 1e-6)
