"""Top-k sweep: the Selector execution of an already trained Markov head, i.e. the calibration restricted to
the top-k candidates of the base logits (equivalence page, "Two implications", second point), against the
full-vocabulary head, greedy, for k in {4, 8, 16, 32, 64} on synthetic and strong-bias inputs.

Property checked on the GPU outputs: along a row the truncated walk equals the full-vocabulary greedy until
the first position whose full pick is not among that position's candidates (an argmax over a subset that
contains the global argmax is the global argmax).  The two paths sum the rank-r products in different orders,
so a divergence with the full pick among the candidates is accepted only as a near-tie of the walked scores."""
import numpy as np
import pytest

import synth as S
from helpers import host, t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu

KS = [4, 8, 16, 32, 64]
NEAR_TIE = 1e-3


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


@pytest.mark.parametrize("strong", [False, True], ids=["synthetic", "strong-bias"])
def test_truncation_exact_until_full_pick_leaves_candidates(D, strong):
    B, K, V, r = 16, 8, 20000, 64
    w = (S.strong if strong else S.workload)("selector", B=B, K=K, V=V, r=r)
    U, A, Bemb, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    full, _ = D.dspark_markov_draft(U, A, Bemb, anc, w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_GREEDY)
    f = host(full)
    agree = []  # reported, not asserted: how often the truncation changes the draft depends on the inputs
    for k in KS:
        res = D.dspark_selector_draft(U, A, Bemb, anc, topk=k, want_cand=True, want_scores=True)
        tok, cand, sc = host(res["tokens"]), host(res["cand"]), host(res["scores"])
        agree.append(float((tok == f).mean()))
        for b in range(B):
            diff = np.nonzero(tok[b] != f[b])[0]
            if diff.size == 0:
                continue
            t = int(diff[0])
            if f[b, t] not in cand[b, t]:
                continue
            # the full pick was a candidate: only a near-tie of the walked row may separate the two picks
            if t == 0:
                row = sc[b, :k]
            else:
                i_prev = int(np.nonzero(cand[b, t - 1] == tok[b, t - 1])[0][0])
                row = sc[b, k + ((t - 1) * k + i_prev) * k: k + ((t - 1) * k + i_prev + 1) * k]
            j_sel = int(np.nonzero(cand[b, t] == tok[b, t])[0][0])
            j_full = int(np.nonzero(cand[b, t] == f[b, t])[0][0])
            assert abs(row[j_sel] - row[j_full]) <= NEAR_TIE, (k, b, t, row[j_sel], row[j_full])
    print("agreement with the full head for k =", KS, ":", agree)
