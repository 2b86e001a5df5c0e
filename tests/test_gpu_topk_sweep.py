"""Top-k sweep: the Selector execution of an already trained Markov head, i.e. the calibration restricted to
the top-k candidates of the base logits (equivalence page, "Two implications", second point), against the
full-vocabulary head, greedy, for k in {4, 8, 16, 32, 64}, on three input recipes:
  * serving: the measured recipe (U = 4z + 8 on 16 hot ids, weights N(0, 0.02)); the bias is far below the
    hot-token boost, so the truncation never changes the draft (agreement 1 is the expected answer there);
  * moderate: U = z + 2 on hot ids, bias of standard deviation 0.3;
  * strong: U = z + 2 on hot ids, bias of standard deviation 1 (the truncation changes most drafts).
At every k the GPU's truncated draft is checked against the oracle's head restricted to the same candidates along
the GPU's own path, and the GPU's full head against the oracle's; the agreement of truncated and full drafts is
computed from the GPU outputs and, independently, from the oracle's own drafts, and the two must match.  Along a
row the truncated walk also equals the full greedy head until the first position whose full pick is not among that
position's candidates (an argmax over a subset that contains the global argmax is the global argmax)."""
import numpy as np
import pytest

import oracle as O
import synth as S
from helpers import check_draft, host, t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu

KS = [4, 8, 16, 32, 64]
B, K, V, R = 16, 8, 20000, 64


def _recipe(name):
    if name == "serving":
        return S.workload("selector", B=B, K=K, V=V, r=R)
    bias_sd = 0.3 if name == "moderate" else 1.0
    return S.workload("selector", B=B, K=K, V=V, r=R, sigma_w=float(np.sqrt(bias_sd / np.sqrt(R))), u_scale=1.0,
                      u_boost=2.0)


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


@pytest.mark.parametrize("recipe", ["serving", "moderate", "strong"])
def test_topk_sweep_against_oracle(D, recipe):
    w = _recipe(recipe)
    U, A, Bemb, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    full, flp = D.dspark_markov_draft(U, A, Bemb, anc, w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_GREEDY)
    f, flp = host(full), host(flp)
    check_draft(f, flp, O.markov_draft(w.U, w.W1, w.W2T, w.anchor, w2_layout=O.W2_VR, follow=f), what=f"{recipe} full")
    oracle_full = O.markov_draft(w.U, w.W1, w.W2T, w.anchor, w2_layout=O.W2_VR)["tokens"]
    report = []
    for k in KS:
        res = D.dspark_selector_draft(U, A, Bemb, anc, topk=k, want_cand=True)
        tok, lp, cand = host(res["tokens"]), host(res["logprobs"]), host(res["cand"])
        ridx, _ = O.topk(w.U, k)
        assert np.array_equal(cand, ridx)
        ref = O.markov_restricted(w.U, w.W1, w.W2T, w.anchor, cand, w2_layout=O.W2_VR, follow=tok)
        check_draft(tok, lp, ref, what=f"{recipe} k={k}")
        gpu_agree = float((tok == f).mean())
        osel = O.selector_draft(w.U, w.W1, w.W2T, w.anchor, topk=k)["tokens"]
        oracle_agree = float((osel == oracle_full).mean())
        # the two agreements come from independent computations; only near-ties may separate them
        assert abs(gpu_agree - oracle_agree) <= 2.0 / tok.size + 0.02, (k, gpu_agree, oracle_agree)
        report.append((k, gpu_agree, oracle_agree))
        # exactness until the full pick leaves the candidates
        for b in range(B):
            diff = np.nonzero(tok[b] != f[b])[0]
            if diff.size:
                t = int(diff[0])
                if f[b, t] in cand[b, t]:
                    assert ref["margins"][b, t] < 2e-2 or ref["reach"][b, t] == 1, (k, b, t)
    if recipe == "serving":
        assert all(g == 1.0 for _, g, _ in report)
    if recipe == "strong":
        assert min(g for _, g, _ in report) < 0.5  # the truncation does bind on these inputs
    print(f"[sweep] {recipe}: (k, GPU agreement, oracle agreement) = {report}")
