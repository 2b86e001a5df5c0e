"""GPU parity of the Selector path (dspark_topk, dspark_selector_draft) and of the gate (dspark_gate)."""
import numpy as np
import pytest

import oracle as O
import synth as S
from helpers import LOGIT_TOL, MARGIN_TOL, check_draft, host, t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


def _tie_rows(rows, V, seed=0):
    rng = np.random.default_rng(seed)
    U = np.round(rng.standard_normal((rows, V)) * 3).astype(np.float32)
    U[0] = 0.0
    U[1, ::2] = -0.0
    U[2] = 7.0
    if rows > 3:
        U[3, ::5] = 100.0
    return U


TOPK_CASES = [(V, k) for V in (16, 100, 1001, 4096, 151936) for k in (1, 5, 16, 17, 40, 64) if k <= V]


@pytest.mark.parametrize("V,k", TOPK_CASES, ids=lambda c: str(c))
def test_topk_exact(D, V, k):
    rows = 6 if V > 10000 else 40
    U = _tie_rows(rows, V, seed=V + k) if V <= 10000 else S.logits(0xD5A10004, (rows,), V, 16)
    idx, val = D.dspark_topk(t_f32(U), k)
    ridx, rval = O.topk(U, k)
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(val), rval)


@pytest.mark.parametrize("V,k", [(64, 64), (512, 512), (300, 40), (4096, 100)])
def test_topk_large_k_small_vocab(D, V, k):
    U = _tie_rows(12, V, seed=k)
    idx, val = D.dspark_topk(t_f32(U), k)
    ridx, rval = O.topk(U, k)
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(val), rval)


SEL_SHAPES = [(3, 4, 200, 32, 16, S.BF16), (5, 3, 1000, 64, 5, S.BF16), (2, 5, 96, 16, 16, S.F32),
              (130, 2, 513, 48, 16, S.BF16), (2, 3, 300, 520, 16, S.BF16), (3, 3, 2000, 32, 32, S.BF16),
              (2, 3, 5000, 64, 64, S.BF16),
              # K = 16 with k = 32 (the row-parallel walk with more than 64 KB of LDS) and k = 64 (tables
              # beyond the workgroup's LDS, walked step by step from global memory)
              (2, 16, 1000, 32, 32, S.BF16), (2, 16, 1000, 32, 64, S.BF16)]


@pytest.mark.parametrize("shape", SEL_SHAPES, ids=lambda s: "B%d-K%d-V%d-r%d-k%d" % s[:5])
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
def test_selector_parity(D, shape, mode, gated):
    B, K, V, r, topk, wd = shape
    w = S.strong("selector", B=B, K=K, V=V, r=r, wdtype=wd, mode=mode)
    A, Bemb = w.W1, w.W2T
    H = np.random.default_rng(2).uniform(0, 1, (B, K, r)).astype(np.float32) if gated else None
    T = 0.7 if mode == S.SAMPLE else 1.0
    res = D.dspark_selector_draft(t_f32(w.U), t_w(A), t_w(Bemb), t_i32(w.anchor), H=None if H is None else t_f32(H),
                                  topk=topk, mode=mode, seed=77, temperature=T, want_cand=True, want_scores=True)
    tok, lp, cand, scores = (host(res[k]) for k in ("tokens", "logprobs", "cand", "scores"))
    ref = O.selector_draft(w.U, A, Bemb, w.anchor, H=None if H is None else H.astype(np.float64), topk=topk,
                           mode=mode, seed=77, temperature=T)
    assert np.array_equal(cand, ref["cand"])
    tol = LOGIT_TOL if gated else 1e-3
    assert np.abs(scores - ref["tables"]).max() <= tol
    # walk: along the GPU's own path the oracle's pick agrees wherever its margin is not tiny
    ref_r = O.markov_restricted(w.U, A, Bemb, w.anchor, cand, w2_layout=O.W2_VR,
                                H=None if H is None else H.astype(np.float64), mode=mode, seed=77, temperature=T)
    flagged = ref_r["margins"] < MARGIN_TOL
    agree = tok == ref_r["tokens"]
    first_bad = np.where(~agree & ~flagged)
    # compare each row up to its first flagged divergence (a divergence changes all later predecessors)
    for b in range(B):
        for t in range(K):
            if tok[b, t] != ref_r["tokens"][b, t]:
                assert flagged[b, t], (b, t, first_bad)
                break
            assert abs(lp[b, t] - ref_r["logprobs"][b, t]) <= tol


def test_selector_topk_V_equals_full_head(D):
    """top-k = V: the truncated execution is the full-vocabulary Markov head.  Greedy: the same picks as the
    full head, the oracle's and the library's.  Sampling: the candidate set is the whole vocabulary, drawn
    by Gumbel-max per candidate (the full head draws by the block race: the same distribution, other
    noise), so the reference is the head restricted to the whole vocabulary."""
    w = S.strong("tiny")
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), topk=w.V, mode=S.GREEDY, seed=3)
    tok, lp = host(res["tokens"]), host(res["logprobs"])
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=S.GREEDY, seed=3, follow=tok)
    check_draft(tok, lp, ref)
    gtok, glp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2), t_i32(w.anchor), w2_layout=D.DSPARK_W2_RV,
                                      mode=S.GREEDY, seed=3)
    gtok = host(gtok)
    agree_until = np.cumprod(gtok == tok, axis=1).astype(bool)
    assert agree_until[:, 0].all() or (ref["margins"][:, 0] < MARGIN_TOL).all()
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), topk=w.V, mode=S.SAMPLE, seed=3)
    tok, lp = host(res["tokens"]), host(res["logprobs"])
    cand = np.broadcast_to(np.arange(w.V, dtype=np.int32), (w.B, w.K, w.V))
    ref = O.markov_restricted(w.U, w.W1, w.W2, w.anchor, cand, mode=S.SAMPLE, seed=3)
    # the restricted oracle runs its own path: compare up to the first flagged position of each row
    for b in range(w.B):
        for t in range(w.K):
            if ref["margins"][b, t] < MARGIN_TOL:
                break
            assert tok[b, t] == ref["tokens"][b, t]
            assert abs(lp[b, t] - ref["logprobs"][b, t]) <= 1e-2


def test_full_selector_sampled_rows(D):
    w = S.workload("selector")
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), topk=16, want_cand=True)
    tok, cand = host(res["tokens"]), host(res["cand"])
    rows = [0, 50, 127]
    for b in rows:
        ridx, _ = O.topk(w.U[b], 16)
        assert np.array_equal(cand[b], ridx)
    ref = O.selector_draft(w.U, w.W1, w.W2T, w.anchor, topk=16, rows=rows)
    flagged = ref["margins"][rows] < MARGIN_TOL
    for i, b in enumerate(rows):
        for t in range(w.K):
            if tok[b, t] != ref["tokens"][b, t]:
                assert flagged[i, t]
                break


# -------------------------------------------------------------------------------------------- gate

@pytest.mark.parametrize("rows,Dm,r", [(5, 256, 32), (64, 512, 64), (100, 1024, 256)])
def test_gate_parity(D, rows, Dm, r):
    rng = np.random.default_rng(rows)
    h = S.f32_to_bf16(rng.standard_normal((rows, Dm)).astype(np.float32))
    Wg = S.f32_to_bf16((rng.standard_normal((Dm, r)) * 0.05).astype(np.float32))
    H = host(D.dspark_gate(t_w(h), t_w(Wg)))
    ref = O.gate(h, Wg)
    assert np.abs(H - ref).max() <= 1e-3
    H0 = host(D.dspark_gate(t_w(h), t_w(np.zeros_like(Wg))))
    assert np.all(H0 == 0.5)


def test_full_gated_workload(D):
    """B=64, K=16, V=129280, r=256, D=4096: gate for the whole block, then the gated full-vocabulary head
    and its top-16 Selector form, sampled rows against the oracle (which computes its own gate)."""
    w = S.workload("gated")
    H = D.dspark_gate(t_w(w.h), t_w(w.Wg))
    Hh = host(H)
    rows = [0, 31, 63]
    Href = O.gate(w.h[rows], w.Wg)
    assert np.abs(Hh[rows] - Href).max() <= 1e-3
    Hd = np.zeros((w.B, w.K, w.r))
    Hd[rows] = Href
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), H=H)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2T, w.anchor, w2_layout=O.W2_VR, H=Hd, follow=tok, rows=rows)
    check_draft(tok[rows], lp[rows], {k: v[rows] for k, v in ref.items()})
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), H=H, topk=16, want_cand=True)
    stok, cand = host(res["tokens"]), host(res["cand"])
    sref = O.markov_restricted(w.U, w.W1, w.W2T, w.anchor, cand, w2_layout=O.W2_VR, H=Hd, rows=rows)
    for b in rows:
        for t in range(w.K):
            if stok[b, t] != sref["tokens"][b, t]:
                assert sref["margins"][b, t] < MARGIN_TOL
                break
