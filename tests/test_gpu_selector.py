"""GPU parity of the Selector path (dspark_topk, dspark_selector_draft) and of the gate (dspark_gate)."""
import numpy as np
import pytest
import torch

import oracle as O
import synth as S
from helpers import LOGIT_TOL, check_draft, host, t_f32, t_i32, t_w

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


@pytest.mark.parametrize("V,k", [(64, 64), (512, 512), (300, 40), (4096, 100), (65, 65), (100, 77), (2000, 1999),
                                 (4096, 4096)])
def test_topk_large_k_small_vocab(D, V, k):
    """k > 64 at V <= 4096 takes the whole-row bitonic sort in LDS (padded to a power of two: 65 -> 128,
    100 -> 128, 2000 -> 2048; 4096 fills it)."""
    U = _tie_rows(12, V, seed=k)
    idx, val = D.dspark_topk(t_f32(U), k)
    ridx, rval = O.topk(U, k)
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(val), rval)


@pytest.mark.parametrize("V,k", [(4097, 65), (5000, 100), (10007, 1024), (151936, 65), (151936, 256),
                                 (151936, 1024), (129280, 700)], ids=lambda c: str(c))
def test_topk_radix_select(D, V, k):
    """64 < k <= 1024 at V > 4096: radix selection.  Rows with heavy ties, an all-equal row (the k lowest ids),
    +-0 and a row of repeated maxima exercise the count of the k-th key's equals; large V uses logits rows."""
    rows = 6 if V > 10000 else 8
    U = _tie_rows(rows, V, seed=V + k) if V <= 10000 else S.logits(0xD5A10005, (rows,), V, 16)
    if V > 10000:
        U[1, ::3] = U[1].max()  # many equal maxima: the top-k is the lowest ids among them
        U[2] = -0.0
    idx, val = D.dspark_topk(t_f32(U), k)
    ridx, rval = O.topk(U, k)
    assert np.array_equal(host(idx), ridx)
    assert np.array_equal(host(val), rval)


SEL_SHAPES = [(3, 4, 200, 32, 16, S.BF16), (5, 3, 1000, 64, 5, S.BF16), (2, 5, 96, 16, 16, S.F32),
              (130, 2, 513, 48, 16, S.BF16), (2, 3, 300, 520, 16, S.BF16), (3, 3, 2000, 32, 32, S.BF16),
              (2, 3, 5000, 64, 64, S.BF16),
              # r = 256 (the measured rank: the matrix-core pair scores loop over several rank batches)
              (4, 4, 3000, 256, 16, S.BF16),
              # K = 16 with k = 32 (the row-parallel walk with more than 64 KB of LDS) and k = 64 (tables
              # beyond the workgroup's LDS, walked step by step from global memory)
              (2, 16, 1000, 32, 32, S.BF16), (2, 16, 1000, 32, 64, S.BF16),
              # k > 64 at V > 4096 (radix-selected candidates)
              (2, 3, 5000, 32, 100, S.BF16), (2, 3, 5000, 16, 1024, S.BF16)]


def _restricted_check(D, w, A, Bemb, H, cand, tok, lp, mode, seed, T, what, rows=None):
    """The walk's tokens against the head restricted to the same candidates, along the GPU's own path."""
    ref = O.markov_restricted(w.U, A, Bemb, w.anchor, cand, w2_layout=O.W2_VR,
                              H=None if H is None else H.astype(np.float64), mode=mode, seed=seed, temperature=T,
                              follow=tok, rows=rows)
    if rows is not None:
        ref = {k: v[rows] for k, v in ref.items()}
        tok, lp = tok[rows], None if lp is None else lp[rows]
    return check_draft(tok, lp, ref, what=what)


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
    _restricted_check(D, w, A, Bemb, H, cand, tok, lp, mode, 77, T, f"selector {shape} {mode} gated={gated}")


@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_selector_topk_V_equals_full_head(D, mode):
    """top-k = V on the tiny workload (V = 512): the truncated execution is the full-vocabulary head, in both
    modes.  The Selector's tokens are checked against the oracle's full head (not a restricted one) along the
    Selector's own path, and so are the full head's tokens; in sampling mode both draw with the same noise
    (keyed on vocabulary blocks), so the two GPU paths draft the same tokens wherever no near-tie separates them."""
    w = S.strong("tiny")
    T = 0.9 if mode == S.SAMPLE else 1.0
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), topk=w.V, mode=mode, seed=3,
                                  temperature=T)
    tok, lp = host(res["tokens"]), host(res["logprobs"])
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=3, temperature=T, follow=tok)
    check_draft(tok, lp, ref, what=f"selector top-k=V {mode}")
    gtok, glp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2), t_i32(w.anchor), w2_layout=D.DSPARK_W2_RV,
                                      mode=mode, seed=3, temperature=T)
    gtok, glp = host(gtok), host(glp)
    gref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=3, temperature=T, follow=gtok)
    check_draft(gtok, glp, gref, what=f"full head {mode}")
    # the two GPU paths share their predecessors up to their first difference, which needs a near-tie there
    for b in range(w.B):
        diff = np.nonzero(tok[b] != gtok[b])[0]
        if diff.size:
            t = int(diff[0])
            assert min(ref["margins"][b, t], gref["margins"][b, t]) < 2e-2, (b, t)


@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_full_selector_all_rows(D, mode):
    """B=128, K=16, V=151936, r=256, top-16 (the measured Selector workload): every row's candidates exactly,
    the pair tables of sampled rows, and every row's walk against the restricted head along the GPU's path."""
    w = S.workload("selector")
    T = 1.0
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), topk=16, mode=mode,
                                  seed=w.noise_seed, temperature=T, want_cand=True, want_scores=True)
    tok, lp, cand, scores = (host(res[k]) for k in ("tokens", "logprobs", "cand", "scores"))
    ridx, _ = O.topk(w.U, 16)
    assert np.array_equal(cand, ridx)
    rows = [0, 50, 127]
    ref = O.selector_draft(w.U, w.W1, w.W2T, w.anchor, topk=16, mode=mode, seed=w.noise_seed, rows=rows)
    assert np.abs(scores[rows] - ref["tables"][rows]).max() <= 1e-3
    _restricted_check(D, w, w.W1, w.W2T, None, cand, tok, lp, mode, w.noise_seed, T, f"full selector {mode}")


@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
@pytest.mark.parametrize("cfg", ["small", "full"])
def test_gated_selector_with_unit_gate_is_the_markov_head_on_the_candidates(D, mode, cfg):
    """H = 1: the gated Selector is the (ungated) Markov head restricted to the same candidates (equivalence page,
    "The equivalence: remove the gate, recover the Markov Head").  The gated tables equal the ungated ones bit for
    bit (a bf16 row times 1 is itself), so do the drafts, and both follow the oracle's restricted head."""
    if cfg == "full":
        w = S.workload("selector", mode=mode)
    else:
        w = S.strong("selector", B=6, K=5, V=3000, r=64, mode=mode)
    T = 0.8 if mode == S.SAMPLE else 1.0
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    kw = dict(topk=16, mode=mode, seed=5, temperature=T, want_cand=True, want_scores=True)
    a = D.dspark_selector_draft(*args, **kw)
    ones = torch.ones((w.B, w.K, w.r), dtype=torch.float32, device="cuda")
    b = D.dspark_selector_draft(*args, H=ones, **kw)
    for key in ("cand", "scores", "tokens", "logprobs"):
        assert np.array_equal(host(a[key]), host(b[key])), key
    tok, lp, cand = host(b["tokens"]), host(b["logprobs"]), host(b["cand"])
    rows = None if cfg == "small" else [0, 64, 127]
    _restricted_check(D, w, w.W1, w.W2T, None, cand, tok, lp, mode, 5, T, f"unit gate {cfg}", rows=rows)


# -------------------------------------------------------------------------------------------- gate

@pytest.mark.parametrize("split_k", [True, False], ids=["split-k", "single"])
@pytest.mark.parametrize("rows,Dm,r", [(5, 256, 32), (64, 512, 64), (100, 1024, 256), (130, 4096, 128)])
def test_gate_parity(D, rows, Dm, r, split_k):
    """Both forms against the oracle (the split-k form takes r % 64 == 0 and D % 512 == 0; rows 100 and 130
    leave a ragged 64-row tile)."""
    rng = np.random.default_rng(rows)
    h = S.f32_to_bf16(rng.standard_normal((rows, Dm)).astype(np.float32))
    Wg = S.f32_to_bf16((rng.standard_normal((Dm, r)) * 0.05).astype(np.float32))
    H = host(D.dspark_gate(t_w(h), t_w(Wg), split_k=split_k))
    ref = O.gate(h, Wg)
    assert np.abs(H - ref).max() <= 1e-3
    H0 = host(D.dspark_gate(t_w(h), t_w(np.zeros_like(Wg)), split_k=split_k))
    assert np.all(H0 == 0.5)


def test_gate_forms_agree_at_full_size(D):
    """rows = 1024 (B = 64, K = 16), D = 4096, r = 256: the split-k and single-launch forms differ only in
    the order of the fp32 sums; twice through one workspace gives the same bits."""
    w = S.workload("gated")
    h, Wg = t_w(w.h), t_w(w.Wg)
    rows = h.numel() // Wg.shape[0]
    ws = torch.full((D.dspark_gate_workspace_bytes(rows, Wg.shape[0], Wg.shape[1]),), 0xA5, dtype=torch.uint8,
                    device=h.device)  # arbitrary contents: the partial sums are written before they are read
    assert ws.numel() == 4 * rows * Wg.shape[1] * 4
    a = host(D.dspark_gate(h, Wg, workspace=ws))
    b = host(D.dspark_gate(h, Wg, workspace=ws))
    c = host(D.dspark_gate(h, Wg, split_k=False))
    assert np.array_equal(a, b)
    assert np.abs(a - c).max() <= 1e-6


def test_gate_misaligned_output_takes_the_unsplit_form(D):
    """A workspace with an H that is not 16-byte aligned: the call falls back to the unsplit form (bit for bit
    the split_k=False result) instead of the split-k sum's 16-byte stores."""
    rng = np.random.default_rng(11)
    rows, Dm, r = 128, 1024, 128
    hn = S.f32_to_bf16(rng.standard_normal((rows, Dm)).astype(np.float32))
    Wn = S.f32_to_bf16((rng.standard_normal((Dm, r)) * 0.05).astype(np.float32))
    h, Wg = t_w(hn), t_w(Wn)
    flat = torch.empty(rows * r + 1, dtype=torch.float32, device=h.device)
    out = flat[1:].view(rows, r)
    assert out.data_ptr() % 16 != 0
    ws = torch.empty(D.dspark_gate_workspace_bytes(rows, Dm, r), dtype=torch.uint8, device=h.device)
    D.dspark_gate(h, Wg, out=out, workspace=ws)
    ref = host(D.dspark_gate(h, Wg, split_k=False))
    assert np.array_equal(host(out), ref)
    assert np.abs(ref - O.gate(hn, Wn)).max() <= 1e-3


def test_gate_graph_replays(D):
    """The split-k gate (its two launches) captured in a HIP graph: every replay, with eager calls between,
    equals the eager call."""
    rng = np.random.default_rng(7)
    rows, Dm, r = 192, 1024, 128
    h = t_w(S.f32_to_bf16(rng.standard_normal((rows, Dm)).astype(np.float32)))
    Wg = t_w(S.f32_to_bf16((rng.standard_normal((Dm, r)) * 0.05).astype(np.float32)))
    ws = torch.empty(D.dspark_gate_workspace_bytes(rows, Dm, r), dtype=torch.uint8, device=h.device)
    out = torch.empty((rows, r), dtype=torch.float32, device=h.device)
    eager = host(D.dspark_gate(h, Wg, workspace=ws))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        D.dspark_gate(h, Wg, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        D.dspark_gate(h, Wg, out=out, workspace=ws)
    for i in range(4):
        out.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), eager), i
        assert np.array_equal(host(D.dspark_gate(h, Wg, workspace=ws)), eager), i


def test_full_gated_workload(D):
    """B=64, K=16, V=129280, r=256, D=4096: the gate for the whole block, then the gated full-vocabulary head
    and its top-16 Selector form, every row against the oracle (which computes its own gate)."""
    w = S.workload("gated")
    H = D.dspark_gate(t_w(w.h), t_w(w.Wg))
    Hh = host(H)
    Href = O.gate(w.h, w.Wg)
    assert np.abs(Hh - Href).max() <= 1e-3
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), H=H)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2T, w.anchor, w2_layout=O.W2_VR, H=Href, follow=tok)
    check_draft(tok, lp, ref, what="gated head")
    res = D.dspark_selector_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), H=H, topk=16, want_cand=True,
                                  want_scores=True)
    stok, slp, cand, scores = (host(res[k]) for k in ("tokens", "logprobs", "cand", "scores"))
    rows = [0, 31, 63]
    sref = O.selector_draft(w.U, w.W1, w.W2T, w.anchor, H=Href, topk=16, rows=rows)
    assert np.array_equal(cand[rows], sref["cand"][rows])
    assert np.abs(scores[rows] - sref["tables"][rows]).max() <= LOGIT_TOL
    _restricted_check(D, w, w.W1, w.W2T, Href, cand, stok, slp, S.GREEDY, 0, 1.0, "gated selector")
