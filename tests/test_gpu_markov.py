"""GPU parity of the Markov-head path (dspark_markov_logits / _step / _draft) against the fp64 oracle.

Small shapes span several 32-wide vocabulary tiles, ragged vocabulary tails, ragged 128-row batch blocks,
both W2 storage orders, fp32 and bf16 weights, every rank path, greedy and Gumbel-max picks, weak (the
measured recipe) and strong (bias of unit size) weights, and the gate.  Full-size cases run the measured
workloads in the launch configuration the bench times and compare sampled rows.
"""
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


def _w2(w, layout):
    return w.W2 if layout == O.W2_RV else np.ascontiguousarray(w.W2.T)


def _rand_H(B, K, r, seed=0):
    return np.random.default_rng(seed).uniform(0.0, 1.0, (B, K, r)).astype(np.float32)


# (B, K, V, r, wdtype): tile-spanning small shapes.  bf16 with r a power-of-two multiple of 16 and V % 4 == 0
# drafts with the persistent whole-round kernel; V % 4 != 0 with the per-position kernels; r=24 and r=48 and
# fp32 weights take the vector-ALU path
SHAPES = [
    (8, 3, 3000, 256, S.BF16),   # the largest small block (at most 8 rows), ragged vocabulary tail
    (2, 2, 2050, 128, S.BF16),
    (9, 2, 1000, 256, S.BF16),   # the smallest half block (9 .. 64 rows: two sets of consumer waves)
    (64, 2, 3000, 256, S.BF16),  # the largest half block, ragged vocabulary tail
    (65, 2, 1500, 256, S.BF16),  # the smallest batch on the full 128-row block
    (40, 2, 2000, 64, S.BF16),
    (1, 4, 512, 16, S.F32),
    (3, 3, 1000, 16, S.BF16),
    (130, 2, 776, 32, S.BF16),
    (128, 3, 4096, 256, S.BF16),
    (5, 3, 1000, 64, S.BF16),
    (130, 2, 777, 32, S.BF16),
    (3, 3, 100, 24, S.BF16),
    (4, 2, 600, 48, S.BF16),
    (2, 2, 300, 512, S.BF16),  # r = 512: per-position kernels
    (7, 2, 257, 16, S.F32),
    (1, 3, 3000, 256, S.BF16),  # one row at r = 256: greedy drafts keep W2 resident (most lanes hold no id)
    (1, 2, 200, 256, S.BF16),   # fewer ids than workgroups: some workgroups hold none
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d-K%d-V%d-r%d-%s" % (s[0], s[1], s[2], s[3], "bf16" if s[4] else "f32"))
@pytest.mark.parametrize("layout", [O.W2_RV, O.W2_VR], ids=["rv", "vr"])
@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
def test_logits_parity(D, shape, layout, gated):
    B, K, V, r, wd = shape
    w = S.strong("serving", B=B, K=1, V=V, r=r, wdtype=wd)
    prev = np.random.default_rng(1).integers(0, V, B).astype(np.int32)
    H = _rand_H(B, 1, r)[:, 0] if gated else None
    out = D.dspark_markov_logits(t_f32(w.U[:, 0]), t_w(w.W1), t_w(_w2(w, layout)), t_i32(prev), w2_layout=layout,
                                 H_k=None if H is None else t_f32(H))
    got = host(out)
    ref = O.markov_logits(w.U[:, 0], w.W1, _w2(w, layout), prev, w2_layout=layout,
                          Hk=None if H is None else H.astype(np.float64))
    err = np.abs(got - ref).max()
    # fp32 accumulation of exact products; the gated bf16 path also rounds W1[a] (.) H to bf16
    assert err <= (LOGIT_TOL if gated and wd == S.BF16 else 1e-3), err
    assert np.abs(ref - w.U[:, 0]).max() > 0.5  # the bias is far from negligible in this variant


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%d-K%d-V%d-r%d" % s[:4])
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
@pytest.mark.parametrize("strength", ["weak", "strong"])
def test_draft_parity(D, shape, mode, strength):
    B, K, V, r, wd = shape
    make = S.strong if strength == "strong" else S.workload
    w = make("serving", B=B, K=K, V=V, r=r, wdtype=wd, mode=mode)
    T = 0.8 if mode == S.SAMPLE else 1.0
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), w2_layout=D.DSPARK_W2_VR,
                                    mode=mode, seed=w.noise_seed, temperature=T)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=w.noise_seed, temperature=T, follow=tok)
    check_draft(tok, lp, ref, what=f"{shape} {mode} {strength}")


@pytest.mark.parametrize("B,V,r,wd", [(9, 900, 64, S.BF16), (4, 20000, 64, S.BF16), (6, 700, 24, S.F32),
                                      (5, 1001, 48, S.BF16), (1, 3000, 256, S.BF16)],
                         ids=["B9-half-block", "B4-small-block", "B6-f32-small-round", "B5-r48-small-round",
                              "B1-resident"])
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_draft_gated_and_rv_layout(D, mode, B, V, r, wd):
    """The gated head with W2 stored [r, V]: the matrix-core round kernel (a transposed copy of W2 first) and the
    one-launch vector-ALU round (fp32 weights, a rank that is not a power-of-two multiple of 16)."""
    w = S.strong("gated", B=B, K=4, V=V, r=r, D=0, mode=mode, wdtype=wd)
    H = _rand_H(w.B, w.K, w.r, seed=3)
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2), t_i32(w.anchor), w2_layout=D.DSPARK_W2_RV,
                                    H=t_f32(H), mode=mode, seed=11)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, H=H.astype(np.float64), mode=mode, seed=11, follow=tok)
    check_draft(tok, lp, ref)


def test_gate_ones_equals_ungated_bitwise(D):
    """H = 1 makes X = W1[a] exactly.  At this size every workgroup holds one vocabulary tile, so the gated and
    ungated small-block forms (one consumer set against four) also merge their log-sum-exp terms in the same
    order and the log-probabilities agree bit for bit; with several tiles per workgroup the tokens still do."""
    w = S.strong("serving", B=6, K=3, V=700, r=64, mode=S.SAMPLE)
    a = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), mode=D.DSPARK_SAMPLE, seed=5)
    b = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), mode=D.DSPARK_SAMPLE, seed=5,
                              H=t_f32(np.ones((w.B, w.K, w.r), np.float32)))
    assert np.array_equal(host(a[0]), host(b[0]))
    assert np.array_equal(host(a[1]), host(b[1]))


def test_w2_zero_is_argmax_of_U(D):
    """The head disabled (W2 = 0): greedy tokens are exactly the per-position argmax of U (ties low)."""
    w = S.workload("serving", B=3, K=4, V=2000, r=32, mode=S.GREEDY)
    U = np.round(w.U).astype(np.float32)  # plenty of exact ties
    W2T = np.zeros_like(w.W2T)
    tok, lp = D.dspark_markov_draft(t_f32(U), t_w(w.W1), t_w(W2T), t_i32(w.anchor))
    assert np.array_equal(host(tok), np.argmax(U, axis=-1))


def test_step_teacher_forced_and_determinism(D):
    w = S.strong("serving", B=33, K=3, V=1500, r=128, mode=S.SAMPLE)
    U = t_f32(w.U)
    W1, W2 = t_w(w.W1), t_w(w.W2T)
    rng = np.random.default_rng(4)
    for k in range(w.K):
        prev = rng.integers(0, w.V, w.B).astype(np.int32)
        tok, lp, bl = D.dspark_markov_step(U[:, k], W1, W2, t_i32(prev), k, mode=D.DSPARK_SAMPLE, seed=9)
        tok2, lp2, _ = D.dspark_markov_step(U[:, k], W1, W2, t_i32(prev), k, mode=D.DSPARK_SAMPLE, seed=9)
        tok, lp, bl = host(tok), host(lp), host(bl)
        assert np.array_equal(tok, host(tok2)) and np.array_equal(lp, host(lp2))
        # oracle at position k with the same predecessors (the noise counter is the position k)
        Ufull = np.zeros((w.B, k + 1, w.V), np.float32)
        Ufull[:, k] = w.U[:, k]
        follow = np.zeros((w.B, k + 1), np.int32)
        follow[:, k] = tok
        if k > 0:
            follow[:, k - 1] = prev
        anchor = prev if k == 0 else np.zeros(w.B, np.int32)
        ref = O.markov_draft(Ufull, w.W1, w.W2, anchor, mode=O.SAMPLE, seed=9, follow=follow)
        sub = {key: v[:, k:k + 1] for key, v in ref.items()}
        check_draft(tok[:, None], lp[:, None], sub)
        agree = tok == sub["tokens"][:, 0]
        assert np.abs(bl[agree] - ref["best_logit"][agree, k]).max() <= LOGIT_TOL


def test_repeat_runs_bit_identical(D):
    w = S.workload("serving", B=64, K=4, V=4096, r=256, mode=S.SAMPLE)
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    a = D.dspark_markov_draft(*args, mode=D.DSPARK_SAMPLE, seed=1)
    b = D.dspark_markov_draft(*args, mode=D.DSPARK_SAMPLE, seed=1)
    assert np.array_equal(host(a[0]), host(b[0])) and np.array_equal(host(a[1]), host(b[1]))


def test_k1_and_single_row(D):
    w = S.strong("serving", B=1, K=1, V=31, r=16)
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, follow=tok)
    check_draft(tok, lp, ref)


# ------------------------------------------------------------------------------------------ full size

@pytest.fixture(scope="module")
def serving():
    return S.workload("serving")


def _full_draft_check(D, w, rows, mode, seed, H=None, Hd=None, what=""):
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), w2_layout=D.DSPARK_W2_VR,
                                    H=H, mode=mode, seed=seed)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2T, w.anchor, w2_layout=O.W2_VR, H=Hd, mode=mode, seed=seed, follow=tok,
                         rows=rows)
    if rows is None:
        return check_draft(tok, lp, ref, what=what)
    sub = {k: v[rows] for k, v in ref.items()}
    return check_draft(tok[rows], lp[rows], sub, what=what)


def test_full_serving_all_rows(D, serving):
    """B=128, K=16, V=151936, r=256, sampling at T=1 (the measured workload and launch): every position of
    every row against the oracle along the GPU's path."""
    _full_draft_check(D, serving, None, S.SAMPLE, serving.noise_seed, what="serving sample")


def test_full_serving_greedy_all_rows(D, serving):
    """The serving shape with greedy picks (the bench's greedy line): every position of every row."""
    _full_draft_check(D, serving, None, S.GREEDY, 0, what="serving greedy")


def test_full_serving_logits_sampled_rows(D, serving):
    """The per-position kernels' logits at the serving shape (teacher-forced predecessors)."""
    w = serving
    prev = w.anchor.copy()
    for k in (0, w.K // 2, w.K - 1):
        out = host(D.dspark_markov_logits(t_f32(w.U[:, k]), t_w(w.W1), t_w(w.W2T), t_i32(prev)))
        rows = [3, 64, 126]
        ref = O.markov_logits(w.U[:, k], w.W1, w.W2T, prev, w2_layout=O.W2_VR, rows=rows)
        assert np.abs(out[rows] - ref[rows]).max() <= 1e-3
        prev = (prev * 7 + 13) % w.V


def test_full_serving_round_kernel_logits(D, serving):
    """The whole-round kernel's own calibrated logits (its store variant: same contraction, same pick) at the
    serving shape, sampling: tokens and log-probabilities are bit-identical to dspark_markov_draft's, and the
    logits of positions 0, 7 and 15 of every row, at the GPU's own predecessors, match the oracle's."""
    w = serving
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    kw = dict(w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_SAMPLE, seed=w.noise_seed)
    tok, lp, logits = D.dspark_markov_draft_logits(*args, **kw)
    tok2, lp2 = D.dspark_markov_draft(*args, **kw)
    tok, lp = host(tok), host(lp)
    assert np.array_equal(tok, host(tok2)) and np.array_equal(lp, host(lp2))
    for k in (0, 7, w.K - 1):
        got = host(logits[:, k].contiguous())
        prev = w.anchor if k == 0 else tok[:, k - 1]
        ref = O.markov_logits(w.U[:, k], w.W1, w.W2T, prev, w2_layout=O.W2_VR)
        err = np.abs(got - ref).max()
        assert err <= 1e-3, (k, err)
    del logits


ROUND_SHAPES = [(8, 3, 3000, 256), (3, 2, 1000, 32), (130, 2, 776, 64), (128, 3, 4096, 256), (40, 2, 2000, 128),
                # half blocks: five positions through the gate-row buffer at r = 256; a single position
                (64, 5, 3000, 256), (9, 1, 1000, 256),
                # one row at r = 256 (greedy: the resident round), with empty workgroups in the second
                (1, 3, 3000, 256), (1, 2, 200, 256)]


@pytest.mark.parametrize("shape", ROUND_SHAPES, ids=lambda s: "B%d-K%d-V%d-r%d" % s)
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
def test_round_kernel_logits(D, shape, mode, gated):
    """Every calibrated logit the whole-round kernel computes, at every position, against the oracle's at the
    GPU's own predecessors: small and full row blocks, ragged vocabulary tails, several ranks, both picks, the
    gate.  Strong weights, so that a dropped or misplaced bias term shows."""
    B, K, V, r = shape
    w = S.strong("serving", B=B, K=K, V=V, r=r, mode=mode)
    H = _rand_H(B, K, r, seed=9) if gated else None
    tok, lp, logits = D.dspark_markov_draft_logits(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor),
                                                   H=None if H is None else t_f32(H), mode=mode, seed=13,
                                                   temperature=0.9)
    tok, lp, got = host(tok), host(lp), host(logits)
    for k in range(K):
        prev = w.anchor if k == 0 else tok[:, k - 1]
        ref = O.markov_logits(w.U[:, k], w.W1, w.W2T, prev, w2_layout=O.W2_VR,
                              Hk=None if H is None else H[:, k].astype(np.float64))
        err = np.abs(got[:, k] - ref).max()
        assert err <= (LOGIT_TOL if gated else 1e-3), (k, err)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, H=None if H is None else H.astype(np.float64), mode=mode,
                         seed=13, temperature=0.9, follow=tok)
    check_draft(tok, lp, ref, what=f"round logits {shape}")


def test_round_logits_rejects_other_paths(D):
    """The validation call exists for the whole-round kernel only: an fp32-weight shape is refused."""
    w = S.strong("serving", B=2, K=2, V=300, r=16, wdtype=S.F32)
    with pytest.raises(D.DsparkError) as e:
        D.dspark_markov_draft_logits(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    assert e.value.status == D.DSPARK_EUNSUPPORTED


@pytest.mark.parametrize("cfg,mode", [("batch1", S.GREEDY), ("serving", S.SAMPLE)])
def test_gate_ones_equals_ungated_at_full_shapes(D, cfg, mode):
    """H = 1 makes the gated head the ungated one (equivalence page, "The equivalence: remove the gate"), at the
    batch-1 (greedy) and serving (sampling) shapes: the gated and ungated kernels draft the same tokens.  At the
    serving shape both run the same consumer arrangement, so log-probabilities agree bit for bit too."""
    w = S.workload(cfg)
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    a = D.dspark_markov_draft(*args, mode=mode, seed=w.noise_seed)
    ones = torch.ones((w.B, w.K, w.r), dtype=torch.float32, device="cuda")
    b = D.dspark_markov_draft(*args, mode=mode, seed=w.noise_seed, H=ones)
    assert np.array_equal(host(a[0]), host(b[0]))
    if cfg == "serving":
        assert np.array_equal(host(a[1]), host(b[1]))
    else:
        np.testing.assert_allclose(host(a[1]), host(b[1]), rtol=0, atol=1e-5)


def test_full_batch1_greedy(D):
    w = S.workload("batch1")
    _full_draft_check(D, w, None, S.GREEDY, 0, what="batch-1 greedy")


@pytest.mark.parametrize("extra", [0, 4], ids=["at-limit", "past-limit"])
@pytest.mark.parametrize("gated", [False, True], ids=["ungated", "gated"])
def test_batch1_resident_vocabulary_limit(D, extra, gated):
    """One row at r = 256, greedy: the resident round covers at most 640 ids per workgroup (one per lane of ten
    waves), so V = 640 x CUs is its largest vocabulary; four ids more take the tiled round.  Both against the
    oracle at every position."""
    V = 640 * torch.cuda.get_device_properties(0).multi_processor_count + extra
    w = S.workload("batch1", K=2, V=V)
    H = _rand_H(1, 2, 256, seed=5) if gated else None
    _full_draft_check(D, w, None, S.GREEDY, 0, H=None if H is None else t_f32(H),
                      Hd=None if H is None else H.astype(np.float64), what=f"batch-1 V={V}")


def test_cooperative_launch_matches_default(D):
    """The whole-round kernel launched cooperatively (guaranteed co-residency) drafts bit for bit what the
    default ordinary launch drafts."""
    w = S.strong("serving", B=128, K=3, V=4096, r=256, mode=S.SAMPLE)
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    a = D.dspark_markov_draft(*args, mode=D.DSPARK_SAMPLE, seed=4)
    D.dspark_set_cooperative_launch(True)
    try:
        b = D.dspark_markov_draft(*args, mode=D.DSPARK_SAMPLE, seed=4)
    finally:
        D.dspark_set_cooperative_launch(False)
    assert np.array_equal(host(a[0]), host(b[0])) and np.array_equal(host(a[1]), host(b[1]))


@pytest.mark.parametrize("B,r", [(16, 64), (1, 256), (16, 256)], ids=["tiled", "resident", "resident-mfma"])
def test_device_timeout_is_reported(D, B, r):
    """Failure path of the whole-round kernels (the tiled round, the resident round of a single row at r = 256,
    and the matrix-core resident round of up to 64 rows at r = 256), forced from the host: a spin limit of one
    sleep makes their bounded waits give up (every wait still ends, so the kernel exits normally).  The status
    call then reports DSPARK_EDEVICE; with the default limit restored the same workspace drafts correctly and
    reports OK."""
    w = S.workload("serving", B=B, K=3, V=4096, r=r, mode=S.GREEDY)
    args = (t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor))
    nbytes = D.dspark_markov_workspace_bytes(w.B, w.K, w.V, w.r, D.DSPARK_BF16, D.DSPARK_W2_VR)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    D.dspark_set_spin_limit(1)
    try:
        D.dspark_markov_draft(*args, workspace=ws)
        status = D.dspark_markov_status(ws, w.B, w.K)
    finally:
        D.dspark_set_spin_limit(0)
    assert status == D.DSPARK_EDEVICE
    tok, lp = D.dspark_markov_draft(*args, workspace=ws)
    assert D.dspark_markov_status(ws, w.B, w.K) == D.DSPARK_OK
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, follow=tok)
    check_draft(tok, lp, ref, what="after a forced timeout")


@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_many_row_blocks(D, mode):
    """B = 512: four 128-row blocks per position on the whole-round path (each block is a segment of its own
    with the predecessors of the same position)."""
    w = S.strong("serving", B=512, K=3, V=2048, r=64, mode=mode)
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), w2_layout=D.DSPARK_W2_VR,
                                    mode=mode, seed=w.noise_seed)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=w.noise_seed, follow=tok)
    check_draft(tok, lp, ref, what="B512")


def test_all_logits_equal(D):
    """Degenerate rows: U constant and W2 = 0, so every id ties.  Greedy takes the lowest id at every
    position and its log-probability is -ln V (closed form); the pick keeps the lowest id across lanes,
    tiles and workgroups alike."""
    B, K, V, r = 130, 3, 4000, 64
    U = np.full((B, K, V), 1.25, np.float32)
    W1 = S.f32_to_bf16(np.ones((V, r), np.float32))
    W2T = np.zeros((V, r), np.uint16)
    anchor = np.arange(B, dtype=np.int32) % V
    tok, lp = D.dspark_markov_draft(t_f32(U), t_w(W1), t_w(W2T), t_i32(anchor), w2_layout=D.DSPARK_W2_VR)
    assert np.all(host(tok) == 0)
    np.testing.assert_allclose(host(lp), -np.log(V), rtol=0, atol=1e-5)


@pytest.mark.parametrize("T", [0.05, 10.0])
def test_sampling_temperature_extremes(D, T):
    """Very sharp and very flat sampling both follow the oracle (keys l / T + G, log softmax of l / T)."""
    w = S.strong("serving", B=24, K=4, V=3000, r=64, mode=S.SAMPLE)
    tok, lp = D.dspark_markov_draft(t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor), w2_layout=D.DSPARK_W2_VR,
                                    mode=D.DSPARK_SAMPLE, seed=99, temperature=T)
    tok, lp = host(tok), host(lp)
    ref = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=O.SAMPLE, seed=99, temperature=T, follow=tok)
    check_draft(tok, lp, ref, what=f"T={T}")


@pytest.mark.parametrize("shape", [(128, 3, 4096, 256), (5, 3, 1001, 64), (5, 3, 1001, 80)],
                         ids=["round", "small-round", "per-position"])
def test_timed_draft_matches_plain_draft(D, shape):
    """The bench's timed entry point drafts exactly what dspark_markov_draft drafts and reports its launches."""
    import torch

    B, K, V, r = shape
    w = S.strong("serving", B=B, K=K, V=V, r=r)
    args = (t_f32(w.U), t_w(w.W1), t_w(np.ascontiguousarray(w.W2.T)), t_i32(w.anchor))
    kw = dict(w2_layout=D.DSPARK_W2_VR, mode=D.DSPARK_SAMPLE, seed=w.noise_seed)
    tok, lp = D.dspark_markov_draft(*args, **kw)
    tok2, lp2, kms, nl, rms = D.dspark_markov_draft_timed(*args, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(host(tok), host(tok2)) and np.array_equal(host(lp), host(lp2))
    round_path = V % 4 == 0 and r % 16 == 0 and r <= 256
    small_round = V * r <= 65536  # the one-launch vector-ALU round
    assert nl == (1 if round_path or small_round else K)
    assert 0.0 < kms <= rms * 1.05
