"""Pins of the fp64 CPU oracle against what the pages and the mathematics fix (CPU only).

Each test names what it pins: a value the pages print, a closed form, a special case that reduces to
a textbook/library routine, an invariant, or brute force on tiny inputs.  Nothing here compares the
oracle with itself.
"""
import math
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle as O
import synth as S

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f64(w):
    """Stored weights (float32, or uint16 bf16 bits) as exact float64."""
    return S.bf16_to_f32(w).astype(np.float64) if w.dtype == np.uint16 else w.astype(np.float64)


def rng_weights(rng, shape, sigma, dtype):
    w = (rng.standard_normal(shape) * sigma).astype(np.float32)
    return S.f32_to_bf16(w) if dtype == "bf16" else w


# ------------------------------------------------------------------------------------------ noise

def test_fmix32_published_vectors():
    """MurmurHash3's finaliser against the published empty-key verification vectors."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "murmur3_fmix32.txt")) if l.strip() and l[0] != "#"]
    assert len(rows) == 3
    for seed, expect in rows:
        assert O.fmix32(int(seed, 16)) == int(expect, 16)


def test_noise_uniform_is_odd_lattice_in_open_interval():
    u, _ = O.noise_fill(0x5EED, 3, 5, 0, 1 << 16)
    assert np.all(u > 0) and np.all(u < 1)
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m).astype(np.int64) % 2 == 1)


def test_noise_uniform_chi2():
    u, _ = O.noise_fill(0x1234, 7, 2, 0, 1 << 20)
    counts = np.bincount((u * 256).astype(np.int64), minlength=256)
    chi2 = ((counts - u.size / 256) ** 2 / (u.size / 256)).sum()
    assert stats.chi2.sf(chi2, 255) > 1e-4


def test_gumbel_moments_and_transform():
    """Closed form: a standard Gumbel has mean = Euler-Mascheroni and variance pi^2/6."""
    gs, us = [], []
    for pos in range(4):
        u, g = O.noise_fill(0x5EED, 11, pos, 0, 1 << 20)
        gs.append(g)
        us.append(u)
    g = np.concatenate(gs)
    u = np.concatenate(us)
    n = g.size
    sigma2 = math.pi ** 2 / 6
    assert abs(g.mean() - np.euler_gamma) < 5 * math.sqrt(sigma2 / n)
    # var of the sample variance: (mu4 - sigma^4)/n with mu4 = (3 + 12/5) sigma^4
    assert abs(g.var() - sigma2) < 5 * sigma2 * math.sqrt(4.4 / n)
    # G = -log(-log(u)) as numpy computes it
    np.testing.assert_allclose(g[:4096], -np.log(-np.log(u[:4096])), rtol=0, atol=1e-15)
    # support of the 23-bit lattice
    assert g.min() > -2.82 and g.max() < 16.65


def test_noise_depends_on_every_key_field():
    base = O.noise_bits(0x5EED, 1, 2, 3)
    assert O.noise_bits(0x5EED + 1, 1, 2, 3) != base
    assert O.noise_bits(0x5EED, 0, 2, 3) != base
    assert O.noise_bits(0x5EED, 1, 3, 3) != base
    assert O.noise_bits(0x5EED, 1, 2, 4) != base
    assert O.noise_bits(0x5EED | (1 << 40), 1, 2, 3) != base


# ------------------------------------------------------------------------------------ the bias term

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout", [O.W2_RV, O.W2_VR])
def test_logits_match_numpy_matmul(dtype, layout):
    """Library routine: U_k + W1[prev] @ W2 by numpy float64 matmul, in both storage orders."""
    rng = np.random.default_rng(1)
    B, V, r = 5, 37, 12
    U = rng.standard_normal((B, V)).astype(np.float32)
    W1 = rng_weights(rng, (V, r), 0.7, dtype)
    W2 = rng_weights(rng, (r, V), 0.7, dtype)
    prev = rng.integers(0, V, B).astype(np.int32)
    W2s = W2 if layout == O.W2_RV else np.ascontiguousarray(W2.T)
    got = O.markov_logits(U, W1, W2s, prev, w2_layout=layout)
    want = U.astype(np.float64) + f64(W1)[prev] @ f64(W2)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert np.abs(want - U).max() > 0.5  # the bias is not negligible here


def test_logits_onehot_closed_form():
    """Closed form: W1[a] = e_(a mod r) makes the bias row a copy of W2[a mod r, :], exactly."""
    rng = np.random.default_rng(2)
    B, V, r = 6, 50, 8
    U = rng.standard_normal((B, V)).astype(np.float32)
    W1 = np.zeros((V, r), np.float32)
    W1[np.arange(V), np.arange(V) % r] = 1.0
    W2 = rng.standard_normal((r, V)).astype(np.float32)
    prev = np.array([0, 3, 7, 8, 13, 49], np.int32)
    got = O.markov_logits(U, W1, W2, prev)
    want = U.astype(np.float64) + W2[prev % r].astype(np.float64)
    assert np.array_equal(got, want)


def test_logits_rank1_closed_form():
    """Closed form: W1[a] = alpha_a u and W2[:, v] = beta_v w give bias = alpha_a beta_v (u . w)."""
    rng = np.random.default_rng(3)
    B, V, r = 4, 33, 16
    alpha = rng.integers(-4, 5, V).astype(np.float64) / 4
    beta = rng.integers(-4, 5, V).astype(np.float64) / 8
    u = rng.integers(-3, 4, r).astype(np.float64)
    w = rng.integers(-3, 4, r).astype(np.float64)
    W1 = np.outer(alpha, u).astype(np.float32)
    W2 = np.outer(w, beta).astype(np.float32)
    U = rng.standard_normal((B, V)).astype(np.float32)
    prev = rng.integers(0, V, B).astype(np.int32)
    got = O.markov_logits(U, W1, W2, prev)
    want = U.astype(np.float64) + np.outer(alpha[prev], beta) * float(u @ w)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------- the pick and chain

def test_w2_zero_greedy_is_per_position_argmax():
    """Special case ("markov rank 0 disables the head"): with W2 = 0 the greedy draft is the
    per-position argmax of U, ties to the lower id, and the log-probability is log softmax(U)."""
    rng = np.random.default_rng(4)
    B, K, V, r = 6, 5, 40, 8
    U = np.round(rng.standard_normal((B, K, V)) * 2).astype(np.float32)  # many exact ties
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = np.zeros((r, V), np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    res = O.markov_draft(U, W1, W2, anchor)
    U64 = U.astype(np.float64)
    assert np.array_equal(res["tokens"], np.argmax(U64, axis=-1))
    want_lp = np.take_along_axis(U64, res["tokens"][..., None].astype(np.int64), -1)[..., 0] - special.logsumexp(U64, -1)
    np.testing.assert_allclose(res["logprobs"], want_lp, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_whole_vocabulary_draw_follows_softmax(T):
    """Statistics: with W2 = 0 the logits are U, so a whole-vocabulary draw must follow softmax(U/T).
    V = 40 spans three blocks of the race (16, 16 and a short one of 8); one row replicated over 2^16
    rows (the noise keys on the row) gives independent draws, compared by chi-square.  A wrong race
    value (block mass without its variate, or the variate without the mass), a wrong block grouping or a
    reversed inverse CDF each fail.  The reported log-probability is the exact log-softmax."""
    rng = np.random.default_rng(5)
    V, r, n = 40, 8, 1 << 16
    u = (rng.standard_normal(V) * 1.3).astype(np.float32)
    U = np.broadcast_to(u, (n, 1, V)).copy()
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = np.zeros((r, V), np.float32)
    anchor = np.zeros(n, np.int32)
    res = O.markov_draft(U, W1, W2, anchor, mode=O.SAMPLE, seed=99, temperature=T)
    p = special.softmax(u.astype(np.float64) / T)
    counts = np.bincount(res["tokens"][:, 0], minlength=V)
    expect = p * n
    keep = expect > 5
    chi2 = ((counts[keep] - expect[keep]) ** 2 / expect[keep]).sum()
    assert stats.chi2.sf(chi2, keep.sum() - 1) > 1e-4
    lp = np.log(p)
    np.testing.assert_allclose(res["logprobs"][:, 0], lp[res["tokens"][:, 0]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("V", [1, 7, 16])
def test_single_block_draw_is_inverse_transform_sampling(V):
    """Special case: with V <= 16 the race has one block, and the draw reduces to inverse transform
    sampling of softmax(l/T) with the uniform of noise id 1: numpy's searchsorted over the cumulative
    masses (first id whose inclusive prefix exceeds u times the total)."""
    rng = np.random.default_rng(40 + V)
    B, K, r, T = 64, 3, 4, 0.8
    U = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    W1 = np.zeros((V, r), np.float32)
    W2 = np.zeros((r, V), np.float32)
    res = O.markov_draft(U, W1, W2, np.zeros(B, np.int32), mode=O.SAMPLE, seed=3, temperature=T)
    for b in range(B):
        for k in range(K):
            z = U[b, k].astype(np.float64) / T
            w = np.exp(z - z.max())
            cum = np.cumsum(w)
            tok = int(np.searchsorted(cum, O.noise_uniform(3, b, k, 1) * cum[-1], side="right"))
            assert res["tokens"][b, k] == min(tok, V - 1)


def test_two_point_race_is_the_exponential_race():
    """Special case: two blocks, each with its mass on one id (ids 3 and 20, logits a and b; every other
    logit is -1e30).  The draw is then the plain exponential race of two clocks: id 3 exactly when
    e^a / E_0 > e^b / E_1 with E_j = -ln u(2j), and id 3 has probability e^a / (e^a + e^b)."""
    rng = np.random.default_rng(17)
    n, V, r = 1 << 14, 32, 4
    a, b = 0.4, -0.3
    U = np.full((n, 1, V), -1e30, np.float32)
    U[:, 0, 3] = a
    U[:, 0, 20] = b
    res = O.markov_draft(U, np.zeros((V, r), np.float32), np.zeros((r, V), np.float32), np.zeros(n, np.int32),
                         mode=O.SAMPLE, seed=11)
    for row in rng.integers(0, n, 200):
        e0 = -math.log(O.noise_uniform(11, int(row), 0, 0))
        e1 = -math.log(O.noise_uniform(11, int(row), 0, 2))
        assert res["tokens"][row, 0] == (3 if math.exp(a) / e0 > math.exp(b) / e1 else 20)
    frac = float(np.mean(res["tokens"][:, 0] == 3))
    pa = math.exp(a) / (math.exp(a) + math.exp(b))
    assert abs(frac - pa) < 5 * math.sqrt(pa * (1 - pa) / n)


def _strong_tiny(V=5, K=3, r=4, seed=6, gated=False):
    rng = np.random.default_rng(seed)
    U = (rng.standard_normal((1, K, V)) * 1.5).astype(np.float32)
    W1 = (rng.standard_normal((V, r)) * 0.9).astype(np.float32)
    W2 = (rng.standard_normal((r, V)) * 0.9).astype(np.float32)
    anchor = np.array([rng.integers(0, V)], np.int32)
    H = rng.uniform(0.1, 1.0, (1, K, r)) if gated else None
    return U, W1, W2, anchor, H


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("T", [1.0, 1.6])
def test_enumeration_is_normalised(gated, T):
    """Local normalisation: the K locally normalised factors make a distribution over all V^K paths."""
    U, W1, W2, anchor, H = _strong_tiny(gated=gated)
    logq = O.enumerate_paths(U[0], W1, W2, anchor[0], H_row=None if H is None else H[0], temperature=T)
    assert abs(np.exp(logq).sum() - 1.0) < 1e-12


def test_follow_logprob_sums_to_path_probability():
    """Brute force: sum over positions of the per-position log-probability of a path equals the
    enumerated log q of that path (the draft distribution is the product of local factors)."""
    U, W1, W2, anchor, _ = _strong_tiny(V=6, K=3)
    logq = O.enumerate_paths(U[0], W1, W2, anchor[0])
    rng = np.random.default_rng(7)
    for _ in range(20):
        path = rng.integers(0, 6, 3).astype(np.int32)
        res = O.markov_draft(U, W1, W2, anchor, follow=path[None])
        assert abs(res["lp_follow"][0].sum() - logq[tuple(path)]) < 1e-12


def test_greedy_chain_matches_brute_force_conditionals():
    """Brute force: the first greedy token maximises the enumerated marginal q(t1) (which equals the
    local softmax because later factors sum to one); each later token maximises q(prefix, t)."""
    for seed in range(8):
        U, W1, W2, anchor, _ = _strong_tiny(V=5, K=3, seed=100 + seed)
        q = np.exp(O.enumerate_paths(U[0], W1, W2, anchor[0]))
        res = O.markov_draft(U, W1, W2, anchor)
        t = res["tokens"][0]
        assert t[0] == np.argmax(q.sum(axis=(1, 2)))
        assert t[1] == np.argmax(q[t[0]].sum(axis=1))
        assert t[2] == np.argmax(q[t[0], t[1]])


@pytest.mark.parametrize("gated", [False, True])
def test_gumbel_max_sampler_matches_enumerated_distribution(gated):
    """Statistics against brute force: one row replicated over 2^16 rows (the noise keys on the row)
    gives independent samples whose path frequencies follow the enumerated q (chi-square)."""
    V, K, r = 4, 2, 4
    U, W1, W2, anchor, H = _strong_tiny(V=V, K=K, r=r, seed=8, gated=gated)
    q = np.exp(O.enumerate_paths(U[0], W1, W2, anchor[0], H_row=None if H is None else H[0]))
    n = 1 << 16
    Ub = np.repeat(U, n, axis=0)
    Hb = None if H is None else np.repeat(H, n, axis=0)
    res = O.markov_draft(Ub, W1, W2, np.repeat(anchor, n), H=Hb, mode=O.SAMPLE, seed=0xABCD)
    idx = res["tokens"][:, 0] * V + res["tokens"][:, 1]
    counts = np.bincount(idx, minlength=V ** K)
    expect = q.reshape(-1) * n
    keep = expect > 5
    chi2 = ((counts[keep] - expect[keep]) ** 2 / expect[keep]).sum()
    assert stats.chi2.sf(chi2, keep.sum() - 1) > 1e-4
    # the reported log-probability of every sample is its exact local log-softmax: sum = log q(path)
    lq = np.log(q.reshape(-1))[idx[:100]]
    np.testing.assert_allclose(res["logprobs"][:100].sum(axis=1), lq, rtol=0, atol=1e-12)


def _np_torch(L=40.0, markov=True):
    """The page's np/torch example: ids 0 = anchor 'x =', 1 = np, 2 = torch, 3 = .array, 4 = .tensor."""
    V, K, r = 5, 2, 2
    U = np.full((1, K, V), -L, np.float32)
    U[0, 0, [1, 2]] = 0.0
    U[0, 1, [3, 4]] = 0.0
    W1 = np.zeros((V, r), np.float32)
    W1[1] = (1, 0)
    W1[2] = (0, 1)
    W2 = np.zeros((r, V), np.float32)
    if markov:
        W2[:, 3] = (0, -L)
        W2[:, 4] = (-L, 0)
    return U, W1, W2, np.zeros(1, np.int32)


def _golden_tables():
    t = {}
    for line in open(os.path.join(GOLDEN, "np_torch_tables.txt")):
        if line.strip() and line[0] != "#":
            k, *vals = line.split()
            t[k] = vals
    return (np.array(t["joint"], float).reshape(2, 2), np.array(t["product"], float).reshape(2, 2),
            math.log(2) if t["kl_joint_product"] == ["ln2"] else None)


def test_np_torch_worked_example_tables():
    """Values the page prints: the Markov head reproduces the joint table; with the head disabled the
    draft is the product of the marginals; KL(joint || product) = total correlation = ln 2."""
    joint, product, kl = _golden_tables()
    q = np.exp(O.enumerate_paths(*[a[0] if i in (0, 3) else a for i, a in enumerate(_np_torch())]))
    np.testing.assert_allclose(q[1:3, 3:5], joint, rtol=0, atol=1e-12)
    assert abs(q.sum() - 1) < 1e-12
    U, W1, W2, anchor = _np_torch(markov=False)
    q0 = np.exp(O.enumerate_paths(U[0], W1, W2, anchor[0]))
    np.testing.assert_allclose(q0[1:3, 3:5], product, rtol=0, atol=1e-12)
    p = q[1:3, 3:5]
    prod = np.outer(p.sum(1), p.sum(0))
    nz = p > 1e-300
    assert abs((p[nz] * np.log(p[nz] / prod[nz])).sum() - kl) < 1e-9


def test_np_torch_sampled_pairs_never_splice():
    """The page's sampled table: with the Markov head the off-diagonal cells (np .tensor, torch
    .array) receive no samples, the diagonal about half each; without it each cell gets a quarter."""
    n = 1 << 14
    for markov, want in ((True, np.array([[0.5, 0], [0, 0.5]])), (False, np.full((2, 2), 0.25))):
        U, W1, W2, anchor = _np_torch(markov=markov)
        res = O.markov_draft(np.repeat(U, n, 0), W1, W2, np.repeat(anchor, n), mode=O.SAMPLE, seed=0x5EED)
        t = res["tokens"]
        tab = np.zeros((2, 2))
        np.add.at(tab, (t[:, 0] - 1, t[:, 1] - 3), 1)
        assert tab.sum() == n
        if markov:
            assert tab[0, 1] == 0 and tab[1, 0] == 0
        frac = tab / n
        assert np.all(np.abs(frac - want) < 5 * np.sqrt(np.maximum(want * (1 - want), 1e-12) / n) + 1e-12)


# --------------------------------------------------------------------------------------------- gate

def test_gate_matches_numpy_and_zero_weights():
    rng = np.random.default_rng(9)
    rows, D, r = 7, 64, 16
    h = S.f32_to_bf16(rng.standard_normal((rows, D)).astype(np.float32))
    Wg = S.f32_to_bf16((rng.standard_normal((D, r)) * 0.2).astype(np.float32))
    H = O.gate(h, Wg)
    want = 1.0 / (1.0 + np.exp(-(f64(h) @ f64(Wg))))
    np.testing.assert_allclose(H, want, rtol=0, atol=1e-14)
    H0 = O.gate(h, np.zeros_like(Wg))
    assert np.all(H0 == 0.5)  # sigma(0) = 1/2 exactly


def test_gate_ones_is_ungated_and_half_halves_bias():
    """[MvS] "The equivalence": H = 1 recovers the ungated head exactly; H = 1/2 halves the bias."""
    rng = np.random.default_rng(10)
    B, K, V, r = 3, 4, 30, 8
    U = rng.standard_normal((B, K, V)).astype(np.float32)
    W1 = rng.standard_normal((V, r)).astype(np.float32)
    W2 = rng.standard_normal((r, V)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    a = O.markov_draft(U, W1, W2, anchor, mode=O.SAMPLE, seed=3)
    b = O.markov_draft(U, W1, W2, anchor, H=np.ones((B, K, r)), mode=O.SAMPLE, seed=3)
    for key in ("tokens", "logprobs", "margins"):
        assert np.array_equal(a[key], b[key])
    prev = rng.integers(0, V, B).astype(np.int32)
    l1 = O.markov_logits(U[:, 0], W1, W2, prev)
    lh = O.markov_logits(U[:, 0], W1, W2, prev, Hk=np.full((B, r), 0.5))
    np.testing.assert_allclose(lh - U[:, 0], 0.5 * (l1 - U[:, 0]), rtol=0, atol=1e-12)


# -------------------------------------------------------------------------------------------- top-k

@pytest.mark.parametrize("k", [1, 16, 61])
def test_topk_matches_lexsort(k):
    """Textbook routine: a full sort by (value desc, id asc); ties and signed zeros included."""
    rng = np.random.default_rng(11)
    rows, V = 40, 61
    U = np.round(rng.standard_normal((rows, V)) * 2).astype(np.float32)
    U[0] = 0.0
    U[1, ::2] = -0.0
    U[2, :] = 5.0
    U[3, ::3] = np.float32(3.0)
    idx, val = O.topk(U, k)
    for i in range(rows):
        order = np.lexsort((np.arange(V), -U[i].astype(np.float64)))[:k]
        assert np.array_equal(idx[i], order)
        assert np.array_equal(val[i], U[i, order])


# ----------------------------------------------------------------------------------------- selector

@pytest.mark.parametrize("mode", [O.GREEDY, O.SAMPLE])
@pytest.mark.parametrize("gated", [False, True])
def test_selector_equals_markov_restricted_to_its_candidates(mode, gated):
    """[MvS] "Two implications": the Selector is the (gated) Markov head executed on fixed top-k sets;
    with W1 := A and W2 := Bemb^T it must equal the head restricted to the same candidate sets."""
    rng = np.random.default_rng(12)
    B, K, V, r, topk = 4, 5, 48, 8, 6
    U = (rng.standard_normal((B, K, V)) * 2).astype(np.float32)
    A = S.f32_to_bf16((rng.standard_normal((V, r)) * 0.8).astype(np.float32))
    Bemb = S.f32_to_bf16((rng.standard_normal((V, r)) * 0.8).astype(np.float32))
    anchor = rng.integers(0, V, B).astype(np.int32)
    H = rng.uniform(0, 1, (B, K, r)) if gated else None
    sel = O.selector_draft(U, A, Bemb, anchor, H=H, topk=topk, mode=mode, seed=21, temperature=0.9)
    cand, _ = O.topk(U, topk)
    assert np.array_equal(sel["cand"], cand)
    res = O.markov_restricted(U, A, Bemb, anchor, cand, w2_layout=O.W2_VR, H=H, mode=mode, seed=21, temperature=0.9)
    for key in ("tokens", "logprobs", "margins"):
        assert np.array_equal(sel[key], res[key])
    assert np.all(np.isin(sel["tokens"], cand.reshape(B, -1)))


@pytest.mark.parametrize("mode", [O.GREEDY, O.SAMPLE])
def test_selector_with_topk_V_is_the_full_head(mode):
    """Special case (spec: top-k = V on a tiny vocabulary): with the candidate set equal to the whole
    vocabulary the truncation is exact, in both modes and bit for bit: the sampling draw is one definition
    over a set of ids (race between vocabulary blocks, noise keyed on the block, sums in ascending id order),
    so a candidate list in any slot order that holds every id draws what the whole vocabulary draws."""
    w = S.strong("tiny", V=64, K=4)
    sel = O.selector_draft(w.U, w.W1, np.ascontiguousarray(w.W2.T), w.anchor, topk=w.V, mode=mode, seed=5,
                           temperature=0.8)
    full = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=5, temperature=0.8)
    assert np.array_equal(sel["tokens"], full["tokens"])
    assert np.array_equal(sel["logprobs"], full["logprobs"])
    assert np.array_equal(sel["margins"], full["margins"])
    # the candidate order is (U desc, id asc), not id order, so the equality is not a trivial one
    assert not np.array_equal(sel["cand"][0, 0], np.arange(w.V))


def _one_row_restricted(U_row, cand_row, mode, seed, T, n):
    """The restricted head at one position (W2 = 0, so the logits are U) for n replicated rows."""
    V = U_row.shape[0]
    r = 2
    U = np.broadcast_to(U_row, (n, 1, V)).copy()
    cand = np.broadcast_to(np.asarray(cand_row, np.int32), (n, 1, len(cand_row))).copy()
    return O.markov_restricted(U, np.zeros((V, r), np.float32), np.zeros((r, V), np.float32),
                               np.zeros(n, np.int32), cand, mode=mode, seed=seed, temperature=T)


@pytest.mark.parametrize("T", [0.5, 2.0])
def test_restricted_draw_one_member_per_block_is_gumbel_max(T):
    """Special case: when every candidate sits in a vocabulary block of its own, the race between blocks is
    the textbook Gumbel-max over the candidates, argmax_c l_c / T + G(seed, row, pos, 2 (c div 16)), with G
    the noise function pinned above (published hash vectors, Gumbel moments).  numpy argmax over the same
    keys, per row; at T != 1 a key of l T instead of l / T, or noise subtracted instead of added, differs."""
    rng = np.random.default_rng(60)
    V, n = 400, 512
    blocks = rng.choice(V // 16, 12, replace=False)
    cand = (16 * blocks + rng.integers(0, 16, blocks.size)).astype(np.int32)
    rng.shuffle(cand)
    u = (rng.standard_normal(V) * 1.5).astype(np.float32)
    res = _one_row_restricted(u, cand, O.SAMPLE, 41, T, n)
    l = u[cand].astype(np.float64)
    for row in range(n):
        g = np.array([O.gumbel(41, row, 0, 2 * int(c // 16)) for c in cand])
        assert res["tokens"][row, 0] == cand[int(np.argmax(l / T + g))]
    p = special.softmax(l / T)
    lp = np.log(p)[[int(np.nonzero(cand == t)[0][0]) for t in res["tokens"][:, 0]]]
    np.testing.assert_allclose(res["logprobs"][:, 0], lp, rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [0.6, 1.7])
def test_restricted_draw_inside_one_block_is_inverse_transform(T):
    """Special case: when every candidate sits in one vocabulary block q, the race has one entrant and the
    draw is inverse transform sampling of softmax(l / T) over the candidates in ascending id order with the
    uniform of noise id 2q + 1: numpy searchsorted over the cumulative masses (first inclusive prefix above u
    times the total), whatever the slot order of the candidate list."""
    rng = np.random.default_rng(61)
    V, n = 200, 256
    q = 7
    cand = (16 * q + rng.choice(16, 9, replace=False)).astype(np.int32)
    u = (rng.standard_normal(V) * 2.0).astype(np.float32)
    res = _one_row_restricted(u, cand, O.SAMPLE, 5, T, n)
    ids = np.sort(cand)
    z = u[ids].astype(np.float64) / T
    w = np.exp(z - z.max())
    cum = np.cumsum(w)
    for row in range(n):
        j = int(np.searchsorted(cum, O.noise_uniform(5, row, 0, 2 * q + 1) * cum[-1], side="right"))
        assert res["tokens"][row, 0] == ids[min(j, ids.size - 1)]


@pytest.mark.parametrize("T", [0.6, 1.7])
def test_restricted_draw_follows_softmax_over_the_set(T):
    """Statistics: a candidate set spread over blocks with one, several and all but one of their ids, one
    row replicated over 2^16 rows (the noise keys on the row): the draw frequencies follow softmax(l / T)
    over the set (chi-square), and the reported log-probability is the exact log-softmax over the set.  A
    temperature applied as l T, noise with the wrong sign, block masses without their variates or a
    reversed inverse CDF each fail."""
    rng = np.random.default_rng(62)
    V, n = 160, 1 << 16
    cand = np.concatenate([[5], 16 * 2 + np.arange(4), 16 * 5 + np.delete(np.arange(16), 3), [16 * 9 + 11]])
    cand = rng.permutation(cand).astype(np.int32)
    u = (rng.standard_normal(V) * 1.2).astype(np.float32)
    u[16 * 5: 16 * 6] -= 1.5  # the big block is not the obvious winner
    res = _one_row_restricted(u, cand, O.SAMPLE, 0xBEEF, T, n)
    l = u[cand].astype(np.float64)
    p = special.softmax(l / T)
    order = np.argsort(cand)  # ascending ids
    counts = np.bincount(np.searchsorted(cand[order], res["tokens"][:, 0]), minlength=cand.size)
    expect = p[order] * n
    keep = expect > 5
    chi2 = ((counts[keep] - expect[keep]) ** 2 / expect[keep]).sum()
    assert stats.chi2.sf(chi2, keep.sum() - 1) > 1e-4
    lp_of = dict(zip(cand.tolist(), np.log(p).tolist()))
    want = np.array([lp_of[int(t)] for t in res["tokens"][:, 0]])
    np.testing.assert_allclose(res["logprobs"][:, 0], want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("k", [2, 4, 8, 16])
def test_truncated_greedy_is_exact_until_the_full_pick_leaves_the_candidates(k):
    """[MvS] "Two implications", second point: an already trained head executed on the top-k candidates.
    An argmax over a subset that contains the global argmax is the global argmax, so along every row the
    truncated greedy walk equals the full-vocabulary greedy head up to the first position whose full pick
    is not a candidate (fp64: no ties).  Strong bias so that the truncation does change some drafts."""
    rng = np.random.default_rng(30 + k)
    B, K, V, r = 12, 6, 200, 16
    U = rng.standard_normal((B, K, V)).astype(np.float32)
    A = S.f32_to_bf16((rng.standard_normal((V, r)) * 0.7).astype(np.float32))
    Bemb = S.f32_to_bf16((rng.standard_normal((V, r)) * 0.7).astype(np.float32))
    anchor = rng.integers(0, V, B).astype(np.int32)
    sel = O.selector_draft(U, A, Bemb, anchor, topk=k)
    full = O.markov_draft(U, A, Bemb, anchor, w2_layout=O.W2_VR)
    diverged = 0
    for b in range(B):
        d = np.nonzero(sel["tokens"][b] != full["tokens"][b])[0]
        if d.size:
            t = int(d[0])
            assert full["tokens"][b, t] not in sel["cand"][b, t]
            diverged += 1
    if k == 2:
        assert diverged > 0  # the inputs do exercise the truncation


def test_selector_tables_match_numpy():
    rng = np.random.default_rng(13)
    B, K, V, r, topk = 2, 4, 30, 8, 5
    U = rng.standard_normal((B, K, V)).astype(np.float32)
    A = rng.standard_normal((V, r)).astype(np.float32)
    Bemb = rng.standard_normal((V, r)).astype(np.float32)
    anchor = rng.integers(0, V, B).astype(np.int32)
    H = rng.uniform(0, 1, (B, K, r))
    sel = O.selector_draft(U, A, Bemb, anchor, H=H, topk=topk)
    A64, B64 = A.astype(np.float64), Bemb.astype(np.float64)
    for b in range(B):
        c = sel["cand"][b]
        T0 = U[b, 0, c[0]] + (A64[anchor[b]] * H[b, 0]) @ B64[c[0]].T
        np.testing.assert_allclose(sel["tables"][b, :topk], T0, rtol=0, atol=1e-12)
        for t in range(1, K):
            Tt = U[b, t, c[t]][None, :] + (A64[c[t - 1]] * H[b, t][None, :]) @ B64[c[t]].T
            got = sel["tables"][b, topk + (t - 1) * topk * topk: topk + t * topk * topk].reshape(topk, topk)
            np.testing.assert_allclose(got, Tt, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------------- invariants

def test_rows_are_independent_and_restricted_full_sets_is_full():
    w = S.strong("tiny", B=4, V=96, K=3)
    full = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=O.SAMPLE, seed=7)
    one = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=O.SAMPLE, seed=7, rows=[2])
    assert np.array_equal(one["tokens"][2], full["tokens"][2])
    assert np.all(one["tokens"][[0, 1, 3]] == -1)
    # the head restricted to the whole vocabulary (as a shuffled candidate list) is the head, in both modes
    cand = np.stack([np.random.default_rng(i).permutation(w.V) for i in range(w.B * w.K)]).astype(np.int32)
    cand = cand.reshape(w.B, w.K, w.V)
    for mode in (O.GREEDY, O.SAMPLE):
        f = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=7)
        res = O.markov_restricted(w.U, w.W1, w.W2, w.anchor, cand, mode=mode, seed=7)
        assert np.array_equal(res["tokens"], f["tokens"])
        assert np.array_equal(res["logprobs"], f["logprobs"])


def test_shift_invariance():
    """Adding a constant to every base logit of a position changes neither the pick nor the
    log-probability (softmax and Gumbel-max are shift invariant).  The shifted U is re-rounded to
    fp32 (spacing 2^-13 near 1024), so picks are compared where the margin exceeds that rounding."""
    w = S.strong("tiny", B=3, V=80, K=4)
    U2 = (w.U.astype(np.float64) + 1024.0).astype(np.float32)
    for mode in (O.GREEDY, O.SAMPLE):
        a = O.markov_draft(w.U, w.W1, w.W2, w.anchor, mode=mode, seed=1)
        b = O.markov_draft(U2, w.W1, w.W2, w.anchor, mode=mode, seed=1)
        ok = a["margins"] > 1e-3
        assert ok.mean() > 0.9
        assert np.array_equal(a["tokens"][ok], b["tokens"][ok])
        np.testing.assert_allclose(a["logprobs"], b["logprobs"], rtol=0, atol=1e-3)


# -------------------------------------------------------------------------------------- reachability

@pytest.mark.parametrize("mode,T", [(O.GREEDY, 1.0), (O.SAMPLE, 1.0), (O.SAMPLE, 0.6)])
def test_reach_accepts_every_token_a_small_perturbation_selects(mode, T):
    """Brute force: the parity rule accepts a GPU token that differs from the oracle's pick only when a
    perturbation of at most eps of every key (greedy: l; sampling: l / T) selects it.  On positions whose
    margin is below 2 eps, random and corner perturbations (|delta| <= 0.98 eps) of the logits are applied and
    the position drawn again (same row, position and noise): every token so drawn must be declared reachable
    at the unperturbed logits.  The declared set stays small (it is not "anything goes"), and the
    perturbations do change some picks (the check is not vacuous)."""
    eps = O.REACH_EPS
    rng = np.random.default_rng(70 + int(10 * T) + mode)
    V, r = 48, 2
    W1, W2 = np.zeros((V, r), np.float32), np.zeros((r, V), np.float32)
    changed, checked, sizes = 0, 0, []
    for seed in range(4000):
        u = (rng.standard_normal(V) * (0.1 if mode == O.GREEDY else 1.0)).astype(np.float32)
        U = u[None, None, :]
        base = O.markov_draft(U, W1, W2, np.zeros(1, np.int32), mode=mode, seed=seed, temperature=T)
        if not base["margins"][0, 0] < 2 * eps:
            continue
        checked += 1
        reach = [int(O.markov_draft(U, W1, W2, np.zeros(1, np.int32), mode=mode, seed=seed, temperature=T,
                                    follow=np.array([[f]], np.int32))["reach"][0, 0]) for f in range(V)]
        assert reach[base["tokens"][0, 0]] == 1
        sizes.append(sum(reach))
        for j in range(48):
            d = rng.uniform(-1, 1, V) if j % 2 else rng.choice([-1.0, 1.0], V)
            Up = (u.astype(np.float64) + 0.98 * eps * T * d).astype(np.float32)[None, None, :]
            t2 = int(O.markov_draft(Up, W1, W2, np.zeros(1, np.int32), mode=mode, seed=seed, temperature=T)["tokens"][0, 0])
            changed += t2 != base["tokens"][0, 0]
            assert reach[t2] == 1, (seed, t2, base["tokens"][0, 0], base["margins"][0, 0])
        if checked >= 60:
            break
    assert checked >= 20 and changed > 0
    assert np.mean(sizes) < 6 and max(sizes) < V // 2, sizes


def test_reach_is_exact_for_greedy_and_rejects_far_tokens():
    """Closed form for greedy: a token is reachable exactly when its logit is within 2 eps of the largest."""
    rng = np.random.default_rng(80)
    V, r, eps = 64, 2, O.REACH_EPS
    u = (rng.standard_normal(V) * 0.03).astype(np.float32)
    U = u[None, None, :]
    W1, W2 = np.zeros((V, r), np.float32), np.zeros((r, V), np.float32)
    follow = np.arange(V, dtype=np.int32)[:, None]
    res = O.markov_draft(np.repeat(U, V, 0), W1, W2, np.zeros(V, np.int32), follow=follow)
    want = u.astype(np.float64) >= u.astype(np.float64).max() - 2 * eps
    assert np.array_equal(res["reach"][:, 0].astype(bool), want)
    assert 1 < want.sum() < V


# -------------------------------------------------------------------------------------- confidence head

def _conf_inputs(seed, B=3, K=5, D=40, V=30, r=8):
    rng = np.random.default_rng(seed)
    h = S.f32_to_bf16(rng.standard_normal((B, K, D)).astype(np.float32))
    W1 = S.f32_to_bf16((rng.standard_normal((V, r)) * 0.9).astype(np.float32))
    anchor = rng.integers(0, V, B).astype(np.int32)
    tokens = rng.integers(0, V, (B, K)).astype(np.int32)
    return h, W1, anchor, tokens


def test_confidence_zero_weights_halves_and_survival_is_a_power_of_two():
    """[DSp] "Confidence-scheduled verification": c_k = sigmoid(w^T [h_k; W1[x_{k-1}]]) and a_j = prod c_i.
    With w = 0 every c_k is sigmoid(0) = 1/2 and a_k = 2^-(k+1), exactly."""
    h, W1, anchor, tokens = _conf_inputs(40)
    D, r = h.shape[2], W1.shape[1]
    conf, surv = O.confidence(h, np.zeros(D + r, np.float32), W1, anchor, tokens)
    assert np.all(conf == 0.5)
    assert np.array_equal(surv, np.broadcast_to(0.5 ** np.arange(1, h.shape[1] + 1), surv.shape))


@pytest.mark.parametrize("j", [0, 5])
def test_confidence_predecessor_part_reads_the_previous_token(j):
    """With the h part zero and the W1 part the unit vector e_j, c_k is the sigmoid of one weight of the
    predecessor's row: W1[anchor, j] at k = 0 and W1[tokens[k-1], j] after (not the token at k)."""
    h, W1, anchor, tokens = _conf_inputs(41)
    B, K, D = h.shape
    r = W1.shape[1]
    w = np.zeros(D + r, np.float32)
    w[D + j] = 1.0
    conf, _ = O.confidence(h, w, W1, anchor, tokens)
    Wd = S.bf16_to_f32(W1).astype(np.float64)
    prev = np.concatenate([anchor[:, None], tokens[:, :-1]], axis=1)
    np.testing.assert_allclose(conf, 1.0 / (1.0 + np.exp(-Wd[prev, j])), rtol=0, atol=1e-15)


def test_confidence_hidden_part_and_symmetry():
    """With the W1 part zero and the h part s e_i, c_k = sigmoid(s h[b, k, i]); negating w maps c to 1 - c
    (sigmoid(-z) = 1 - sigmoid(z)), and survival is the running product, so it never increases."""
    h, W1, anchor, tokens = _conf_inputs(42)
    B, K, D = h.shape
    r = W1.shape[1]
    w = np.zeros(D + r, np.float32)
    w[7] = 0.75
    conf, _ = O.confidence(h, w, W1, anchor, tokens)
    hd = S.bf16_to_f32(h).astype(np.float64)
    np.testing.assert_allclose(conf, 1.0 / (1.0 + np.exp(-0.75 * hd[:, :, 7])), rtol=0, atol=1e-15)
    rng = np.random.default_rng(43)
    w = (rng.standard_normal(D + r) * 0.3).astype(np.float32)
    c1, s1 = O.confidence(h, w, W1, anchor, tokens)
    c2, _ = O.confidence(h, -w, W1, anchor, tokens)
    np.testing.assert_allclose(c1 + c2, 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(s1, axis=1) <= 0)
    np.testing.assert_allclose(s1, np.cumprod(c1, axis=1), rtol=1e-15, atol=0)


# ------------------------------------------------------------------------------------ prefix scheduling

def _survival(R, K, seed):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.3, 0.99, (R, K))
    return np.cumprod(c, axis=1).astype(np.float32)


def test_schedule_constant_sps_admits_everything():
    """[DSp] "Hardware-aware prefix scheduling": with a flat steps-per-second curve Theta is proportional to
    the expected committed tokens R + sum a, so every extension with positive survival is admitted."""
    a = _survival(4, 5, 1)
    lengths, theta = O.schedule_greedy(a, np.full(4 * 6 + 1, 2.0, np.float32))
    assert np.array_equal(lengths, np.full(4, 5))
    assert theta == pytest.approx(2.0 * (4 + a.astype(np.float64).sum()), rel=1e-12)


def test_schedule_cliff_admits_nothing():
    """If the target cannot run more than R tokens per step (SPS = 0 beyond B = R) the baseline wins."""
    R, K = 3, 4
    sps = np.zeros(R * (K + 1) + 1, np.float32)
    sps[: R + 1] = 1.0
    lengths, theta = O.schedule_greedy(_survival(R, K, 2), sps)
    assert np.array_equal(lengths, np.zeros(R)) and theta == 3.0


def test_schedule_hand_example():
    """SPS(B) = 1 / B makes Theta the committed tokens per target token: an extension is admitted while its
    survival exceeds the current ratio.  R = 2, a = [[0.9, 0.5], [0.8, 0.1]]: Theta(0) = 2/2 = 1 and
    adding 0.9 gives 2.9/3 < 1, so nothing is admitted; with SPS(B) = 1 (flat) everything is."""
    a = np.array([[0.9, 0.5], [0.8, 0.1]], np.float32)
    B = np.arange(0, 2 * 3 + 1, dtype=np.float64)
    sps = np.where(B > 0, 1.0 / np.maximum(B, 1), 0).astype(np.float32)
    lengths, theta = O.schedule_greedy(a, sps)
    assert np.array_equal(lengths, [0, 0]) and theta == pytest.approx(1.0, rel=1e-7)


def test_schedule_stops_when_theta_does_not_strictly_increase():
    """The stop rule of the greedy ("admit them while Theta increases", read as strictly increases): with a flat
    SPS an extension of survival 0 leaves Theta unchanged and is not admitted, nor is anything after it."""
    a = np.array([[0.5, 0.0, 0.0]], np.float32)
    sps = np.ones(1 * 4 + 1, np.float32)
    lengths, theta = O.schedule_greedy(a, sps)
    assert lengths.tolist() == [1] and theta == 1.5


@pytest.mark.parametrize("seed", range(6))
def test_schedule_greedy_against_brute_force(seed):
    """For n admitted extensions the best set is the top n by survival, so the optimum is the best Theta along
    the greedy order; the greedy stops at the first local maximum.  With a linear SPS curve Theta is
    unimodal along that order and the greedy is optimal; with any curve it never beats the optimum."""
    rng = np.random.default_rng(seed)
    R, K = 4, 4
    a = _survival(R, K, 100 + seed)
    B = np.arange(R * (K + 1) + 1, dtype=np.float64)
    lin = (10.0 - 0.35 * B).clip(0).astype(np.float32)
    lg, tg = O.schedule_greedy(a, lin)
    lb, tb = O.schedule_best(a, lin)
    assert tg == pytest.approx(tb, rel=1e-12)
    assert np.array_equal(lg, lb)
    bumpy = (10.0 - 0.35 * B + 0.8 * np.sin(B * (1.3 + 0.1 * seed))).clip(0).astype(np.float32)
    lg, tg = O.schedule_greedy(a, bumpy)
    _, tb = O.schedule_best(a, bumpy)
    assert tg <= tb + 1e-12
    assert np.all(lg >= 0) and np.all(lg <= K)
