"""Graph capture: a draft round (whole-round launch and position-by-position path), the Selector, and the
confidence head followed by the prefix scheduler, captured once on a side stream and replayed several times
with eager work and synchronisations between the replays; every replay must reproduce the eager outputs
bit for bit (the library clears its own counters inside its kernels and records no memset)."""
import numpy as np
import pytest
import torch

import synth as S
from helpers import t_f32, t_i32, t_w

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


def _replays_match(run, outputs, n=4):
    run()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outputs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for i in range(n):
        for o in outputs:
            o.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(o, r), i
        _ = (torch.randn(4096, device=outputs[0].device) * i).sum().item()  # eager work between replays


@pytest.mark.parametrize("shape", [(128, 4, 4096, 256, S.BF16), (8, 3, 1002, 64, S.BF16), (3, 3, 300, 24, S.F32),
                                   (1, 4, 3000, 256, S.BF16), (16, 4, 3000, 256, S.BF16)],
                         ids=["whole-round", "per-position-V%4", "per-position-fp32", "one-row-r256",
                              "16-rows-r256"])
@pytest.mark.parametrize("mode", [S.GREEDY, S.SAMPLE], ids=["greedy", "sample"])
def test_markov_draft_graph(D, shape, mode):
    B, K, V, r, wd = shape
    w = S.strong("serving", B=B, K=K, V=V, r=r, wdtype=wd, mode=mode)
    U, W1, W2T, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    tok = torch.empty((B, K), dtype=torch.int32, device="cuda")
    lp = torch.empty((B, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(D.dspark_markov_workspace_bytes(B, K, V, r, D.DSPARK_BF16 if wd == S.BF16 else D.DSPARK_F32,
                                                     D.DSPARK_W2_VR), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: D.dspark_markov_draft(U, W1, W2T, anc, w2_layout=D.DSPARK_W2_VR, mode=mode, seed=11,
                                                 temperature=0.8, tokens=tok, logprobs=lp, workspace=ws), [tok, lp])


def test_selector_graph(D):
    w = S.strong("selector", B=16, K=4, V=3000, r=64)
    U, A, Bm, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    ws = torch.empty(D.dspark_selector_workspace_bytes(16, 4, 3000, 64, 16), dtype=torch.uint8, device="cuda")
    out = {}

    def run():
        out.update(D.dspark_selector_draft(U, A, Bm, anc, topk=16, mode=D.DSPARK_SAMPLE, seed=3, workspace=ws))

    run()
    torch.cuda.synchronize()
    ref = (out["tokens"].clone(), out["logprobs"].clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run()  # outputs allocated inside the capture belong to the graph's pool
    torch.cuda.synchronize()
    for i in range(3):
        out["tokens"].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out["tokens"], ref[0]) and torch.equal(out["logprobs"], ref[1]), i


def test_confidence_and_schedule_graph(D):
    B, K, V, r, Dm = 32, 6, 2048, 64, 256
    w = S.strong("serving", B=B, K=K, V=V, r=r)
    U, W1, W2T, anc = t_f32(w.U), t_w(w.W1), t_w(w.W2T), t_i32(w.anchor)
    rng = np.random.default_rng(9)
    h = torch.from_numpy(S.f32_to_bf16(rng.standard_normal((B, K, Dm)).astype(np.float32)).view(np.int16)).cuda()
    h = h.view(torch.bfloat16)
    cw = t_f32((rng.standard_normal(Dm + r) * 0.1).astype(np.float32))
    bsz = np.arange(B * (K + 1) + 1, dtype=np.float64)
    sps = t_f32((100.0 - 0.4 * bsz).astype(np.float32))
    ws = torch.empty(D.dspark_markov_workspace_bytes(B, K, V, r, D.DSPARK_BF16, D.DSPARK_W2_VR), dtype=torch.uint8,
                     device="cuda")
    res = {}

    def run():
        t, l, c, s = D.dspark_markov_draft_confidence(U, W1, W2T, anc, h, cw, w2_layout=D.DSPARK_W2_VR, workspace=ws)
        ln, th = D.dspark_schedule_prefixes(s, sps)
        res.update(t=t, c=c, s=s, ln=ln)

    run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in res.items()}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        for v in res.values():
            v.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(res[k], ref[k]), (i, k)
