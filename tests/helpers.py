"""Shared helpers of the GPU parity tests: host <-> device marshalling and the comparison rules.

Comparison rules (tolerances of the draft-calibration path):
  * calibrated logits, pair scores and log-probabilities: |gpu - oracle| <= 1e-2 (tighter where stated);
  * tokens: the oracle follows the GPU's own path (teacher forcing), so every position is compared under the
    same prefix.  A GPU token equals the oracle's pick, or differs only where a perturbation of at most 1e-2 of
    every key (greedy: logits; sampling: log-masses l / T) selects it (the oracle's ``reach``); such positions
    have an oracle margin below 2e-2.  Differing tokens are counted and stay under a ceiling;
  * top-k candidate lists: identical ids in identical order.
"""
import numpy as np
import torch

LOGIT_TOL = 1e-2
MARGIN_TOL = 2e-2
MISMATCH_CEIL = 0.02  # at most this fraction of positions (and at least 2) may differ, each reachable


def dev():
    return torch.device("cuda:0")


def t_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def t_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def t_w(a):
    """Stored weights: float32 stays float32, uint16 bf16 bits become torch.bfloat16."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32)).to(dev())


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def check_draft(gpu_tok, gpu_lp, ref, *, lp_tol=LOGIT_TOL, mismatch_ceil=MISMATCH_CEIL, what=""):
    """ref: oracle output run with follow=gpu_tok (it carries ``reach`` and ``lp_follow``).
    Returns (n_flagged, n_mismatched) and prints them."""
    assert "reach" in ref, "the oracle must follow the GPU's path"
    agree = gpu_tok == ref["tokens"]
    reach = ref["reach"] == 1
    bad = ~agree & ~reach
    assert not bad.any(), (f"{what}: GPU token not reachable from the oracle's logits at "
                           f"{np.argwhere(bad)[:8].tolist()} (gpu {gpu_tok[bad][:8].tolist()}, "
                           f"oracle {ref['tokens'][bad][:8].tolist()}, margin {ref['margins'][bad][:8].tolist()})")
    flagged = ref["margins"] < MARGIN_TOL
    n_mis = int((~agree).sum())
    assert n_mis <= max(2, mismatch_ceil * agree.size), f"{what}: {n_mis} of {agree.size} tokens differ"
    if gpu_lp is not None:
        lp_ref = np.where(agree, ref["logprobs"], ref["lp_follow"])
        ok = ~np.isnan(lp_ref)
        assert ok.all(), f"{what}: a GPU token outside the oracle's set"
        err = np.abs(gpu_lp[ok] - lp_ref[ok]).max() if ok.any() else 0.0
        assert err <= lp_tol, f"{what}: log-probability error {err}"
    print(f"[parity] {what}: {agree.size} positions, {int(flagged.sum())} flagged (margin < {MARGIN_TOL}), "
          f"{n_mis} differ (all reachable)")
    return int(flagged.sum()), n_mis
