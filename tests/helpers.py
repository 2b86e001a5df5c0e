"""Shared helpers of the GPU parity tests: host <-> device marshalling and the comparison rules.

Comparison rules (tolerances of the draft-calibration path):
  * calibrated logits, pair scores and log-probabilities: |gpu - oracle| <= 1e-2;
  * tokens: equal to the oracle's pick at every position whose oracle top-2 key margin is >= 2e-2;
    positions with a smaller margin are flagged, and there either token is accepted (the oracle follows
    the GPU's own path, so every later position is still compared under the same prefix);
  * top-k candidate lists: identical ids in identical order.
"""
import numpy as np
import torch

LOGIT_TOL = 1e-2
MARGIN_TOL = 2e-2


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


def check_draft(gpu_tok, gpu_lp, ref, *, lp_tol=LOGIT_TOL, margin_tol=MARGIN_TOL, what=""):
    """ref: oracle output run with follow=gpu_tok.  Returns (n_flagged, n_mismatched_flagged)."""
    agree = gpu_tok == ref["tokens"]
    flagged = ref["margins"] < margin_tol
    bad = ~agree & ~flagged
    assert not bad.any(), f"{what}: unflagged token mismatch at {np.argwhere(bad)[:8].tolist()}"
    if gpu_lp is not None:
        lp_ref = np.where(agree, ref["logprobs"], ref["lp_follow"])
        ok = ~np.isnan(lp_ref)
        err = np.abs(gpu_lp[ok] - lp_ref[ok]).max() if ok.any() else 0.0
        assert err <= lp_tol, f"{what}: log-probability error {err}"
    return int(flagged.sum()), int((~agree).sum())
