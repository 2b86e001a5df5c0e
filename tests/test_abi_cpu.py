"""The C-ABI library loads and exports every declared symbol; host-side argument errors (CPU only).

These calls never reach a kernel: each one is rejected by the host-side checks before anything is
enqueued, so no GPU is needed.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")
LIB = os.path.join(ROOT, "rank_markov_draft_amd", "_lib", "libdspark.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built")
    import rank_markov_draft_amd as D
    return D.library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("dspark_markov_draft", "dspark_selector_draft", "dspark_markov_step", "dspark_markov_logits",
                 "dspark_gate", "dspark_topk", "dspark_pack_w2", "dspark_abi_version"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    import rank_markov_draft_amd as D
    assert D.dspark_abi_version() == 2
    assert lib.dspark_status_str(0) == b"DSPARK_OK"
    assert lib.dspark_status_str(3) == b"DSPARK_EWORKSPACE"
    assert lib.dspark_status_str(99) == b"DSPARK_UNKNOWN_STATUS"


def test_workspace_sizes(lib):
    import rank_markov_draft_amd as D
    assert D.dspark_markov_workspace_bytes(0, 16, 100, 16, 1, 1) == 0
    a = D.dspark_markov_workspace_bytes(128, 16, 151936, 256, D.DSPARK_BF16, D.DSPARK_W2_VR)
    b = D.dspark_markov_workspace_bytes(128, 16, 151936, 256, D.DSPARK_BF16, D.DSPARK_W2_RV)
    assert a > 0 and b >= a + 151936 * 256 * 2
    assert D.dspark_selector_workspace_bytes(128, 16, 151936, 256, 16) >= 4 * 128 * 16 * 16 + 4 * 128 * (16 + 15 * 256)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host-side checks


def _err(lib):
    return lib.dspark_last_error().decode()


def test_markov_draft_argument_errors(lib):
    f = lib.dspark_markov_draft
    base = dict(U=FAKE, W1=FAKE, W2=FAKE, wd=1, lay=1, anchor=FAKE, H=None, B=4, K=2, V=64, r=16, mode=0, seed=0,
                T=1.0, tok=FAKE, lp=None, ws=FAKE, wsb=1 << 30, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["U"], a["W1"], a["W2"], a["wd"], a["lay"], a["anchor"], a["H"], a["B"], a["K"], a["V"], a["r"],
                 a["mode"], a["seed"], a["T"], a["tok"], a["lp"], a["ws"], a["wsb"], a["st"])

    assert call(U=None) == 1
    assert call(W1=None) == 1
    assert call(tok=None) == 1
    assert call(B=0) == 1
    assert call(K=0) == 1
    assert call(V=-3) == 1
    assert call(r=0) == 1
    assert call(wd=7) == 1
    assert call(lay=5) == 1
    assert call(mode=3) == 1
    assert call(mode=1, T=0.0) == 1 and "temperature" in _err(lib)
    assert call(r=2048) == 2
    assert call(wsb=16) == 3 and "workspace" in _err(lib)
    assert call(ws=None) == 3


def test_confidence_argument_errors(lib):
    f = lib.dspark_markov_draft_confidence

    def call(h=FAKE, D=64, w=FAKE, conf=FAKE, surv=FAKE, U=FAKE):
        return f(U, FAKE, FAKE, 1, 1, FAKE, None, 4, 2, 64, 16, 0, 0, 1.0, h, D, w, FAKE, None, conf, surv, FAKE,
                 1 << 30, None)

    assert call(h=None) == 1
    assert call(w=None) == 1
    assert call(conf=None) == 1
    assert call(surv=None) == 1
    assert call(D=12) == 2 and "D % 8" in _err(lib)
    assert call(D=0) == 2
    assert call(h=ctypes.c_void_p(0x1008)) == 1  # not 16-byte aligned
    assert call(U=None) == 1  # the draft's own checks still apply


def test_schedule_argument_errors(lib):
    f = lib.dspark_schedule_prefixes
    assert f(None, FAKE, 4, 4, FAKE, None, None) == 1
    assert f(FAKE, FAKE, 0, 4, FAKE, None, None) == 1
    assert f(FAKE, FAKE, 4, 0, FAKE, None, None) == 1
    assert f(FAKE, FAKE, 128, 64, FAKE, None, None) == 2 and "4096" in _err(lib)


def test_selector_gate_topk_argument_errors(lib):
    s = lib.dspark_selector_draft
    assert s(FAKE, FAKE, FAKE, 1, FAKE, None, 2, 2, 100, 16, 0, 0, 0, 1.0, FAKE, None, None, None, FAKE, 1 << 20, None) == 1
    assert s(FAKE, FAKE, FAKE, 1, FAKE, None, 2, 2, 100, 16, 101, 0, 0, 1.0, FAKE, None, None, None, FAKE, 1 << 20, None) == 1
    assert s(FAKE, FAKE, FAKE, 1, FAKE, None, 2, 2, 8192, 16, 1025, 0, 0, 1.0, FAKE, None, None, None, FAKE, 1 << 20, None) == 2
    assert s(FAKE, FAKE, FAKE, 1, FAKE, None, 2, 2, 100, 16, 16, 0, 0, 1.0, FAKE, None, None, None, FAKE, 8, None) == 3
    g = lib.dspark_gate
    assert g(None, FAKE, 4, 256, 32, FAKE, None, 0, None) == 1
    assert g(FAKE, FAKE, 4, 100, 32, FAKE, None, 0, None) == 2
    assert g(FAKE, FAKE, 4, 256, 20, FAKE, None, 0, None) == 2
    need = lib.dspark_gate_workspace_bytes(1024, 4096, 256)
    assert g(FAKE, FAKE, 1024, 4096, 256, FAKE, FAKE, need - 16, None) == 1 and "workspace" in _err(lib)
    assert g(FAKE, FAKE, 1024, 4096, 256, FAKE, ctypes.c_void_p(0x1008), need, None) == 1 and "aligned" in _err(lib)
    t = lib.dspark_topk
    assert t(FAKE, 100, 4, 100, 0, FAKE, None, None, 0, None) == 1
    assert t(FAKE, 50, 4, 100, 4, FAKE, None, None, 0, None) == 1
    assert t(FAKE, 8192, 4, 8192, 1025, FAKE, None, None, 0, None) == 2
    p = lib.dspark_pack_w2
    assert p(None, 10, 10, 1, FAKE, None) == 1
    assert p(FAKE, 10, 10, 9, FAKE, None) == 1


def test_gate_workspace_bytes(lib):
    """The split-k gate takes 4 fp32 partial sums per output; sizes it does not take ask for none."""
    w = lib.dspark_gate_workspace_bytes
    assert w(1024, 4096, 256) == 4 * 1024 * 256 * 4
    assert w(100, 1024, 256) == 4 * 100 * 256 * 4
    assert w(64, 512, 64) == 4 * 64 * 64 * 4
    assert w(5, 256, 32) == 0        # r not a multiple of 64
    assert w(64, 256, 64) == 0       # D not a multiple of 512
    assert w(0, 4096, 256) == 0 and w(4, 100, 32) == 0


def test_stream_read_argument_errors(lib):
    f = lib.dspark_stream_read
    assert f(FAKE, 64, FAKE, 64, None, None) == 1                                  # no sink
    assert f(None, 64, FAKE, 64, FAKE, None) == 1                                  # NULL with a size
    assert f(FAKE, 60, FAKE, 64, FAKE, None) == 1 and "16" in _err(lib)           # not a multiple of 16
    assert f(ctypes.c_void_p(0x1008), 64, FAKE, 64, FAKE, None) == 1              # misaligned
