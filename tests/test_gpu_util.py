"""GPU checks of the measurement utility dspark_stream_read: it reads its buffers and writes nothing else."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def D():
    import rank_markov_draft_amd as D
    return D


@pytest.mark.parametrize("na,nb", [(0, 4), (4, 0), (1 << 10, 3 << 8), (5 << 20, 7 << 20)])
def test_stream_read_leaves_buffers_and_sink(D, na, nb):
    import torch

    dev = torch.device("cuda:0")
    a = torch.arange(na * 4, dtype=torch.int32, device=dev)  # na 16-byte units
    b = torch.full((nb * 4,), 7, dtype=torch.int32, device=dev)
    a0, b0 = a.clone(), b.clone()
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    D.dspark_stream_read(a, b, sink)
    torch.cuda.synchronize()
    assert torch.equal(a, a0) and torch.equal(b, b0)
    assert int(sink.item()) in (0, 0x9E3779B9 - (1 << 32))
