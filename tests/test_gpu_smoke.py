"""The smoke entry point (`__graft_entry__.smoke`) on the GPU: the tiny fp32 W8A8 layer and a small
W4A4 layer on the codebook product path, each against the oracle (the function asserts its own
bounds: 1e-4 and 2e-2 relative Frobenius)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def test_smoke_entry_point_runs_and_matches_the_oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import __graft_entry__

    __graft_entry__.smoke()
