"""GPU checks of the calibration kernels the roofline's achievable peaks come from: the copy is
exact, and the MFMA loop did all of its work (every thread's sum is 8 * 32 * iters)."""
import pytest
import torch

from hierarchical_top_sparse_amd import _abi

pytestmark = pytest.mark.gpu


def test_calib_copy_exact():
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (3 * 2 ** 20 + 4,), dtype=torch.int32,
                        device="cuda")
    dst = torch.zeros_like(src)
    _abi.llsa_calib_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 100), (1024, 64)])
def test_calib_mfma_counts(blocks, iters):
    out = torch.zeros(blocks * 256, device="cuda")
    _abi.llsa_calib_mfma(out, blocks, iters)
    torch.cuda.synchronize()
    assert torch.all(out == 8 * 32 * iters)
