"""GPU parity of q4_quant_error (the NF4 vs uniform 4-bit quantization-error
measurement) against the oracle's quant_error, through the C ABI. The
maximum error is compared bit for bit. Both sums add nonnegative fp64 terms,
the oracle pairwise and the GPU in fixed chains of at most ~40 additions,
so they agree to ~1e-14 relative; the test allows 1e-12."""

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

RTOL = 1e-12


@pytest.fixture(scope="module")
def qn():
    import bit_nf4_quantized_16_amd as qn

    assert torch.cuda.is_available()
    return qn


def _check(qn, W, grid, dtype=torch.float32):
    Wd = W.to(dtype).contiguous()
    got = qn.q4_quant_error(Wd.cuda(), grid).cpu().numpy()
    want = oracle.quant_error(Wd.float().numpy(), oracle.GRIDS[grid])
    assert got[2] == want[2], (grid, got[2], want[2])
    for i in range(2):
        assert abs(got[i] - want[i]) <= RTOL * abs(want[i]), (grid, i, got[i], want[i])
    return got


SHAPES = [(256, 256), (1, 1), (1, 63), (1, 64), (1, 65), (3, 100), (7, 33), (513, 77), (64, 4096), (37, 511),
          (2, 257), (1, 1024 + 64 * 3 + 5)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("grid", ["nf4", "uniform"])
def test_quant_error_matches_oracle(qn, shape, dtype, grid):
    W = workloads.normal_weight(shape[0], shape[1], 0.02, seed=shape[0] * 31 + shape[1])
    _check(qn, W, grid, dtype)


@pytest.mark.parametrize("grid", ["nf4", "uniform"])
def test_heavy_tails_and_outliers(qn, grid):
    _check(qn, workloads.student_t_weight(512, 1024, 3.0, 0.02, seed=7), grid)
    _check(qn, workloads.normal_weight(512, 1024, 0.02, seed=8, outlier_frac=1e-3, outlier_scale=20.0), grid)


def test_zero_weight(qn):
    for grid in ("nf4", "uniform"):
        got = qn.q4_quant_error(torch.zeros(64, 300, device="cuda"), grid).cpu().numpy()
        assert np.all(got == 0.0)


def test_values_on_the_grid_have_no_error(qn):
    # every block holds +-1 (its absmax) and otherwise only grid values
    for grid, table in oracle.GRIDS.items():
        rng = np.random.default_rng(9)
        w = table[rng.integers(0, 16, size=(128, 256))].astype(np.float32)
        w[:, ::64] = 1.0
        got = qn.q4_quant_error(torch.tensor(w).cuda(), grid).cpu().numpy()
        assert got[0] == 0.0 and got[2] == 0.0


def test_bitwise_repeatable(qn):
    W = workloads.normal_weight(1024, 4096, 0.02, seed=10).cuda()
    a = qn.q4_quant_error(W, "uniform").cpu().numpy()
    b = qn.q4_quant_error(W, "uniform").cpu().numpy()
    assert a.tobytes() == b.tobytes()


def test_full_size_mlp_weight(qn):
    # the 7B MLP gate projection, 11008 x 4096, fp32, with outliers
    W = workloads.normal_weight(11008, 4096, 0.02, seed=2, outlier_frac=1e-3, outlier_scale=20.0)
    for grid in ("nf4", "uniform"):
        _check(qn, W, grid)
