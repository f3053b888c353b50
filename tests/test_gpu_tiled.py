"""GPU parity of the GEMV on the repacked (tiled) 4-bit layout: within the
fp32 bound of the fp64 oracle's GEMV on the source matrix, and bit for bit
equal to qmoe_gemv_affine4 on the source matrix (the same arithmetic in the
same order; only the addresses differ)."""
import numpy as np
import pytest

import oracle
import synth
import synth.device
from tests.helpers import bf16_to_f64, gemv4_bound, log, rel_l2

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch

    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def q():
    import bit_quantized_gemv_amd as q

    return q


def _dev(torch, a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


@pytest.mark.parametrize("rows,cols,rbw", [(2112, 2816, 0), (20003, 2816, 1), (13, 2816, 0),
                                           (2816, 704, 1), (2816, 704, 2), (70001, 704, 2),
                                           (9, 704, 2), (1, 704, 1)])
def test_gemv_tiled_matches_oracle_and_mlx_layout(torch_cuda, q, rows, cols, rbw):
    torch = torch_cuda
    log(f"tiled gemv rows={rows} cols={cols} row_blocks_per_wave={rbw}")
    m = synth.random_qmat(rows, cols, 4, rows * 3 + cols)
    x = synth.random_bf16(cols, 11)
    xd = bf16_to_f64(x)
    ref = oracle.qgemv(m, xd)
    t = _dev(torch, q.qmoe_repack_tiled4(m.q.view(np.uint8), m.s, m.b, rows, cols))
    xg = _dev(torch, x)
    y = torch.full((rows + 8,), float("nan"), dtype=torch.float32, device="cuda")
    q.qmoe_gemv_tiled4(t, rows, cols, xg, y, rbw)
    y0 = torch.empty(rows, dtype=torch.float32, device="cuda")
    q.qmoe_gemv_affine4(synth.device.qtensor(m), xg, y0)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.all(np.isnan(got[rows:])), "rows past the matrix are never written"
    got = got[:rows].astype(np.float64)
    bound = gemv4_bound(m, xd)
    assert np.all(np.abs(got - ref) <= bound), np.nanmax(np.abs(got - ref) / bound)
    assert rel_l2(got, ref) <= 1e-5
    assert np.array_equal(got.astype(np.float32).view(np.uint32),
                          y0.cpu().numpy().view(np.uint32))


def test_gemv_tiled_rejects_bad_arguments(torch_cuda, q):
    torch = torch_cuda
    m = synth.random_qmat(16, 2112, 4, 3)
    t = _dev(torch, q.qmoe_repack_tiled4(m.q.view(np.uint8), m.s, m.b, 16, 2112))
    x = _dev(torch, synth.random_bf16(2112, 1))
    y = torch.empty(16, dtype=torch.float32, device="cuda")
    with pytest.raises(q.QmoeError, match="UNSUPPORTED"):
        q.qmoe_gemv_tiled4(t, 16, 2112, x, y)  # not a compiled width
    with pytest.raises(q.QmoeError, match="BAD_SHAPE"):
        q.qmoe_gemv_tiled4(t, 16, 2112, x, y, 3)
    with pytest.raises(q.QmoeError, match="ALIGN"):
        m2 = synth.random_qmat(16, 704, 4, 4)
        t2 = _dev(torch, q.qmoe_repack_tiled4(m2.q.view(np.uint8), m2.s, m2.b, 16, 704))
        q.qmoe_gemv_tiled4(t2.data_ptr() + 4, 16, 704, x, y)
