"""GPU parity of the fused residual add + RMS norm + A1 step (qg_add_rmsnorm_prepare): h bit for bit against
the fp32 add, y against the double-precision oracle, and the workspace bytes equal to qg_prepare_rows of the
kernel's own y (the quantization in the order and rounding of the separate launch it replaces)."""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import bits, gauss, log

pytestmark = pytest.mark.gpu

EPS = 1e-5


def _ws(rows, k):
    # plane padding is written by neither side: compare workspaces that start with the same bytes
    return q.empty_ws(rows, k).fill_(0xA5)


def _inputs(rows, k, seed):
    x = gauss((rows, k), 1.0, 25, seed).numpy()
    res = gauss((rows, k), 0.5, 25, seed + 1).numpy()
    gamma = (1.0 + gauss((k,), 0.1, 25, seed + 2).numpy()).astype(np.float32)
    return x, res, gamma


@pytest.mark.parametrize("rows,k", [(1, 2048), (2, 8192), (3, 96), (8, 2048), (9, 3072), (16, 8192), (100, 512)])
def test_add_rmsnorm_prepare_parity(rows, k):
    log(f"add_rmsnorm_prepare rows={rows} k={k}")
    x, res, gamma = _inputs(rows, k, 3 * k + rows)
    xd, rd, gd = (torch.from_numpy(a).cuda() for a in (x, res, gamma))
    h = torch.empty_like(xd)
    y = torch.empty_like(xd)
    ws = _ws(rows, k)
    q.add_rmsnorm_prepare(xd, gd, EPS, residual=rd, ws=ws, h_out=h, y_out=y)
    ho, yo = O.add_rmsnorm(x, res, gamma, EPS)
    assert np.array_equal(bits(h), bits(ho))
    yg = y.cpu().numpy().astype(np.float64)
    err = np.abs(yg - yo) / np.maximum(np.abs(yo), 1e-30)
    log(f"  max rel err of y {err.max():.3e}")
    assert err.max() <= 2e-6
    assert torch.equal(ws, q.prepare_rows(y, _ws(rows, k)))


def test_add_rmsnorm_prepare_without_residual_and_in_place():
    rows, k = 5, 4096
    x, res, gamma = _inputs(rows, k, 77)
    gd = torch.from_numpy(gamma).cuda()
    # no residual: h = x
    xd = torch.from_numpy(x).cuda()
    ws, _, _ = q.add_rmsnorm_prepare(xd, gd, EPS, ws=_ws(rows, k))
    _, yo = O.add_rmsnorm(x, None, gamma, EPS)
    y = torch.empty_like(xd)
    q.add_rmsnorm_prepare(xd, gd, EPS, y_out=y)
    assert np.abs(y.cpu().numpy() - yo).max() <= 2e-6 * np.abs(yo).max()
    assert torch.equal(ws, q.prepare_rows(y, _ws(rows, k)))
    # in place: the new residual stream overwrites the old one, y overwrites x
    xd2, rd2 = torch.from_numpy(x).cuda(), torch.from_numpy(res).cuda()
    h_ref = torch.empty_like(xd2)
    y_ref = torch.empty_like(xd2)
    ws_ref, _, _ = q.add_rmsnorm_prepare(xd2.clone(), gd, EPS, residual=rd2.clone(), h_out=h_ref, y_out=y_ref,
                                         ws=_ws(rows, k))
    ws2 = _ws(rows, k)
    q.add_rmsnorm_prepare(xd2, gd, EPS, residual=rd2, h_out=rd2, y_out=xd2, ws=ws2)
    assert torch.equal(rd2, h_ref) and torch.equal(xd2, y_ref) and torch.equal(ws2, ws_ref)


def test_add_rmsnorm_prepare_feeds_the_set_gemv():
    """A layer's attention input through the fused step and the prepared-rows set GEMV equals the separate
    norm output quantized by the set call's own quantization."""
    rows, k = 8, 2048
    x, res, gamma = _inputs(rows, k, 91)
    xd, rd, gd = (torch.from_numpy(a).cuda() for a in (x, res, gamma))
    ws, _, _ = q.add_rmsnorm_prepare(xd, gd, EPS, residual=rd)
    y = torch.empty_like(xd)
    q.add_rmsnorm_prepare(xd, gd, EPS, residual=rd, y_out=y)
    n = 1024
    w = gauss((n, k), 0.02, 25, 5, device="cuda")
    img = q.quantize_weights(q.Q8_0, w)
    out_fused = torch.empty((rows, n), device="cuda")
    q.qgemv_set(q.Q8_0, [(img, n, k, ws, out_fused)], rows)
    out_sep = q.qgemv_q8_0(img, n, k, y)
    assert np.array_equal(bits(out_fused), bits(out_sep))
