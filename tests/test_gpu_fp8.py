"""GPU parity of the FP8 lane (block-FP8 weights, 1 x 128 FP8 activation groups): the device weight image
and activation groups bit for bit against the oracle, the GEMV within the error bar against the oracle's exact
group sums, and rows of a batch equal to the same rows alone."""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, outliers

pytestmark = pytest.mark.gpu

ROWS = [1, 2, 3, 5, 8, 9, 12, 16]


def _dequant_w(codes, scales, n):
    return O.e4m3_decode(codes) * np.repeat(np.repeat(scales.astype(np.float64), 128, 0)[:n], 128, 1)


def _dequant_x(xc, xs):
    return O.e4m3_decode(xc) * np.repeat(xs.astype(np.float64), 128, 1)


def _err(y, yo, wd, xd):
    """max |y - yo| / sum_k |w||x| over the outputs (dequantized operands)."""
    denom = np.abs(xd) @ np.abs(wd).T
    return float((np.abs(y.astype(np.float64) - yo) / np.where(denom > 0, denom, 1.0)).max())


@pytest.mark.parametrize("n,k", [(1, 128), (200, 384), (1000, 2048)])
def test_fp8_weight_image_bit_exact(n, k):
    w = outliers((n, k), 0.02, 26, n + k).numpy()
    w[:, :128] *= 1e-4  # small blocks: subnormal codes
    codes, scales = O.quantize_fp8_weights(w)
    img = q.quantize_weights(q.FP8, torch.from_numpy(w).cuda())
    assert np.array_equal(img.cpu().numpy(), q.pack_fp8(codes, scales))


@pytest.mark.parametrize("rows,k", [(1, 128), (5, 384), (16, 4096), (100, 512)])
def test_fp8_activation_groups_bit_exact(rows, k):
    x = outliers((rows, k), 1.0, 27, rows + k).numpy()
    x[0, :128] *= 1e-6
    if k >= 256:
        x[:, 128:256] = 0.0  # all-zero groups
    xc, xs = O.quantize_fp8_acts(x)
    ws = q.prepare_fp8(torch.from_numpy(x).cuda())
    wsn = ws.cpu().numpy()
    assert np.array_equal(wsn[:rows * k].reshape(rows, k), xc)
    off = -(-rows * k // 256) * 256
    assert np.array_equal(wsn[off:off + rows * (k // 128) * 4].view(np.float32).reshape(rows, k // 128), xs)


@pytest.mark.parametrize("n,k", [(1000, 1024), (33, 128), (257, 4096)])
def test_fp8_gemv_parity(n, k):
    w = gauss((n, k), 0.02, 28, n).numpy()
    codes, scales = O.quantize_fp8_weights(w)
    img = torch.from_numpy(q.pack_fp8(codes, scales)).cuda()
    wd = _dequant_w(codes, scales, n)
    worst = 0.0
    for rows in ROWS:
        x = outliers((rows, k), 1.0, 28, 32 + rows).numpy()
        y = q.qgemv_fp8(img, n, k, torch.from_numpy(x).cuda()).cpu().numpy()
        yo = O.gemv_fp8(codes, scales, x, threads=8)
        xc, xs = O.quantize_fp8_acts(x)
        e = _err(y, yo, wd, _dequant_x(xc, xs))
        worst = max(worst, e)
        assert e <= TOL, (rows, e)
    log(f"fp8 {n}x{k}: worst error {worst:.3e} of sum|w||x|")
    # the bar is TOL; the rest is fp32 rounding of 128-product group sums and of the scaled accumulation
    assert worst < 5e-5


@pytest.mark.parametrize("n", [500, 9000])  # 9000: wider tiles above 8 rows
def test_fp8_rows_in_a_batch_equal_rows_alone(n):
    k = 2048
    codes, scales = O.quantize_fp8_weights(gauss((n, k), 0.02, 29, 0).numpy())
    img = torch.from_numpy(q.pack_fp8(codes, scales)).cuda()
    x = torch.from_numpy(gauss((16, k), 1.0, 29, 1).numpy()).cuda()
    y16 = q.qgemv_fp8(img, n, k, x)
    for r in range(16):
        assert np.array_equal(bits(y16[r]), bits(q.qgemv_fp8(img, n, k, x[r:r + 1].contiguous())[0]))


def test_fp8_lm_head_sampled():
    """128256 x 4096 (the wide tiles of the large-n launch) on three whole 128-row blocks, whose codes and
    scales the oracle computes from the same fp32 weights: image bytes, and outputs at 1, 8 and 16 rows."""
    n, k = 128256, 4096
    log("fp8 LM head: weights")
    w = gauss((n, k), 0.02, 30, 0, device="cuda")
    img = q.quantize_weights(q.FP8, w)
    blocks = [0, 517, n // 128 - 1]
    sel = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    w_sel = w[torch.from_numpy(sel).cuda()].cpu().numpy()
    del w
    codes, scales = [], []
    for j in range(len(blocks)):
        c, s_ = O.quantize_fp8_weights(w_sel[128 * j:128 * j + 128])
        codes.append(c)
        scales.append(s_)
    codes, scales = np.concatenate(codes), np.concatenate(scales)
    dev_codes, dev_scales = q.unpack_fp8(img.cpu().numpy(), n, k)
    assert np.array_equal(dev_codes[sel], codes) and np.array_equal(dev_scales[blocks], scales)
    wd = _dequant_w(codes, scales, len(sel))
    for rows in (1, 8, 16):
        x = gauss((rows, k), 1.0, 30, 32 + rows).numpy()
        xd = torch.from_numpy(x).cuda()
        yd = q.qgemv_fp8(img, n, k, xd)
        y = yd.cpu().numpy()[:, sel]
        yo = O.gemv_fp8(codes, scales, x, threads=8)
        xc, xs = O.quantize_fp8_acts(x)
        e = _err(y, yo, wd, _dequant_x(xc, xs))
        log(f"  rows={rows} max error {e:.3e}")
        assert e <= TOL
        # above 8 rows the launch takes wider tiles: the sums, and so the bits, stay those of a row alone
        for r in (0, rows - 1):
            assert torch.equal(yd[r], q.qgemv_fp8(img, n, k, xd[r:r + 1].contiguous())[0])


@pytest.mark.parametrize("n,k", [(80, 512), (4096, 256), (65536, 128)])  # 8, 4 and 2 wave ranges of k
def test_fp8_grouped_equals_dense_and_oracle(n, k):
    """qgemv_fp8_grouped: each assignment has the bits of the one-row dense FP8 call on its row (items of 16, 2,
    9, 5 and 1 assignments, an expert with 18 split over two items), a few assignments against the oracle, and
    out-of-range entries skipped (their rows untouched) and counted."""
    E, x_rows = 4, 20
    codes, scales, imgs = [], [], []
    for e in range(E):
        c, s_ = O.quantize_fp8_weights(gauss((n, k), 0.02, 32, 10 * e + n % 7).numpy())
        codes.append(c)
        scales.append(s_)
        imgs.append(torch.from_numpy(q.pack_fp8(c, s_)).cuda())
    stacked = torch.cat(imgs)
    x = outliers((x_rows, k), 1.0, 32, n).numpy()
    xd = torch.from_numpy(x).cuda()
    rng = np.random.default_rng(n)
    expert = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate([18, 9, 5, 1])])
    x_index = rng.integers(0, x_rows, size=expert.size).astype(np.int32)
    perm = rng.permutation(expert.size)
    expert, x_index = expert[perm], x_index[perm]
    expert = np.concatenate([expert, [-1, 2]]).astype(np.int32)  # then two bad entries
    x_index = np.concatenate([x_index, [0, x_rows]]).astype(np.int32)
    m = expert.size
    log(f"fp8 grouped n={n} k={k} m={m}")
    y = torch.full((m, n), float("nan"), device="cuda")
    _, ws = q.qgemv_fp8_grouped(stacked, E, n, k, xd, torch.from_numpy(expert).cuda(), torch.from_numpy(x_index).cuda(),
                                y=y)
    assert q.grouped_status(ws) == 2
    yg = y.cpu().numpy()
    assert np.all(np.isnan(yg[m - 2:]))
    for j in range(m - 2):
        dense = q.qgemv_fp8(imgs[expert[j]], n, k, xd[x_index[j]:x_index[j] + 1].contiguous())
        assert np.array_equal(bits(y[j]), bits(dense[0])), (j, expert[j])
    for j in (0, (m - 2) // 2, m - 3):
        e = expert[j]
        xr = x[x_index[j]:x_index[j] + 1]
        yo = O.gemv_fp8(codes[e], scales[e], xr, threads=8)
        xc, xs = O.quantize_fp8_acts(xr)
        err = _err(yg[j:j + 1], yo, _dequant_w(codes[e], scales[e], n), _dequant_x(xc, xs))
        assert err <= TOL, (j, err)


def test_fp8_grouped_empty():
    n, k = 64, 256
    img = q.quantize_weights(q.FP8, gauss((n, k), 0.02, 33, 0, device="cuda"))
    x = gauss((2, k), 1.0, 33, 1, device="cuda")
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    y, ws = q.qgemv_fp8_grouped(img, 1, n, k, x, empty, empty)
    assert y.shape == (0, n) and q.grouped_status(ws) == 0
