"""HIP path against the CPU oracle, through the C ABI, on an MI355X.

Integer work (activation codes, weight images, block dots) must be bit-exact;
fp32 outputs must satisfy max |y_gpu - y_oracle| / sum|w_hat||x| <= 2e-3.
Shapes span several workgroup tiles with ragged row and block tails.
"""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, oracle_image, outliers, rel_err, rel_err_f16

pytestmark = pytest.mark.gpu

FMTS = [(q.Q8_0, O.Q8_0), (q.Q4_0, O.Q4_0)]
ROWS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 15, 16]


def _special_blocks(x):
    """Overwrite a few 32-blocks with ties, zeros and subnormal-scale blocks."""
    x = x.copy()
    k = x.shape[1]
    if k >= 96:
        x[0, 0:32] = np.float32([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.5] + [0.25] * 24)
        x[0, 32:64] = 0.0
        x[-1, 64:96] = (np.arange(32, dtype=np.float32) - 7) * np.float32(2.0 ** -149)
    return x


# ---------------------------------------------------------------- A1 ---
@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (16, 2048), (16, 8192), (100, 512)])
def test_quantize_rows_bit_exact(rows, k):
    log(f"quantize_rows rows={rows} k={k}")
    x = _special_blocks(outliers((rows, k), 1.0, 10, 1).numpy())
    qx, dx, sx = q.quantize_rows_q8(torch.from_numpy(x).cuda())
    oq, od, osx = O.quantize_acts(x)
    assert np.array_equal(qx.cpu().numpy(), oq)
    assert np.array_equal(bits(dx), bits(od))
    assert np.array_equal(sx.cpu().numpy(), osx)


# ----------------------------------------------------- weight quantizer ---
@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k", [(1, 32), (37, 800), (512, 2048)])
def test_quantize_weights_bit_exact(fmt, ofmt, n, k):
    log(f"quantize_weights fmt={fmt} n={n} k={k}")
    w = outliers((n, k), 0.02, 11, 2).numpy()
    w[0, :32] = 0.0
    if k >= 64:
        w[-1, 32:64] = np.float32(np.arange(32) - 16) * np.float32(2.0 ** -4)
    img = q.quantize_weights(fmt, torch.from_numpy(w).cuda())
    ref = q.pack_image(fmt, O.quantize_weights(ofmt, w), n, k)
    assert np.array_equal(img.cpu().numpy(), ref)


# ---------------------------------------------------------------- A3 ---
@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k,rows", [(1024, 1024, 1), (77, 800, 7), (16, 8192, 16), (40, 2048, 9)])
def test_blockdots_bit_exact(fmt, ofmt, n, k, rows):
    log(f"blockdots fmt={fmt} n={n} k={k} rows={rows}")
    w = gauss((n, k), 0.02, 12, 3).numpy()
    x = _special_blocks(outliers((rows, k), 1.0, 12, 4).numpy())
    blocks, img = oracle_image(ofmt, w)
    qx, _, _ = O.quantize_acts(x)
    got = q.blockdots(fmt, img, n, k, torch.from_numpy(qx).cuda())
    assert np.array_equal(got.cpu().numpy(), O.blockdots(ofmt, blocks, n, k, qx))


@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k,rows", [(40, 96, 3), (77, 800, 8), (16, 8192, 16), (257, 2048, 9), (1024, 1024, 12)])
def test_pair_blockdots_bit_exact(fmt, ofmt, n, k, rows):
    """The 3..16-row kernel's int32 block dots (its block-pair matrix product on the pair-order workspace that
    qg_prepare_rows writes) equal the oracle's, bit for bit."""
    log(f"pair blockdots fmt={fmt} n={n} k={k} rows={rows}")
    w = gauss((n, k), 0.02, 12, 5).numpy()
    x = _special_blocks(outliers((rows, k), 1.0, 12, 6).numpy())
    blocks, img = oracle_image(ofmt, w)
    qx, _, _ = O.quantize_acts(x)
    ws = q.prepare_rows(torch.from_numpy(x).cuda())
    got = q.blockdots_pairs(fmt, img, n, k, ws, rows)
    assert np.array_equal(got.cpu().numpy(), O.blockdots(ofmt, blocks, n, k, qx))


# ------------------------------------------------------------- A2-A4 ---
@pytest.mark.parametrize("fmt,ofmt", FMTS)
@pytest.mark.parametrize("n,k", [(1024, 1024), (1000, 800), (33, 96), (257, 4096), (1, 32)])
def test_qgemv_parity(fmt, ofmt, n, k):
    w = gauss((n, k), 0.02, 13, 5).numpy()
    blocks, img = oracle_image(ofmt, w)
    fn = q.qgemv_q8_0 if fmt == q.Q8_0 else q.qgemv_q4_0
    worst = 0.0
    for rows in ROWS:
        log(f"qgemv fmt={fmt} n={n} k={k} rows={rows}")
        x = _special_blocks(outliers((rows, k), 1.0, 13, 32 + rows).numpy())
        y = fn(img, n, k, torch.from_numpy(x).cuda()).cpu().numpy()
        yo = O.gemv_q(ofmt, blocks, n, k, x, threads=8)
        e = rel_err(y, yo, blocks, ofmt, x)
        worst = max(worst, e)
        assert e <= TOL, (rows, e)
    log(f"  worst relative error {worst:.3e}")
    assert worst < 1e-5  # only the fp32 summation order differs from the oracle


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_rows_in_a_batch_equal_rows_alone(fmt, ofmt):
    """Tails of 9 and 16 rows hold the same bits as each row computed by itself."""
    n, k = 600, 3072
    w = gauss((n, k), 0.02, 14, 6).numpy()
    _, img = oracle_image(ofmt, w)
    fn = q.qgemv_q8_0 if fmt == q.Q8_0 else q.qgemv_q4_0
    x = torch.from_numpy(gauss((16, k), 1.0, 14, 7).numpy()).cuda()
    alone = [fn(img, n, k, x[r:r + 1].contiguous()) for r in range(16)]
    for rows in (2, 8, 9, 16):
        y = fn(img, n, k, x[:rows].contiguous())
        for r in range(rows):
            assert np.array_equal(bits(y[r]), bits(alone[r][0])), (rows, r)


@pytest.mark.parametrize("fmt,ofmt", FMTS)
def test_guard_rows_and_offsets(fmt, ofmt):
    """Outputs outside the written rows stay NaN; inputs at nonzero offsets inside larger buffers."""
    n, k, rows = 300, 1536, 9
    w = gauss((n, k), 0.02, 15, 8).numpy()
    blocks, img = oracle_image(ofmt, w)
    big_img = torch.zeros(img.numel() + 4096, dtype=torch.uint8, device="cuda")
    big_img[1024:1024 + img.numel()] = img
    img_view = big_img[1024:1024 + img.numel()]
    x = gauss((rows, k), 1.0, 15, 9).numpy()
    xbuf = torch.full((rows * k + 64,), float("nan"), device="cuda")
    xbuf[16:16 + rows * k] = torch.from_numpy(x).cuda().reshape(-1)
    xs = xbuf[16:16 + rows * k].view(rows, k)  # 64 bytes into its buffer
    ybuf = torch.full(((rows + 4) * n,), float("nan"), device="cuda")
    y_view = ybuf[2 * n:(2 + rows) * n].view(rows, n)
    wsb = torch.zeros(q.workspace_bytes(rows, k) + 512, dtype=torch.uint8, device="cuda")
    ws_view = wsb[256:]
    fn = q.qgemv_q8_0 if fmt == q.Q8_0 else q.qgemv_q4_0
    fn(img_view, n, k, xs, y=y_view, ws=ws_view)
    yb = ybuf.cpu().numpy()
    assert np.all(np.isnan(yb[:2 * n])) and np.all(np.isnan(yb[(2 + rows) * n:]))
    yo = O.gemv_q(ofmt, blocks, n, k, x, threads=8)
    assert rel_err(y_view.cpu().numpy(), yo, blocks, ofmt, x) <= TOL


def test_set_launch_equals_single_calls():
    layer = [(2048, 1024), (512, 1024), (512, 1024), (4096, 1024), (1024, 4096)]
    for fmt, ofmt in FMTS:
        for rows in (1, 5, 16):
            log(f"set fmt={fmt} rows={rows}")
            imgs, singles, projs = [], [], []
            xin = torch.from_numpy(gauss((rows, 1024), 1.0, 16, 10).numpy()).cuda()
            xdn = torch.from_numpy(gauss((rows, 4096), 1.0, 16, 11).numpy()).cuda()
            zeros = lambda k: torch.zeros(q.workspace_bytes(rows, k), dtype=torch.uint8, device="cuda")
            ws_in = q.prepare_rows(xin, zeros(1024))
            ws_dn = q.prepare_rows(xdn, zeros(4096))
            for i, (n, k) in enumerate(layer):
                _, img = oracle_image(ofmt, gauss((n, k), 0.02, 16, i).numpy())
                x, ws = (xin, ws_in) if k == 1024 else (xdn, ws_dn)
                imgs.append(img)
                singles.append(q.qgemv_prepared(fmt, img, n, k, ws, rows))
                y = torch.full((rows, n), float("nan"), device="cuda")
                projs.append((img, n, k, ws, y))
            q.qgemv_set(fmt, projs, rows)
            for (img, n, k, ws, y), ys in zip(projs, singles):
                assert np.array_equal(bits(y), bits(ys))
            # the set prepare equals two single prepares
            w2a = torch.zeros_like(ws_in)
            w2b = torch.zeros_like(ws_dn)
            q.prepare_rows_set([xin, xdn], [w2a, w2b])
            assert torch.equal(w2a, ws_in) and torch.equal(w2b, ws_dn)


# ------------------------------------------------------------- f16 lane ---
@pytest.mark.parametrize("n,k", [(256, 2048), (1000, 800), (33, 104), (130, 4096), (1, 8)])
def test_f16_parity(n, k):
    w = gauss((n, k), 0.02, 17, 12).numpy()
    w16, _ = O.f32_to_f16(w)
    wd = torch.from_numpy(w16.view(np.int16)).cuda()
    img = q.f16_image(wd)
    assert np.array_equal(img.cpu().numpy(), q.pack_image(q.F16, w16, n, k)), "device F16 image"
    worst = 0.0
    for rows in ROWS:
        log(f"gemv_f16 n={n} k={k} rows={rows}")
        x = outliers((rows, k), 1.0, 17, 32 + rows).numpy()
        y = q.gemv_f16(img, n, k, torch.from_numpy(x).cuda()).cpu().numpy()
        yo = O.gemv_f16(w16, x, threads=8)
        e = rel_err_f16(y, yo, w16, x)
        worst = max(worst, e)
        assert e <= TOL
    log(f"  worst relative error {worst:.3e}")
    assert worst < 1e-5


def test_f16_rows_in_a_batch_equal_rows_alone():
    n, k = 500, 2048
    w16, _ = O.f32_to_f16(gauss((n, k), 0.02, 18, 13).numpy())
    img = q.f16_image(torch.from_numpy(w16.view(np.int16)).cuda())
    x = torch.from_numpy(gauss((16, k), 1.0, 18, 14).numpy()).cuda()
    y16 = q.gemv_f16(img, n, k, x)
    for r in range(16):
        assert np.array_equal(bits(y16[r]), bits(q.gemv_f16(img, n, k, x[r:r + 1].contiguous())[0]))


# -------------------------------------------------------------- grouped ---
def test_grouped_equals_dense_and_skips_bad_entries():
    E, n, k, x_rows = 12, 384, 1024, 6
    blocks_all, imgs = [], []
    for e in range(E):
        b, img = oracle_image(O.Q8_0, gauss((n, k), 0.02, 19, e).numpy())
        blocks_all.append(b)
        imgs.append(img)
    stacked = torch.cat(imgs)
    x = gauss((x_rows, k), 1.0, 19, 40).numpy()
    xd = torch.from_numpy(x).cuda()
    rng = np.random.default_rng(0)
    expert = rng.integers(0, E, size=60).astype(np.int32)
    x_index = rng.integers(0, x_rows, size=60).astype(np.int32)
    expert[:20] = 3  # one expert with 20 assignments: two work items
    expert[25], x_index[31], expert[40] = E, x_rows, -2
    y = torch.full((60, n), float("nan"), device="cuda")
    _, ws = q.qgemv_q8_0_grouped(stacked, E, n, k, xd, torch.from_numpy(expert).cuda(),
                                 torch.from_numpy(x_index).cuda(), y=y)
    assert q.grouped_status(ws) == 3
    yo, bad = O.gemv_q8_0_grouped(np.stack(blocks_all), E, n, k, x, expert, x_index)
    assert bad == 3
    yg = y.cpu().numpy()
    for j in range(60):
        if j in (25, 31, 40):
            assert np.all(np.isnan(yg[j]))
            continue
        dense = q.qgemv_q8_0(imgs[expert[j]], n, k, xd[x_index[j]:x_index[j] + 1].contiguous())
        assert np.array_equal(bits(y[j]), bits(dense[0]))
        assert rel_err(yg[j:j + 1], yo[j:j + 1], blocks_all[expert[j]], O.Q8_0, x[x_index[j]:x_index[j] + 1]) <= TOL


def test_grouped_empty_assignment_list():
    n, k = 64, 256
    _, img = oracle_image(O.Q8_0, gauss((n, k), 0.02, 20, 0).numpy())
    x = torch.from_numpy(gauss((2, k), 1.0, 20, 1).numpy()).cuda()
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    y, ws = q.qgemv_q8_0_grouped(img, 1, n, k, x, e, e)
    assert y.shape == (0, n) and q.grouped_status(ws) == 0


def test_set_rows_equals_single_calls():
    """The fp32-rows set launch (quantization inside it at 1-2 rows, one shared quantize launch otherwise, and
    for Q4_0 at two rows when every projection brings a workspace) gives the same bits as one call per
    projection."""
    layer = [(2048, 1024), (512, 1024), (1024, 4096), (300, 800)]
    for fmt, ofmt in FMTS:
        imgs = [oracle_image(ofmt, gauss((n, k), 0.02, 21, i).numpy())[1] for i, (n, k) in enumerate(layer)]
        for rows in (1, 2, 3, 5, 16):
            xs = {k: torch.from_numpy(gauss((rows, k), 1.0, 21, 32 + k % 97).numpy()).cuda() for _, k in layer}
            fn = q.qgemv_q8_0 if fmt == q.Q8_0 else q.qgemv_q4_0
            singles = [fn(img, n, k, xs[k]) for (n, k), img in zip(layer, imgs)]
            # workspaces: none, of this row count's size, or (two rows) of one row's size, which the set does
            # not use, quantizing inside the launch as it does without
            for with_ws in (("none", "full") + (("small",) if rows == 2 else ()) if rows <= q.FUSED_ROWS
                            else ("full",)):
                log(f"set_rows fmt={fmt} rows={rows} workspaces={with_ws}")
                wss = {k: q.empty_ws(1 if with_ws == "small" else rows, k) for _, k in layer}
                projs = []
                for (n, k), img in zip(layer, imgs):
                    y = torch.full((rows, n), float("nan"), device="cuda")
                    projs.append((img, n, k, xs[k], None if with_ws == "none" else wss[k], y))
                q.qgemv_set_rows(fmt, projs, rows)
                for p, ys in zip(projs, singles):
                    assert np.array_equal(bits(p[5]), bits(ys))
