"""GPU tests of code paths the shape-driven kernel choices reach only at particular sizes: routing over
more than 256 experts, grouped items on the pair tile for every lane-part count, and the wide pair tiles for
Q4_0 at 9-16 rows."""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, oracle_image, outliers, rel_err

pytestmark = pytest.mark.gpu

FMTS = [(q.Q8_0, O.Q8_0), (q.Q4_0, O.Q4_0)]


@pytest.mark.parametrize("E", [8, 64, 256, 300, 1000])
def test_routing_matches_oracle(E):
    """Top-k experts (ties to the lower index) and softmax weights of qg_moe_route against the oracle, for
    expert counts that take each logits-per-lane width (4, 8, 16)."""
    rows = 16
    rng = np.random.default_rng(E)
    logits = gauss((rows, E), 1.0, 22, E).numpy()
    # exact ties, some of them among the top picks
    for r in range(rows):
        a, b = rng.choice(E, size=2, replace=False)
        logits[r, b] = logits[r, a]
        logits[r, (a + 1) % E] = logits[r].max()
    # and logits on a coarse grid: many experts share each value, so most picks break a tie
    coarse = (np.round(logits * 2.0) / 2.0).astype(np.float32)
    for lg, kind in ((logits, "gauss"), (coarse, "coarse")):
        for topk in sorted({1, min(8, E), min(32, E)}):
            log(f"routing E={E} topk={topk} logits={kind}")
            ex, _, wt = q.moe_route(torch.from_numpy(lg).cuda(), topk)
            ex_o, p_o = O.route_topk(lg, topk)
            assert np.array_equal(ex.cpu().numpy().reshape(rows, topk), ex_o)
            assert np.allclose(wt.cpu().numpy().reshape(rows, topk), p_o, rtol=1e-5, atol=1e-9)


def test_routing_of_nan_logits():
    """A NaN logit ranks as -inf with its own index: a row of NaN picks experts 0..topk-1 (what the oracle's
    strict comparison picks for it too), a row with some NaN picks the largest finite logits, NaN and -inf
    tie by index, and every expert id is in range; the weights of a row with a NaN are NaN (its softmax sum
    is)."""
    E, topk = 256, 8
    rng = np.random.default_rng(5)
    lg = rng.permutation(E).astype(np.float32)[None, :].repeat(4, 0)  # distinct finite values
    lg[0, :] = np.nan
    nan_at = rng.choice(E, size=100, replace=False)
    lg[1, nan_at] = np.nan
    lg[2, :] = -np.inf
    lg[2, ::3] = np.nan  # only -inf and NaN: ties by index
    lg[3, :] = np.nan
    lg[3, 200:205] = np.arange(5, dtype=np.float32)  # five finite, then the NaN / -inf tail by index
    log("routing of NaN logits")
    ex, _, wt = q.moe_route(torch.from_numpy(lg).cuda(), topk)
    ex = ex.cpu().numpy().reshape(4, topk)
    wt = wt.cpu().numpy().reshape(4, topk)
    assert np.array_equal(ex[0], np.arange(topk))
    ex_o, _ = O.route_topk(lg[:1], topk)
    assert np.array_equal(ex[0], ex_o[0])
    fin = np.where(np.isnan(lg[1]), -np.inf, lg[1])
    assert np.array_equal(ex[1], np.argsort(-fin, kind="stable")[:topk])
    assert np.array_equal(ex[2], np.arange(topk))
    assert np.array_equal(ex[3], np.array([204, 203, 202, 201, 200, 0, 1, 2]))
    assert np.all((ex >= 0) & (ex < E))
    assert np.all(np.isnan(wt[[0, 1, 3]]))


@pytest.mark.parametrize("k", [512, 2048, 3072, 4096, 8192])
def test_grouped_items_on_every_tile_shape(k):
    """Work items of 16, 9, 5, 3 and 1-2 rows (the pair tile with two row groups, with one, and the lean
    small-item tile) for k whose partition has 1, 2, 4 or 8 lane parts (k = 3072: twelve blocks per part):
    every assignment's row equals the same row through the one-row GEMV, bit for bit."""
    E, n, x_rows = 5, 80, 20
    blocks, imgs = [], []
    for e in range(E):
        b, img = oracle_image(O.Q8_0, gauss((n, k), 0.02, 23, 100 * e + k % 97).numpy())
        blocks.append(b)
        imgs.append(img)
    stacked = torch.cat(imgs)
    x = gauss((x_rows, k), 1.0, 23, 7).numpy()
    xd = torch.from_numpy(x).cuda()
    rng = np.random.default_rng(k)
    counts = [16, 9, 5, 3, 2]  # expert e gets counts[e] assignments
    expert = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    perm = rng.permutation(expert.size)
    expert = expert[perm]
    x_index = rng.integers(0, x_rows, size=expert.size).astype(np.int32)
    m = expert.size
    log(f"grouped k={k} m={m}")
    y = torch.full((m, n), float("nan"), device="cuda")
    q.qgemv_q8_0_grouped(stacked, E, n, k, xd, torch.from_numpy(expert).cuda(), torch.from_numpy(x_index).cuda(),
                         y=y)
    yg = y.cpu().numpy()
    for j in range(m):
        dense = q.qgemv_q8_0(imgs[expert[j]], n, k, xd[x_index[j]:x_index[j] + 1].contiguous())
        assert np.array_equal(bits(y[j]), bits(dense[0])), (j, expert[j])
    # and the oracle, on a few assignments
    for j in (0, m // 2, m - 1):
        xr = x[x_index[j]:x_index[j] + 1]
        yo = O.gemv_q(O.Q8_0, blocks[expert[j]], n, k, xr)
        assert rel_err(yg[j:j + 1], yo, blocks[expert[j]], O.Q8_0, xr) <= TOL


def test_q4_0_wide_tiles_at_16_rows():
    """Q4_0 at 16 rows on a matrix whose narrow tiling needs two rounds of resident workgroups (so the launch
    takes the wide tiles): sampled outputs against the oracle, and rows 0 and 15 against the same rows
    alone."""
    n, k, rows = 16384, 4096, 16
    w = gauss((n, k), 0.02, 24, 0).numpy()
    blocks, img = oracle_image(O.Q4_0, w)
    x = gauss((rows, k), 1.0, 24, 1).numpy()
    xd = torch.from_numpy(x).cuda()
    y = q.qgemv_q4_0(img, n, k, xd)
    sel = np.sort(np.random.default_rng(24).choice(n, size=256, replace=False))
    yo = O.gemv_q_rows(O.Q4_0, blocks, n, k, x, sel, threads=16)
    e = rel_err(y.cpu().numpy()[:, sel], yo, blocks, O.Q4_0, x, sel=sel)
    log(f"Q4_0 {n}x{k} rows={rows} max rel err {e:.3e}")
    assert e <= TOL
    for r in (0, rows - 1):
        y1 = q.qgemv_q4_0(img, n, k, xd[r:r + 1].contiguous())
        assert np.array_equal(bits(y[r]), bits(y1[0]))


@pytest.mark.parametrize("rows", [5, 9])
def test_q8_0_pair_tiles_over_rounds_with_ragged_edges(rows):
    """Q8_0 pair tiles over several rounds of workgroups (the launch that carries each workgroup's next tile's
    loads across its combine) on a matrix with a ragged last tile group (n = 40007: 626 tiles of 64 or 32
    rows, two rounds) and padded blocks (k = 1056, 33 blocks; one lane part per wave part): sampled outputs,
    the last rows among them, against the oracle, and rows 0 and R-1 against the same rows alone."""
    n, k = 40007, 1056
    w = gauss((n, k), 0.02, 31, rows).numpy()
    blocks, img = oracle_image(O.Q8_0, w)
    x = outliers((rows, k), 1.0, 31, 100 + rows).numpy()
    xd = torch.from_numpy(x).cuda()
    y = q.qgemv_q8_0(img, n, k, xd)
    sel = np.unique(np.concatenate([np.arange(n - 40, n), np.random.default_rng(rows).choice(n, 200, replace=False)]))
    yo = O.gemv_q_rows(O.Q8_0, blocks, n, k, x, sel, threads=8)
    e = rel_err(y.cpu().numpy()[:, sel], yo, blocks, O.Q8_0, x, sel=sel)
    log(f"Q8_0 {n}x{k} rows={rows} max rel err {e:.3e}")
    assert e <= TOL
    for r in (0, rows - 1):
        y1 = q.qgemv_q8_0(img, n, k, xd[r:r + 1].contiguous())
        assert np.array_equal(bits(y[r]), bits(y1[0]))


def test_device_probe_on_the_gpu():
    """The capability probe finds the library's marker on the gfx950 it runs on, answers false for device
    numbers that do not exist, and leaves the current device as it was."""
    dev = torch.cuda.current_device()
    assert q.device_supported(dev)
    assert not q.device_supported(-1) and not q.device_supported(torch.cuda.device_count())
    assert torch.cuda.current_device() == dev


@pytest.mark.parametrize("fmt,n,k,rows", [("q8_0", 20007, 4096, 5), ("q4_0", 40007, 2048, 8), ("q4_0", 20007, 4096, 3)])
def test_wide_tiles_of_three_at_3_to_8_rows(fmt, n, k, rows):
    """One projection whose narrow pair tiles (32 or 64 rows) overflow the workgroups resident at once on 256
    CUs while its wide tiles (48 or 96 rows: three 16-row image tiles per wave) fit: the launch widens it, with
    a ragged last tile. Sampled outputs, the last rows among them, against the oracle, and rows 0 and R-1
    against the same rows alone."""
    F = O.Q8_0 if fmt == "q8_0" else O.Q4_0
    w = gauss((n, k), 0.02, 34, rows).numpy()
    blocks, img = oracle_image(F, w)
    x = outliers((rows, k), 1.0, 34, 100 + rows).numpy()
    xd = torch.from_numpy(x).cuda()
    call = q.qgemv_q8_0 if fmt == "q8_0" else q.qgemv_q4_0
    y = call(img, n, k, xd)
    sel = np.unique(np.concatenate([np.arange(n - 60, n), np.random.default_rng(n).choice(n, 200, replace=False)]))
    yo = O.gemv_q_rows(F, blocks, n, k, x, sel, threads=8)
    e = rel_err(y.cpu().numpy()[:, sel], yo, blocks, F, x, sel=sel)
    log(f"{fmt} {n}x{k} rows={rows} max rel err {e:.3e}")
    assert e <= TOL
    for r in (0, rows - 1):
        y1 = call(img, n, k, xd[r:r + 1].contiguous())
        assert np.array_equal(bits(y[r]), bits(y1[0]))


@pytest.mark.parametrize("fmt,ofmt", FMTS + [(q.Q4_K, O.Q4_K)])
@pytest.mark.parametrize("k", [40960, 73728])
def test_long_rows_at_one_and_two_rows(fmt, ofmt, k):
    """Rows too long for the GEMV launch's staging area (k = 73728: one row of Q8_0 blocks is 82944 bytes; k =
    40960 at two rows) are quantized by a launch of their own into the workspace first; outputs match the
    oracle and a row of a two-row call has its bits alone."""
    n = 100
    w = gauss((n, k), 0.02, 17, 1).numpy()
    blocks = O.quantize_weights(ofmt, w)
    img = torch.from_numpy(q.pack_image(fmt, blocks, n, k)).cuda()
    fn = {q.Q8_0: q.qgemv_q8_0, q.Q4_0: q.qgemv_q4_0, q.Q4_K: q.qgemv_q4_k}[fmt]
    x = gauss((2, k), 1.0, 17, 2).numpy()
    xd = torch.from_numpy(x).cuda()
    ws = torch.full((q.workspace_bytes(2, k),), 0x7F, dtype=torch.uint8, device="cuda")  # not zero: must be written
    y2 = fn(img, n, k, xd, ws=ws)
    y1 = fn(img, n, k, xd[1:2].contiguous(), ws=ws)
    yo = O.gemv_q(ofmt, blocks, n, k, x, threads=8)
    assert rel_err(y2.cpu().numpy(), yo, blocks, ofmt, x) <= TOL
    assert np.array_equal(bits(y1[0]), bits(y2[1]))
