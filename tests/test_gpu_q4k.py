"""Q4_K superblocks (the K-quant one-row / N-row form: 256-weight superblocks, 6-bit sub-scales and sub-mins
under fp16 d and dmin, 4-bit codes) on the GPU against the oracle, through the C ABI: the device quantizer and
the block dots bit for bit, outputs within 2e-3 of sum|w_hat||x| at 1-16 rows, a row in a batch equal to the
row alone, and the Llama-3.2-3B-shaped decode layer at its full size."""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, outliers, rel_err

pytestmark = pytest.mark.gpu

ROWS = [1, 2, 3, 4, 5, 7, 8, 9, 12, 16]
LAYER_3B = [("wq", 3072, 3072), ("wk", 1024, 3072), ("wv", 1024, 3072), ("wo", 3072, 3072), ("gate", 8192, 3072),
            ("up", 8192, 3072), ("down", 3072, 8192)]


def _image(w_np):
    n, k = w_np.shape
    blocks = O.quantize_weights(O.Q4_K, w_np)
    return blocks, torch.from_numpy(q.pack_image(q.Q4_K, blocks, n, k)).cuda()


def _special(x):
    x = x.copy()
    if x.shape[1] >= 96:
        x[0, 0:32] = np.float32([127, 2.5, -2.5, 0.5, -0.5, 1.5, -1.5, 3.5] + [0.25] * 24)
        x[0, 32:64] = 0.0
        x[-1, 64:96] = (np.arange(32, dtype=np.float32) - 7) * np.float32(2.0 ** -149)
    return x


@pytest.mark.parametrize("n,k", [(1, 256), (37, 768), (512, 2048), (100, 4096)])
def test_q4_k_device_quantizer_bit_exact(n, k):
    log(f"q4_k quantize n={n} k={k}")
    w = outliers((n, k), 0.02, 21, 1).numpy()
    w[0, :256] = 0.0  # an all-zero superblock
    if n > 2:
        w[1, :256] = np.abs(w[1, :256]) + 0.01  # all positive: sub-mins 0
        w[2, 256:512] = -np.abs(w[2, 256:512]) if k >= 512 else w[2, 256:512]
    img = q.quantize_weights(q.Q4_K, torch.from_numpy(w).cuda())
    assert np.array_equal(img.cpu().numpy(), q.pack_image(q.Q4_K, O.quantize_weights(O.Q4_K, w), n, k))


@pytest.mark.parametrize("n,k,rows", [(1024, 1024, 1), (77, 768, 7), (16, 8192, 16), (40, 2048, 9), (33, 256, 2)])
def test_q4_k_blockdots_bit_exact(n, k, rows):
    log(f"q4_k blockdots n={n} k={k} rows={rows}")
    w = gauss((n, k), 0.02, 22, 3).numpy()
    x = _special(outliers((rows, k), 1.0, 22, 4).numpy())
    blocks, img = _image(w)
    qx, _, _ = O.quantize_acts(x)
    want = O.blockdots(O.Q4_K, blocks, n, k, qx)
    got = q.blockdots(q.Q4_K, img, n, k, torch.from_numpy(qx).cuda())
    assert np.array_equal(got.cpu().numpy(), want)
    if rows >= 3:  # the 3..16-row kernel's own block-pair products
        ws = q.prepare_rows(torch.from_numpy(x).cuda())
        assert np.array_equal(q.blockdots_pairs(q.Q4_K, img, n, k, ws, rows).cpu().numpy(), want)


@pytest.mark.parametrize("n,k", [(1024, 1024), (1000, 768), (33, 256), (257, 4096), (1, 512), (300, 8192)])
def test_q4_k_qgemv_parity(n, k):
    w = gauss((n, k), 0.02, 23, 5).numpy()
    blocks, img = _image(w)
    worst = 0.0
    for rows in ROWS:
        log(f"q4_k qgemv n={n} k={k} rows={rows}")
        x = _special(outliers((rows, k), 1.0, 23, 32 + rows).numpy())
        y = q.qgemv_q4_k(img, n, k, torch.from_numpy(x).cuda()).cpu().numpy()
        yo = O.gemv_q(O.Q4_K, blocks, n, k, x, threads=8)
        e = rel_err(y, yo, blocks, O.Q4_K, x)
        worst = max(worst, e)
        assert e <= TOL, (rows, e)
    log(f"  worst relative error {worst:.3e}")
    assert worst < 1e-5  # only the fp32 rounding order differs from the oracle


def test_q4_k_rows_in_a_batch_equal_rows_alone():
    n, k = 600, 3072
    _, img = _image(gauss((n, k), 0.02, 24, 6).numpy())
    x = torch.from_numpy(gauss((16, k), 1.0, 24, 7).numpy()).cuda()
    alone = [q.qgemv_q4_k(img, n, k, x[r:r + 1].contiguous()) for r in range(16)]
    for rows in (2, 3, 8, 9, 16):
        y = q.qgemv_q4_k(img, n, k, x[:rows].contiguous())
        for r in range(rows):
            assert np.array_equal(bits(y[r]), bits(alone[r][0])), (rows, r)


def test_q4_k_guard_rows_and_workspace_contents():
    """Outputs past the written rows stay NaN; a workspace full of stale bytes changes nothing."""
    n, k, rows = 300, 1536, 9
    blocks, img = _image(gauss((n, k), 0.02, 25, 8).numpy())
    x = gauss((rows, k), 1.0, 25, 9).numpy()
    ybuf = torch.full(((rows + 4) * n,), float("nan"), device="cuda")
    y_view = ybuf[2 * n:(2 + rows) * n].view(rows, n)
    ws = torch.full((q.workspace_bytes(rows, k),), 0x5A, dtype=torch.uint8, device="cuda")
    q.qgemv_q4_k(img, n, k, torch.from_numpy(x).cuda(), y=y_view, ws=ws)
    yb = ybuf.cpu().numpy()
    assert np.all(np.isnan(yb[:2 * n])) and np.all(np.isnan(yb[(2 + rows) * n:]))
    assert rel_err(y_view.cpu().numpy(), O.gemv_q(O.Q4_K, blocks, n, k, x, threads=8), blocks, O.Q4_K, x) <= TOL


def _sample(n, count, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], r.integers(0, n, count)]))


def test_llama3b_layer_q4_k():
    """The Llama-3.2-3B-shaped layer in Q4_K (the race bed's format) from fp32 rows, as the benchmark runs it, at
    1, 2, 4 and 8 rows: sampled outputs against the oracle, and rows 0 and 7 of 8 equal to those rows alone."""
    blocks, imgs = [], []
    for i, (_, n, k) in enumerate(LAYER_3B):
        b, im = _image(gauss((n, k), 0.02, 5, i, device="cuda").cpu().numpy())
        blocks.append(b)
        imgs.append(im)
    src = {"wo": 1, "down": 2}

    def run(xin, sample):
        xs = [torch.from_numpy(a).cuda() for a in xin]
        rows = xs[0].shape[0]
        projs, outs = [], []
        for i, (name, n, k) in enumerate(LAYER_3B):
            y = torch.full((rows, n), float("nan"), device="cuda")
            outs.append(y)
            projs.append((imgs[i], n, k, xs[src.get(name, 0)], q.empty_ws(rows, k), y))
        q.qgemv_set_rows(q.Q4_K, projs, rows)
        for i, (name, n, k) in enumerate(LAYER_3B if sample else []):
            x = xin[src.get(name, 0)]
            sel = _sample(n, 200, 300 + i)
            yo = O.gemv_q_rows(O.Q4_K, blocks[i], n, k, x, sel, threads=16)
            e = rel_err(outs[i].cpu().numpy()[:, sel], yo, blocks[i], O.Q4_K, x, sel=sel)
            log(f"  {name} {n}x{k} rows={rows} max rel err {e:.3e}")
            assert e <= TOL
        return outs

    for rows in (1, 2, 4, 8):
        log(f"3B layer Q4_K rows={rows}")
        xin = (gauss((rows, 3072), 1.0, 5, 32 + rows).numpy(), gauss((rows, 3072), 1.0, 5, 48 + rows).numpy(),
               gauss((rows, 8192), 1.0, 5, 64 + rows).numpy())
        ys = run(xin, True)
    for r in (0, 7):
        y1 = run(tuple(np.ascontiguousarray(a[r:r + 1]) for a in xin), False)
        for i, (name, _, _) in enumerate(LAYER_3B):
            assert np.array_equal(bits(ys[i][r]), bits(y1[i][0])), (name, r)
