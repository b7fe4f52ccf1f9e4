"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes one by one.

LM head 128256 x 4096 (Q8_0, Q4_0, Q4_K and f16) at rows 1, 2, 8, 16; the Llama-3.2-1B-shaped
Q8_0 decode layer (seven projections, one set launch) at rows 1 and 16, and at
rows 1 and 2 straight from fp32 rows (quantized inside the GEMV launch, as the
benchmark runs it); the Llama-3.2-3B-shaped Q4_0 layer at rows 1, 2, 4, 8."""
import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, rel_err, rel_err_f16

pytestmark = pytest.mark.gpu

LAYER_1B = [("wq", 2048, 2048), ("wk", 512, 2048), ("wv", 512, 2048), ("wo", 2048, 2048), ("gate", 8192, 2048),
            ("up", 8192, 2048), ("down", 2048, 8192)]
LAYER_3B = [("wq", 3072, 3072), ("wk", 1024, 3072), ("wv", 1024, 3072), ("wo", 3072, 3072), ("gate", 8192, 3072),
            ("up", 8192, 3072), ("down", 3072, 8192)]


def _sample(n, count, seed):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], r.integers(0, n, count)]))


def test_lm_head_q8_0():
    n, k = 128256, 4096
    log("LM head Q8_0: weights")
    w = gauss((n, k), 0.02, 4, 0, device="cuda").cpu().numpy()
    blocks = O.quantize_weights(O.Q8_0, w)
    del w
    img = torch.from_numpy(q.pack_image(q.Q8_0, blocks, n, k)).cuda()
    sel = _sample(n, 512, 1)
    ys = {}
    for rows in (1, 2, 8, 16):
        log(f"LM head Q8_0 rows={rows}")
        x = gauss((rows, k), 1.0, 4, 32 + rows).numpy()
        y = q.qgemv_q8_0(img, n, k, torch.from_numpy(x).cuda())
        yo = O.gemv_q_rows(O.Q8_0, blocks, n, k, x, sel, threads=16)
        e = rel_err(y.cpu().numpy()[:, sel], yo, blocks, O.Q8_0, x, sel=sel)
        log(f"  max rel err {e:.3e}")
        assert e <= TOL
        ys[rows] = (x, y)
    # the first rows of the 16-row call equal calls with fewer rows of the same inputs (the pair tile over
    # several rounds of workgroups at 8 and 16 rows, the one-row kernel at 1)
    x16 = torch.from_numpy(ys[16][0]).cuda()
    y8 = q.qgemv_q8_0(img, n, k, x16[:8].contiguous())
    assert np.array_equal(bits(y8), bits(ys[16][1][:8]))
    y1 = q.qgemv_q8_0(img, n, k, x16[:1].contiguous())
    assert np.array_equal(bits(y1), bits(ys[16][1][:1]))
    # two rows (quantized inside the launch, many tiles per CU): each row has its bits alone
    x2 = torch.from_numpy(ys[2][0]).cuda()
    for r in range(2):
        y1 = q.qgemv_q8_0(img, n, k, x2[r:r + 1].contiguous())
        assert np.array_equal(bits(y1), bits(ys[2][1][r:r + 1])), r


@pytest.mark.parametrize("fmt,ofmt,wl", [(q.Q4_0, O.Q4_0, 6), (q.Q4_K, O.Q4_K, 7)])
def test_lm_head_4bit(fmt, ofmt, wl):
    """The LM head in the 4-bit formats at rows 1, 2, 8 and 16 through the entry point (quantization fused at
    1-2 rows; the pair kernel's wide tiles at 16): sampled outputs against the oracle, and the rows of the
    16-row call equal to the same rows in calls of 8 and 1."""
    n, k = 128256, 4096
    log(f"LM head fmt={fmt}: weights")
    w = gauss((n, k), 0.02, wl, 0, device="cuda").cpu().numpy()
    blocks = O.quantize_weights(ofmt, w)
    del w
    img = torch.from_numpy(q.pack_image(fmt, blocks, n, k)).cuda()
    call = q.qgemv_q4_0 if fmt == q.Q4_0 else q.qgemv_q4_k
    sel = _sample(n, 384, 3 + wl)
    ys = {}
    for rows in (1, 2, 8, 16):
        log(f"LM head fmt={fmt} rows={rows}")
        x = gauss((rows, k), 1.0, wl, 32 + rows).numpy()
        y = call(img, n, k, torch.from_numpy(x).cuda())
        yo = O.gemv_q_rows(ofmt, blocks, n, k, x, sel, threads=16)
        e = rel_err(y.cpu().numpy()[:, sel], yo, blocks, ofmt, x, sel=sel)
        log(f"  max rel err {e:.3e}")
        assert e <= TOL
        ys[rows] = (x, y)
    x16 = torch.from_numpy(ys[16][0]).cuda()
    y8 = call(img, n, k, x16[:8].contiguous())
    assert np.array_equal(bits(y8), bits(ys[16][1][:8]))
    y1 = call(img, n, k, x16[15:16].contiguous())
    assert np.array_equal(bits(y1), bits(ys[16][1][15:16]))


def test_lm_head_f16():
    n, k = 128256, 4096
    log("LM head f16: weights")
    w16 = gauss((n, k), 0.02, 4, 0, device="cuda").half().view(torch.int16)
    w16_np = w16.cpu().numpy().view(np.uint16)
    img = q.f16_image(w16)
    sel = _sample(n, 512, 2)
    for rows in (1, 8, 16):
        log(f"LM head f16 rows={rows}")
        x = gauss((rows, k), 1.0, 4, 32 + rows).numpy()
        y = q.gemv_f16(img, n, k, torch.from_numpy(x).cuda())
        yo = O.gemv_f16_rows(w16_np, x, sel, threads=16)
        e = rel_err_f16(y.cpu().numpy()[:, sel], yo, w16_np[sel], x)
        log(f"  max rel err {e:.3e}")
        assert e <= TOL


def _layer(fmt, ofmt, layer, wl):
    blocks, imgs = [], []
    for i, (_, n, k) in enumerate(layer):
        w = gauss((n, k), 0.02, wl, i, device="cuda").cpu().numpy()
        b = O.quantize_weights(ofmt, w)
        blocks.append(b)
        imgs.append(torch.from_numpy(q.pack_image(fmt, b, n, k)).cuda())
    return blocks, imgs


def _run_set(fmt, ofmt, layer, blocks, imgs, rows, wl, full, xin=None, check=True):
    k_in, k_dn = layer[0][2], layer[6][2]
    if xin is None:
        x_in = gauss((rows, k_in), 1.0, wl, 32 + rows).numpy()
        x_o = gauss((rows, k_in), 1.0, wl, 48 + rows).numpy()
        x_dn = gauss((rows, k_dn), 1.0, wl, 64 + rows).numpy()
    else:
        x_in, x_o, x_dn = xin
    xs = [torch.from_numpy(a).cuda() for a in (x_in, x_o, x_dn)]
    wss = [q.empty_ws(rows, a.shape[1]) for a in xs]
    q.prepare_rows_set(xs, wss)
    src = {"wo": 1, "down": 2}
    projs, outs = [], []
    for i, (name, n, k) in enumerate(layer):
        j = src.get(name, 0)
        y = torch.full((rows, n), float("nan"), device="cuda")
        outs.append((y, (x_in, x_o, x_dn)[j]))
        projs.append((imgs[i], n, k, wss[j], y))
    q.qgemv_set(fmt, projs, rows)
    for i, (name, n, k) in enumerate(layer):
        if not check:
            break
        y, x = outs[i]
        sel = np.arange(n) if full else _sample(n, 256, i)
        yo = O.gemv_q_rows(ofmt, blocks[i], n, k, x, sel, threads=16)
        e = rel_err(y.cpu().numpy()[:, sel], yo, blocks[i], ofmt, x, sel=sel)
        log(f"  {name} {n}x{k} rows={rows} max rel err {e:.3e}")
        assert e <= TOL
    return [y for y, _ in outs], (x_in, x_o, x_dn)


def _rows_alone(fmt, ofmt, layer, blocks, imgs, ys, xin, wl, which):
    """Rows of a full-size batch (its tiling and kernel chosen for that row count) have the bits of the
    same rows computed alone (the one-row kernel)."""
    for r in which:
        one = tuple(np.ascontiguousarray(a[r:r + 1]) for a in xin)
        y1, _ = _run_set(fmt, ofmt, layer, blocks, imgs, 1, wl, False, xin=one, check=False)
        for i, (name, n, k) in enumerate(layer):
            assert np.array_equal(bits(ys[i][r]), bits(y1[i][0])), f"{name} row {r}"


def test_llama1b_layer_q8_0_set():
    blocks, imgs = _layer(q.Q8_0, O.Q8_0, LAYER_1B, 1)
    for rows in (1, 16):
        log(f"1B layer Q8_0 rows={rows}")
        ys, xin = _run_set(q.Q8_0, O.Q8_0, LAYER_1B, blocks, imgs, rows, 1, full=rows == 1)
    log("1B layer Q8_0: rows 0 and 15 of 16 alone")
    _rows_alone(q.Q8_0, O.Q8_0, LAYER_1B, blocks, imgs, ys, xin, 1, (0, 15))


def _run_set_rows(fmt, ofmt, layer, blocks, imgs, xin, sample=True):
    """The layer straight from fp32 rows (qgemv_set_rows): at 1-2 rows one launch that quantizes its rows."""
    xs = [torch.from_numpy(a).cuda() for a in xin]
    rows = xs[0].shape[0]
    src = {"wo": 1, "down": 2}
    projs, outs = [], []
    for i, (name, n, k) in enumerate(layer):
        j = src.get(name, 0)
        y = torch.full((rows, n), float("nan"), device="cuda")
        outs.append(y)
        projs.append((imgs[i], n, k, xs[j], None if rows <= q.FUSED_ROWS else q.empty_ws(rows, k), y))
    q.qgemv_set_rows(fmt, projs, rows)
    if sample:
        for i, (name, n, k) in enumerate(layer):
            x = xin[src.get(name, 0)]
            sel = _sample(n, 256, 100 + i)
            yo = O.gemv_q_rows(ofmt, blocks[i], n, k, x, sel, threads=16)
            e = rel_err(outs[i].cpu().numpy()[:, sel], yo, blocks[i], ofmt, x, sel=sel)
            log(f"  {name} {n}x{k} rows={rows} (fused) max rel err {e:.3e}")
            assert e <= TOL
    return outs


@pytest.mark.parametrize("shape,rows", [("1b", 1), ("1b", 2), ("3b", 1), ("3b", 2)])
def test_layer_fused_rows(shape, rows):
    """The benchmark's launch: the 1B-shaped Q8_0 and 3B-shaped Q4_0 layers from fp32 rows at 1 and 2 rows,
    outputs sampled against the oracle, and (2 rows) each row's bits equal to that row computed alone."""
    fmt, ofmt, layer, wl = (q.Q8_0, O.Q8_0, LAYER_1B, 1) if shape == "1b" else (q.Q4_0, O.Q4_0, LAYER_3B, 2)
    blocks, imgs = _layer(fmt, ofmt, layer, wl)
    k_in, k_dn = layer[0][2], layer[6][2]
    xin = (gauss((rows, k_in), 1.0, wl, 32 + rows).numpy(), gauss((rows, k_in), 1.0, wl, 48 + rows).numpy(),
           gauss((rows, k_dn), 1.0, wl, 64 + rows).numpy())
    log(f"{shape} layer from fp32 rows, rows={rows}")
    ys = _run_set_rows(fmt, ofmt, layer, blocks, imgs, xin)
    for r in range(rows if rows > 1 else 0):
        one = tuple(np.ascontiguousarray(a[r:r + 1]) for a in xin)
        y1 = _run_set_rows(fmt, ofmt, layer, blocks, imgs, one, sample=False)
        for i, (name, _, _) in enumerate(layer):
            assert np.array_equal(bits(ys[i][r]), bits(y1[i][0])), f"{name} row {r}"


def test_llama3b_layer_q4_0_set():
    blocks, imgs = _layer(q.Q4_0, O.Q4_0, LAYER_3B, 2)
    for rows in (1, 2, 4, 8):
        log(f"3B layer Q4_0 rows={rows}")
        ys, xin = _run_set(q.Q4_0, O.Q4_0, LAYER_3B, blocks, imgs, rows, 2, full=False)
    log("3B layer Q4_0: rows 0 and 7 of 8 alone")
    _rows_alone(q.Q4_0, O.Q4_0, LAYER_3B, blocks, imgs, ys, xin, 2, (0, 7))
