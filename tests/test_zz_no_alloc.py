"""qgemv_q8_0_noalloc (the allocation-free variant of qgemv_q8_0 on the library's static workspace) against
qgemv_q8_0 through the C ABI: the same kernels, so the same bits, call after call through the one shared
array -- the second call of each pair with a smaller input than the first."""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from helpers import TOL, bits, gauss, log, oracle_image, rel_err

pytestmark = pytest.mark.gpu


def _both(img, n, k, x):
    y_ref = q.qgemv_q8_0(img, n, k, x)
    y = torch.full((x.shape[0], n), float("nan"), device="cuda")
    st = q.lib().qgemv_q8_0_noalloc(C.c_void_p(img.data_ptr()), n, k, C.c_void_p(x.data_ptr()), x.shape[0],
                                    C.c_void_p(y.data_ptr()), C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, q.status_string(st)
    return y, y_ref


@pytest.mark.parametrize("first,second", [((16, 3000, 4096), (5, 1000, 1024)),
                                          ((16, 700, 28672), (9, 300, 2048)),
                                          ((8, 513, 8192), (3, 77, 800)),
                                          ((2, 4000, 4096), (1, 1024, 1024))])
def test_noalloc_equals_qgemv_q8_0(first, second):
    for rows, n, k in (first, second):
        log(f"noalloc rows={rows} n={n} k={k}")
        w = gauss((n, k), 0.02, 20, rows).numpy()
        blocks, img = oracle_image(O.Q8_0, w)
        x_np = gauss((rows, k), 1.0, 20, 40 + rows).numpy()
        x = torch.from_numpy(x_np).cuda()
        y, y_ref = _both(img, n, k, x)
        assert np.array_equal(bits(y), bits(y_ref))
        sel = np.unique(np.linspace(0, n - 1, 64).astype(np.int64))
        yo = O.gemv_q_rows(O.Q8_0, blocks, n, k, x_np, sel, threads=8)
        assert rel_err(y.cpu().numpy()[:, sel], yo, blocks, O.Q8_0, x_np, sel=sel) <= TOL


def test_noalloc_refuses_past_its_workspace():
    n, k, rows = 64, 28704, 16  # needs 1,050,624 bytes
    img = torch.zeros(q.image_bytes(q.Q8_0, n, k), dtype=torch.uint8, device="cuda")
    x = torch.zeros((rows, k), device="cuda")
    y = torch.full((rows, n), float("nan"), device="cuda")
    st = q.lib().qgemv_q8_0_noalloc(C.c_void_p(img.data_ptr()), n, k, C.c_void_p(x.data_ptr()), rows,
                                    C.c_void_p(y.data_ptr()), None)
    assert st == -5
    torch.cuda.synchronize()
    assert torch.isnan(y).all()  # nothing launched
    # two rows need no workspace at that k
    y2 = q.qgemv_q8_0_noalloc(img, n, k, x[:2].contiguous())
    assert torch.equal(y2, torch.zeros_like(y2))
