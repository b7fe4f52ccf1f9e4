"""Shared test plumbing: seeded inputs, oracle-built images, and the parity metric.

The weight images that the HIP path reads in parity tests are packed (by the
library's host packer) from canonical blocks made by the oracle's quantizer, so
both sides see the same quantized weights; the device quantizer is checked
separately against the oracle's bytes.
"""
import numpy as np
import torch

import oracle as O
from block_quantized_few_amd import qgemv as q
from block_quantized_few_amd import synth

TOL = 2e-3  # max |y_gpu - y_oracle| / sum_k |w_hat| |x|


def gauss(shape, sigma, workload, tensor_id, copy=0, device="cpu"):
    return synth.gaussian(shape, sigma, synth.tensor_seed(workload, tensor_id, copy), device=device)


def outliers(shape, sigma, workload, tensor_id, copy=0):
    return synth.gaussian_outliers(shape, sigma, synth.tensor_seed(workload, tensor_id, copy))


def oracle_image(fmt, w_np):
    """Oracle blocks of fp32 weights and the device image packed from them."""
    n, k = w_np.shape
    blocks = O.quantize_weights(fmt, w_np)
    img = torch.from_numpy(q.pack_image(fmt, blocks, n, k)).cuda()
    return blocks, img


def rel_err(y_gpu, y_orc, blocks, fmt, x_np, sel=None):
    """max |dy| / sum_k |w_hat[o][k]| |x[r][k]| over all (r, o); sel picks output rows of blocks."""
    n = blocks.shape[0]
    k = blocks.shape[1] * O.BLOCK_WEIGHTS[fmt]
    b = blocks if sel is None else blocks[sel]
    what = O.dequantize(fmt, b, b.shape[0], k)
    denom = np.abs(x_np.astype(np.float64)) @ np.abs(what).T
    diff = np.abs(np.asarray(y_gpu, np.float64) - np.asarray(y_orc, np.float64))
    zero = denom == 0
    assert np.all(diff[zero] == 0)
    if np.all(zero):
        return 0.0
    return float((diff[~zero] / denom[~zero]).max())


def rel_err_f16(y_gpu, y_orc, w16_np, x_np):
    w = w16_np.view(np.float16).astype(np.float64)
    denom = np.abs(x_np.astype(np.float64)) @ np.abs(w).T
    diff = np.abs(np.asarray(y_gpu, np.float64) - np.asarray(y_orc, np.float64))
    zero = denom == 0
    assert np.all(diff[zero] == 0)
    return float((diff[~zero] / denom[~zero]).max()) if np.any(~zero) else 0.0


def bits(t):
    a = t.detach().cpu().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def log(msg):
    print(msg, flush=True)
