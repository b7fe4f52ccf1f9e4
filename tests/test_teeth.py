"""The parity metric has teeth: each plausible defect of a GEMV kernel, planted on the CPU in the oracle's
inputs, moves the result past the 2e-3 bar that the GPU parity tests apply.

A defect is simulated by computing the oracle on a corrupted copy of what a kernel would read (nibbles in the
other order, blocks or rows off by one, a scale dropped, a code sign flipped, the Q4_0 offset skipped) and
measuring that output with the same metric, max |dy| / sum_k |w_hat| |x|, against the correct oracle output.
No GPU is involved.
"""
import numpy as np
import pytest

import oracle as O
from block_quantized_few_amd import synth

TOL = 2e-3  # the GPU parity bar (tests/helpers.py)


def _metric(y_bad, y_ref, blocks, fmt, x):
    n, k = blocks.shape[0], blocks.shape[1] * 32
    denom = np.abs(x.astype(np.float64)) @ np.abs(O.dequantize(fmt, blocks, n, k)).T
    return float((np.abs(y_bad.astype(np.float64) - y_ref.astype(np.float64)) / denom).max())


def _case(fmt, n=64, k=1024, rows=4, seed=3):
    w = synth.gaussian((n, k), 0.02, synth.tensor_seed(11, seed)).numpy()
    x = synth.gaussian((rows, k), 1.0, synth.tensor_seed(11, 40 + seed)).numpy()
    blocks = O.quantize_weights(fmt, w)
    return blocks, x, O.gemv_q(fmt, blocks, n, k, x)


def _swap_nibbles(blocks):
    b = blocks.copy()
    p = b[:, :, 2:]
    b[:, :, 2:] = ((p & 0x0F) << 4) | (p >> 4)
    return b


def _pair_nibbles_adjacent(blocks):
    # another plausible packing: byte j holds codes 2j (low) and 2j+1 (high) instead of j and j+16
    b = blocks.copy()
    codes = np.concatenate([blocks[:, :, 2:] & 0x0F, blocks[:, :, 2:] >> 4], axis=2)  # codes 0..31 in order
    b[:, :, 2:] = codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)
    return b


def _shift_blocks(blocks):
    return np.concatenate([blocks[:, 1:], blocks[:, :1]], axis=1)  # block b reads block b+1's bytes


def _shift_codes_only(blocks):
    b = blocks.copy()
    b[:, :, 2:] = np.roll(blocks[:, :, 2:], 1, axis=1)  # codes of the next block under this block's scale
    return b


def _shift_rows(blocks):
    return np.concatenate([blocks[1:], blocks[:1]], axis=0)


def _scale_of_next_row(blocks):
    b = blocks.copy()
    b[:-1, :, 0:2] = blocks[1:, :, 0:2]
    return b


def _negate_q8(blocks):
    b = blocks.copy()
    b[:, ::7, 2:] = (-blocks[:, ::7, 2:].view(np.int8)).view(np.uint8)  # one block in seven with its sign lost
    return b


def _drop_last_block(blocks):
    b = blocks.copy()
    b[:, -1, :] = 0  # the tail block never read
    return b


def _high_half_dropped(blocks):
    b = blocks.copy()
    b[:, :, 18:34] = 0  # Q8_0: codes 16..31 of every block never read
    return b


Q8_DEFECTS = [_shift_blocks, _shift_codes_only, _shift_rows, _scale_of_next_row, _negate_q8, _drop_last_block,
              _high_half_dropped]
Q4_DEFECTS = [_swap_nibbles, _pair_nibbles_adjacent, _shift_blocks, _shift_codes_only, _shift_rows,
              _scale_of_next_row, _drop_last_block]


@pytest.mark.parametrize("defect", Q8_DEFECTS, ids=lambda f: f.__name__)
def test_q8_0_defects_fail_the_bar(defect):
    blocks, x, y = _case(O.Q8_0)
    n, k = blocks.shape[0], blocks.shape[1] * 32
    y_bad = O.gemv_q(O.Q8_0, defect(blocks), n, k, x)
    assert _metric(y_bad, y, blocks, O.Q8_0, x) > 10 * TOL


@pytest.mark.parametrize("defect", Q4_DEFECTS, ids=lambda f: f.__name__)
def test_q4_0_defects_fail_the_bar(defect):
    blocks, x, y = _case(O.Q4_0)
    n, k = blocks.shape[0], blocks.shape[1] * 32
    y_bad = O.gemv_q(O.Q4_0, defect(blocks), n, k, x)
    assert _metric(y_bad, y, blocks, O.Q4_0, x) > 10 * TOL


def test_q4_0_offset_skipped_fails_the_bar():
    # codes used as c instead of c - 8: the same as adding 8 * d * sum(x_hat) to every block
    blocks, x, y = _case(O.Q4_0)
    n, k = blocks.shape[0], blocks.shape[1] * 32
    qx, dx, sx = O.quantize_acts(x)
    isum = O.blockdots(O.Q4_0, blocks, n, k, qx).astype(np.float64) + 8.0 * sx[:, None, :]
    d = O.f16_to_f32(blocks[:, :, 0:2].copy().view(np.uint16)[..., 0]).astype(np.float64)
    y_bad = np.einsum("rnb,nb,rb->rn", isum, d, dx.astype(np.float64))
    assert _metric(y_bad, y, blocks, O.Q4_0, x) > 10 * TOL


def test_activation_scale_of_the_wrong_block_fails_the_bar():
    blocks, x, y = _case(O.Q8_0)
    n, k = blocks.shape[0], blocks.shape[1] * 32
    qx, dx, _ = O.quantize_acts(x)
    isum = O.blockdots(O.Q8_0, blocks, n, k, qx).astype(np.float64)
    d = O.f16_to_f32(blocks[:, :, 0:2].copy().view(np.uint16)[..., 0]).astype(np.float64)
    y_bad = np.einsum("rnb,nb,rb->rn", isum, d, np.roll(dx, 1, axis=1).astype(np.float64))
    assert _metric(y_bad, y, blocks, O.Q8_0, x) > 10 * TOL


def test_rows_swapped_in_a_batch_fail_the_bar():
    # a row tiled into another row's output slot (the tail mistake of the audio-towers page's router GEMV)
    blocks, x, y = _case(O.Q8_0, rows=9)
    y_bad = y.copy()
    y_bad[8], y_bad[0] = y[0], y[8]
    assert _metric(y_bad, y, blocks, O.Q8_0, x) > 10 * TOL


def test_fp32_reordering_passes_the_bar():
    # the control: a legitimate change of summation order (fp32 in reverse block order) stays far inside
    blocks, x, y = _case(O.Q8_0)
    n, k = blocks.shape[0], blocks.shape[1] * 32
    qx, dx, _ = O.quantize_acts(x)
    isum = O.blockdots(O.Q8_0, blocks, n, k, qx).astype(np.float32)
    d = O.f16_to_f32(blocks[:, :, 0:2].copy().view(np.uint16)[..., 0]).astype(np.float32)
    y32 = np.zeros(y.shape, np.float32)
    for b in reversed(range(k // 32)):
        y32 = y32 + isum[:, :, b] * (d[None, :, b] * dx[:, None, b])
    assert _metric(y32, y, blocks, O.Q8_0, x) < TOL / 100
