"""The C-ABI library on a host without a GPU: it loads, exports every symbol the
header declares, answers its host-only queries, packs images, and refuses bad
arguments with the documented status before touching HIP."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from block_quantized_few_amd import qgemv as q
from block_quantized_few_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qgemv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s+([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 20, names
    L = C.CDLL(q.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(q._SIGS), set(names) ^ set(q._SIGS)


def test_sizes():
    assert q.image_bytes(q.Q8_0, 1024, 1024) == 1024 * 1024 // 32 * 34
    assert q.image_bytes(q.Q4_0, 3072, 3072) == 3072 * 3072 // 32 * 18
    assert q.image_bytes(q.Q8_0, 128256, 4096) == 558170112
    assert q.image_bytes(q.F16, 128256, 4096) == 1050673152
    assert q.image_bytes(q.Q8_0, 1024, 1000) == 0  # k not a multiple of 32
    assert q.image_bytes(q.F16, 8, 12) == 0
    # F16 image: 16-row tiles x 32-column steps, 1 KB each, padded with zeros
    assert q.image_bytes(q.F16, 33, 104) == 3 * 4 * 1024
    assert q.image_bytes(7, 8, 32) == 0
    # a ragged k is padded to whole 16-block groups
    assert q.image_bytes(q.Q8_0, 3, 96) >= 3 * 512 // 32 * 34
    assert q.workspace_bytes(0, 1024) == 0 and q.workspace_bytes(17, 1024) > 0
    assert q.workspace_bytes(1, 33) == 0
    # row order for 1-2 rows: codes + fp32 scales + int32 start values per block
    assert q.workspace_bytes(2, 2048) == 2 * 2048 + 2 * 64 * 4 * 2
    # pair order for 3-16 rows: per block pair and group of eight rows a 1 KB chunk + 16 scales + 16 start values
    assert q.workspace_bytes(8, 2048) == 32 * 1 * (1024 + 64 + 64)
    assert q.workspace_bytes(16, 2048) == 32 * 2 * (1024 + 64 + 64)
    assert q.workspace_bytes(3, 2048) == q.workspace_bytes(8, 2048)
    assert q.grouped_workspace_bytes(16, 2048, 136) > 16 * 2048 + 136 * 4
    assert q.grouped_workspace_bytes(16, 2048, q.MAX_ASSIGN + 1) == 0


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0])
@pytest.mark.parametrize("n,k", [(5, 32), (7, 512), (3, 800), (2, 8192)])
def test_pack_unpack_roundtrip(fmt, n, k):
    w = synth.gaussian((n, k), 0.02, synth.tensor_seed(9, 1)).numpy()
    blocks = O.quantize_weights(fmt, w)
    img = q.pack_image(fmt, blocks, n, k)
    assert img.size == q.image_bytes(fmt, n, k)
    assert np.array_equal(q.unpack_image(fmt, img, n, k), blocks)


def test_pack_layout_of_one_q8_block():
    # row o, block b: tile t = o // 16, i = o % 16; low half at (t*kbp + b)*512 + 16*i, high half +256;
    # scale (fp16) at scale plane + 2*((t*kbp + b)*16 + i)
    n, k = 40, 1024  # kb = kbp = 32, three tiles (the last one padded)
    blocks = np.zeros((n, k // 32, 34), np.uint8)
    o, b = 21, 17
    blocks[o, b, 0:2] = (0x34, 0x12)
    blocks[o, b, 2:34] = np.arange(1, 33, dtype=np.uint8)
    img = q.pack_image(q.Q8_0, blocks, n, k)
    t, i = o // 16, o % 16
    lo = (t * 32 + b) * 512 + 16 * i
    assert list(img[lo:lo + 16]) == list(range(1, 17))
    assert list(img[lo + 256:lo + 272]) == list(range(17, 33))
    scale_off = (48 * 32 * 32 + 255) // 256 * 256
    si = scale_off + 2 * ((t * 32 + b) * 16 + i)
    assert img[si] == 0x34 and img[si + 1] == 0x12
    assert img.sum() == sum(range(1, 33)) + 0x34 + 0x12  # everything else, padding included, is zero


def test_pack_layout_of_one_q4_block():
    n, k = 16, 512
    blocks = np.zeros((n, k // 32, 18), np.uint8)
    blocks[5, 3, 2:18] = np.arange(16, dtype=np.uint8) * 17
    img = q.pack_image(q.Q4_0, blocks, n, k)
    cell = (0 * 16 + 3) * 256 + 16 * 5
    # the image keeps each code c as c XOR 8 (the 4-bit two's complement of c - 8), nibble order unchanged
    assert list(img[cell:cell + 16]) == list((np.arange(16) * 17) ^ 0x88)
    assert np.array_equal(q.unpack_image(q.Q4_0, img, n, k), blocks)


@pytest.mark.parametrize("n,k", [(16, 32), (33, 104), (5, 8), (40, 200)])
def test_f16_image_layout(n, k):
    # chunk l = i + 16*j of (tile t, step s) holds w[16t + i][32s + 8j : 32s + 8j + 8]: the zero-padded
    # matrix cut into [t][i][s][j][8] and reordered to [t][s][j][i][8]
    rng = np.random.default_rng(n * 1000 + k)
    w = rng.integers(0, 1 << 16, size=(n, k), dtype=np.uint64).astype(np.uint16)
    T, S = -(-n // 16), -(-k // 32)
    pad = np.zeros((T * 16, S * 32), np.uint16)
    pad[:n, :k] = w
    want = pad.reshape(T, 16, S, 4, 8).transpose(0, 2, 3, 1, 4).reshape(-1)
    img = q.pack_image(q.F16, w, n, k)
    assert img.size == q.image_bytes(q.F16, n, k) == want.size * 2
    assert np.array_equal(img.view(np.uint16), want)
    assert np.array_equal(q.unpack_image(q.F16, img, n, k), w)


@pytest.mark.parametrize("n,k", [(16, 128), (33, 256), (200, 384)])
def test_fp8_image_layout(n, k):
    # lane l = i + 16j of (tile t, group g) holds codes[16t + i][128g + 32j : 128g + 32j + 32] as two 16-byte
    # halves h, at 16l and 1024 + 16l: the zero-padded codes cut into [t][i][g][j][h][16] and reordered to
    # [t][g][h][j][i][16]; then the scales, 256-byte aligned
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint64).astype(np.uint8)
    scales = rng.random(((n + 127) // 128, k // 128)).astype(np.float32)
    T, G = -(-n // 16), k // 128
    pad = np.zeros((T * 16, k), np.uint8)
    pad[:n] = codes
    want = pad.reshape(T, 16, G, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5).reshape(-1)
    img = q.pack_fp8(codes, scales)
    assert img.size == q.image_bytes(q.FP8, n, k)
    assert np.array_equal(img[:want.size], want)
    off = -(-want.size // 256) * 256
    assert np.array_equal(img[off:off + scales.nbytes].view(np.float32), scales.ravel())
    c2, s2 = q.unpack_fp8(img, n, k)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    assert q.image_bytes(q.FP8, n, 100) == 0
    assert q.fp8_workspace_bytes(3, k) == 3 * k + (-(-3 * k) % 256) + 256 * (-(-(3 * (k // 128) * 4) // 256))


def _status(fn, *args):
    L = q.lib()
    st = getattr(L, fn)(*args)
    buf = C.create_string_buffer(512)
    assert L.qg_last_error_detail(buf, 512) == st
    return st, buf.value.decode()


A = 256 * 64  # a 256-byte aligned fake address (never dereferenced: validation fails first)
V = C.c_void_p


def test_validation_refuses_before_any_hip_call():
    MB = 1 << 20
    st, msg = _status("qgemv_q8_0", V(A), 1024, 1024, V(A), 17, V(A), V(A), MB, None)
    assert st == -3 and "rows=17" in msg
    st, msg = _status("qgemv_q8_0", V(A), 1024, 1000, V(A), 1, V(A), V(A), MB, None)
    assert st == -2 and "k=1000" in msg
    st, msg = _status("qgemv_q8_0", V(A), 0, 1024, V(A), 1, V(A), V(A), MB, None)
    assert st == -2 and "n=0" in msg
    st, msg = _status("qgemv_q4_0", None, 1024, 1024, V(A), 1, V(A), V(A), MB, None)
    assert st == -1 and "w_image" in msg
    st, msg = _status("qgemv_q4_0", V(A + 16), 1024, 1024, V(A), 1, V(A), V(A), MB, None)
    assert st == -4 and "w_image" in msg
    st, msg = _status("qgemv_q8_0", V(A), 1024, 1024, V(A + 4), 1, V(A), V(A), MB, None)
    assert st == -4 and "x" in msg
    st, msg = _status("qgemv_q8_0", V(A), 1024, 1024, V(A), 2, V(A), V(A), 100, None)
    assert st == -5 and "ws_bytes=100" in msg
    st, msg = _status("gemv_f16", V(A), 64, 12, V(A), 1, V(A), None)
    assert st == -2
    st, msg = _status("gemv_f16", V(A + 16), 64, 64, V(A), 1, V(A), None)
    assert st == -4 and "w_image" in msg
    st, msg = _status("qg_f16_image", V(A), 64, 12, V(A), None)
    assert st == -2 and "k=12" in msg
    st, msg = _status("qg_f16_image", V(A + 8), 64, 64, V(A), None)
    assert st == -4 and "w " in msg
    st, msg = _status("qg_f16_image", V(A), 64, 64, V(A + 16), None)
    assert st == -4 and "image" in msg
    st, msg = _status("qgemv_prepared", 9, V(A), 64, 64, V(A), MB, 1, V(A), None)
    assert st == -1 and "fmt=9" in msg
    # a workspace prepared for two rows (row order) is too small for three (pair order): refused, not read past
    ws2 = q.workspace_bytes(2, 2048)
    assert ws2 < q.workspace_bytes(3, 2048)
    st, msg = _status("qgemv_prepared", q.Q8_0, V(A), 64, 2048, V(A), ws2, 3, V(A), None)
    assert st == -5 and f"ws_bytes={ws2}" in msg
    st, msg = _status("qgemv_prepared", q.Q4_0, V(A), 64, 2048, V(A), 100, 1, V(A), None)
    assert st == -5 and "ws_bytes=100" in msg
    st, msg = _status("qgemv_prepared", q.Q8_0, V(A), 64, 2048, None, MB, 1, V(A), None)
    assert st == -1 and "workspace is null" in msg
    st, msg = _status("qgemv_prepared", q.Q8_0, V(A), 64, 2048, V(A + 16), MB, 1, V(A), None)
    assert st == -4
    st, msg = _status("qgemv_prepared", q.Q8_0, V(A), 64, 2048, None, 0, 0, V(A), None)
    assert st == 0  # rows == 0: a no-op, the workspace is not needed
    # qgemv_set: each entry's workspace is checked against the layout its row count reads
    projs = (q._Proj * 2)(q._Proj(A, 64, 2048, A, MB, A), q._Proj(A, 64, 2048, A, ws2, A))
    st, msg = _status("qgemv_set", q.Q8_0, projs, 2, 3, None)
    assert st == -5 and "projs[1]" in msg
    st, msg = _status("qgemv_set", q.Q8_0, projs, 2, 2, None)
    assert st == -7  # both workspaces hold two rows: a valid call, no GPU here
    st, msg = _status("qgemv_q8_0_grouped", V(A), 8, 64, 64, V(A), 1, V(A), V(A), q.MAX_ASSIGN + 1, V(A), V(A),
                      MB, None)
    assert st == -2
    st, msg = _status("qg_moe_route", V(A), 1, 2000, 8, -1, V(A), V(A), V(A), None)
    assert st == -2
    # FP8 lane: k a multiple of 128, rows within bounds, workspace size
    st, msg = _status("qgemv_fp8", V(A), 64, 96, V(A), 1, V(A), V(A), MB, None)
    assert st == -2 and "k=96" in msg
    st, msg = _status("qgemv_fp8", V(A), 64, 256, V(A), 17, V(A), V(A), MB, None)
    assert st == -3
    st, msg = _status("qgemv_fp8", V(A), 64, 256, V(A), 2, V(A), V(A), 100, None)
    assert st == -5 and "ws_bytes=100" in msg
    st, msg = _status("qg_prepare_fp8", V(A), 2, 200, V(A), MB, None)
    assert st == -2
    st, msg = _status("qgemv_fp8_prepared", V(A + 16), 64, 256, V(A), MB, 1, V(A), None)
    assert st == -4 and "w_image" in msg
    fb = q.fp8_workspace_bytes(4, 256)
    st, msg = _status("qgemv_fp8_prepared", V(A), 64, 256, V(A), fb, 5, V(A), None)
    assert st == -5 and f"ws_bytes={fb}" in msg
    st, msg = _status("qgemv_fp8_prepared", V(A), 64, 256, V(A), fb, 4, V(A), None)
    assert st == -7
    st, msg = _status("qg_quantize_weights", q.FP8, V(A), 64, 96, V(A), None)
    assert st == -2 and "k=96" in msg
    st, msg = _status("qgemv_fp8", V(A), 64, 256, V(A), 0, V(A), V(A), 0, None)
    assert st == 0
    # FP8 grouped: images, n_experts, n, k, x, x_rows, expert, x_index, m, y, ws, ws_bytes
    st, msg = _status("qgemv_fp8_grouped", V(A), 8, 64, 96, V(A), 1, V(A), V(A), 4, V(A), V(A), MB, None)
    assert st == -2 and "k=96" in msg
    st, msg = _status("qgemv_fp8_grouped", V(A), 8, 64, 256, V(A), 1, V(A), V(A), q.MAX_ASSIGN + 1, V(A), V(A),
                      MB, None)
    assert st == -2
    st, msg = _status("qgemv_fp8_grouped", V(A), 8, 64, 256, V(A), 2, V(A), V(A), 4, V(A), V(A), 100, None)
    assert st == -5 and "ws_bytes=100" in msg
    st, msg = _status("qgemv_fp8_grouped", V(A), 8, 64, 256, V(A), 2, None, V(A), 4, V(A), V(A), MB, None)
    assert st == -1
    # its workspace: the grouped plan (256-byte header, then 10 sorted indices and 10 items, each plane 256-byte
    # aligned), then the FP8 groups of the 3 x rows
    assert q.fp8_grouped_workspace_bytes(3, 256, 10) == 256 + 256 + 256 + q.fp8_workspace_bytes(3, 256)
    assert q.fp8_grouped_workspace_bytes(3, 200, 10) == 0 and q.fp8_grouped_workspace_bytes(3, 256, -1) == 0
    # qg_add_rmsnorm_prepare: x, residual, gamma, eps, rows, k, h_out, y_out, ws, ws_bytes
    norm = lambda **kw: _status("qg_add_rmsnorm_prepare", V(kw.get("x", A)), None, V(kw.get("gamma", A)),
                                C.c_float(kw.get("eps", 1e-5)), kw.get("rows", 2), kw.get("k", 2048), None,
                                V(kw["y"]) if "y" in kw else None, V(kw["ws"]) if "ws" in kw else V(A),
                                kw.get("bytes", MB), None)
    st, msg = norm(k=100)
    assert st == -2 and "k=100" in msg
    st, msg = norm(rows=8193)
    assert st == -3 and "rows=8193" in msg
    st, msg = norm(gamma=0)
    assert st == -1 and "gamma" in msg
    st, msg = norm(gamma=A + 4)
    assert st == -4 and "gamma" in msg
    st, msg = norm(eps=-1.0)
    assert st == -1 and "eps" in msg
    st, msg = norm(ws=0)
    assert st == -1 and "no output" in msg
    st, msg = norm(bytes=100)
    assert st == -5 and "ws_bytes=100" in msg
    st, msg = norm(rows=0)
    assert st == 0
    st, msg = norm(ws=0, y=A)
    assert st == -7  # a valid call: no GPU here
    # qg_moe_step: router, E, hidden, ffn, topk, shared, gu, down, x, rows, y, logits, expert, weight, ws, bytes
    moe = lambda **kw: _status("qg_moe_step", V(A), kw.get("E", 256), kw.get("hidden", 2048), kw.get("ffn", 512),
                               kw.get("topk", 8), kw.get("shared", 1), V(A), V(A), V(A), kw.get("rows", 1), V(A),
                               None, None, None, V(A), kw.get("bytes", 1 << 30), None)
    st, msg = moe(rows=17)
    assert st == -3 and "rows=17" in msg
    st, msg = moe(topk=0)
    assert st == -2 and "topk=0" in msg
    st, msg = moe(shared=2)
    assert st == -1 and "shared=2" in msg
    st, msg = moe(ffn=500)
    assert st == -2 and "ffn=500" in msg
    st, msg = moe(bytes=100)
    assert st == -5
    assert q.moe_workspace_bytes(16, 256, 2048, 512, 8, True) > 16 * 9 * (2048 + 1024) * 4
    assert q.moe_workspace_bytes(17, 256, 2048, 512, 8, True) == 0
    assert q.status_string(-3) == "rows outside 0..16"


def test_pair_blockdots_validation():
    # fmt, image, n, k, ws, ws_bytes, rows, isum, stream
    st, msg = _status("qgemv_blockdots_pairs", q.Q8_0, V(A), 64, 2048, V(A), 1 << 20, 2, V(A), None)
    assert st == -3 and "rows=2" in msg
    small = q.workspace_bytes(8, 2048)
    st, msg = _status("qgemv_blockdots_pairs", q.Q4_0, V(A), 64, 2048, V(A), small, 9, V(A), None)
    assert st == -5 and f"ws_bytes={small}" in msg
    st, msg = _status("qgemv_blockdots_pairs", q.Q4_0, V(A), 64, 2048, V(A), small, 8, None, None)
    assert st == -1


def test_noalloc_validation():
    # image, n, k, x, rows, y, stream: a call past the static workspace is refused before any HIP call
    st, msg = _status("qgemv_q8_0_noalloc", V(A), 64, 28704, V(A), 16, V(A), None)
    assert st == -5 and "28704" in msg
    st, msg = _status("qgemv_q8_0_noalloc", V(A), 64, 2048, V(A), 17, V(A), None)
    assert st == -3
    st, msg = _status("qgemv_q8_0_noalloc", V(A), 0, 2048, V(A), 4, V(A), None)
    assert st == -2
    st, msg = _status("qgemv_q8_0_noalloc", V(A), 64, 2048, V(A), 0, V(A), None)
    assert st == 0
    assert q.workspace_bytes(16, 28672) <= q.NOALLOC_SCRATCH_BYTES < q.workspace_bytes(16, 28704)


def test_read_probe_validation():
    # src, bytes, grid, inflight, sink, stream
    st, msg = _status("qg_read_probe", V(A), 100, 256, 4, V(A), None)
    assert st == -4 and "bytes=100" in msg
    st, msg = _status("qg_read_probe", V(A), 1 << 20, 0, 4, V(A), None)
    assert st == -1 and "grid=0" in msg
    st, msg = _status("qg_read_probe", V(A), 1 << 20, 256, 3, V(A), None)
    assert st == -1 and "inflight=3" in msg
    st, msg = _status("qg_read_probe", None, 1 << 20, 256, 4, V(A), None)
    assert st == -1


def test_rows_zero_is_a_noop():
    st, _ = _status("qgemv_q8_0", V(A), 1024, 1024, V(A), 0, V(A), V(A), 0, None)
    assert st == 0


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0, reason="a GPU is present")
def test_valid_call_without_gpu_reports_device():
    st, msg = _status("qgemv_q8_0", V(A), 64, 64, V(A), 1, V(A), V(A), 1 << 20, None)
    assert st == -7, msg


def test_device_probe_answers_false_not_an_error():
    # invalid device numbers are a failure of the driver query: 0, never a negative status
    assert q.lib().qg_device_supported(-1) == 0
    assert q.lib().qg_device_supported(1 << 20) == 0
    import torch
    if torch.cuda.device_count() == 0:
        assert q.device_supported(0) is False


# ---------------------------------------------------------------- Q4_K ---
@pytest.mark.parametrize("n,k", [(5, 256), (17, 768), (40, 3072), (3, 8192)])
def test_q4_k_pack_unpack_roundtrip(n, k):
    w = synth.gaussian((n, k), 0.02, synth.tensor_seed(9, 3)).numpy()
    blocks = O.quantize_weights(O.Q4_K, w)
    img = q.pack_image(q.Q4_K, blocks, n, k)
    assert img.size == q.image_bytes(q.Q4_K, n, k)
    assert np.array_equal(q.unpack_image(q.Q4_K, img, n, k), blocks)


def test_q4_k_image_layout_of_one_superblock():
    # row o, superblock s: header at the scale plane + ((t*(kbp/8) + s)*16 + i)*16; sub-block j of it in the
    # code cell of block 8s + j at (t*kbp + 8s + j)*256 + 16*i, byte l = code l | code l+16 << 4
    n, k = 40, 1024  # kb = kbp = 32, sbp = 4, three tiles
    blocks = np.zeros((n, k // 256, 144), np.uint8)
    o, s = 21, 2
    blocks[o, s, :16] = np.arange(100, 116, dtype=np.uint8)  # header bytes
    codes = [(3 * i + 1) % 16 for i in range(256)]
    for p in range(4):
        for l in range(32):
            blocks[o, s, 16 + 32 * p + l] = codes[64 * p + l] | (codes[64 * p + 32 + l] << 4)
    img = q.pack_image(q.Q4_K, blocks, n, k)
    t, i = o // 16, o % 16
    plane = (3 * 32 * 256 + 255) // 256 * 256  # three tiles of 32 cells
    h = plane + ((t * 4 + s) * 16 + i) * 16
    assert list(img[h:h + 16]) == list(range(100, 116))
    for j in range(8):
        cell = (t * 32 + 8 * s + j) * 256 + 16 * i
        want = [codes[32 * j + l] | (codes[32 * j + l + 16] << 4) for l in range(16)]
        assert list(img[cell:cell + 16]) == want, j
    assert int(img.sum()) == sum(range(100, 116)) + sum(
        codes[32 * j + l] | (codes[32 * j + l + 16] << 4) for j in range(8) for l in range(16))


def test_q4_k_sizes_and_refusals():
    assert q.image_bytes(q.Q4_K, 3072, 3072) == 3072 * 3072 // 256 * 144
    assert q.image_bytes(q.Q4_K, 128256, 4096) == 128256 * 4096 // 256 * 144
    assert q.image_bytes(q.Q4_K, 16, 224) == 0 and q.image_bytes(q.Q4_K, 16, 288) == 0
    MB = 1 << 20
    st, msg = _status("qgemv_q4_k", V(A), 64, 288, V(A), 1, V(A), V(A), MB, None)
    assert st == -2 and "k=288" in msg and "256" in msg
    st, msg = _status("qgemv_q4_k", V(A), 64, 512, V(A), 17, V(A), V(A), MB, None)
    assert st == -3
    st, msg = _status("qgemv_prepared", q.Q4_K, V(A), 64, 288, V(A), MB, 4, V(A), None)
    assert st == -2
    st, msg = _status("qg_quantize_weights", q.Q4_K, V(A), 64, 288, V(A), None)
    assert st == -2
    st, msg = _status("qgemv_q4_k", V(A), 64, 512, V(A), 1, V(A), V(A), MB, None)
    assert st == -7  # a valid call: no GPU here
