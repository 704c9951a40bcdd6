"""GPU test of the allocation-free layer (rtq_rotated_qlinear_noalloc) against the layer with a
workspace (rtq_rotated_qlinear), through the C ABI: the same activation codes and the same exact
int32 sums, so the outputs agree bit for bit.  Two calls in a row, the second on a smaller input
(the static scratch keeps the first call's contents), in INT8 and codebook modes (row-major and
tiled), at the W8A8 DiT shape and at small ragged shapes."""
import numpy as np
import pytest

import rotation_then_quantize_amd as rtq
import workloads
from _helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _int8_weights(N, d, R, seed, mode):
    wh = workloads.f32_to_bf16_bits(workloads.small_case(seed, N, d, "w"))
    wq = torch.empty(((rtq.tiled_rows(N) if mode == rtq.RTQ_INT8_TILED else N), d), dtype=torch.int8, device="cuda")
    ws = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wq, ws, R, mode)
    return wq, ws


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16)) if a.dtype == torch.bfloat16 else torch.equal(a, b)


@pytest.mark.parametrize("mode", [rtq.RTQ_INT8, rtq.RTQ_INT8_TILED])
@pytest.mark.parametrize("d,N,tokens", [(4096, 16384, (4608, 1000)), (1024, 300, (517, 129)), (256, 512, (128, 33))])
def test_noalloc_int8_matches_workspace_layer(d, N, tokens, mode):
    R = rtq.Rpbh.from_seed(61, d)
    wq, ws = _int8_weights(N, d, R, 7100 + d, mode)
    for T in tokens:                       # the second call is smaller
        print(f"noalloc int8 mode={mode} d={d} N={N} T={T}", flush=True)
        xh = workloads.f32_to_bf16_bits(workloads.small_case(7200 + T + d, T, d, "t3"))
        x = to_dev(xh, "bf16")
        y_ref = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        rtq.rotated_qlinear(x, R, wq, ws, y_ref, mode)
        rtq.rotated_qlinear_noalloc(x, R, wq, ws, y, mode)
        torch.cuda.synchronize()
        assert _same_bits(y, y_ref)


@pytest.mark.parametrize("mode,bits_w", [(rtq.RTQ_CODEBOOK_I8, 4), (rtq.RTQ_CODEBOOK, 4), (rtq.RTQ_CODEBOOK_I8, 2),
                                         (rtq.RTQ_CODEBOOK_I8_TILED, 4), (rtq.RTQ_CODEBOOK_I8_TILED, 2)])
def test_noalloc_codebook_matches_workspace_layer(mode, bits_w):
    d, N = 4096, 1024
    R = rtq.Rpbh.from_seed(62, d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, 4), rtq.Codebook.for_dim(d, bits_w)
    wh = workloads.f32_to_bf16_bits(workloads.small_case(7300, N, d, "w"))
    wmode = rtq.RTQ_CODEBOOK_TILED if mode == rtq.RTQ_CODEBOOK_I8_TILED else rtq.RTQ_CODEBOOK
    wc = torch.empty(rtq.tiled_code_bytes(N, d, wmode, bits_w) or N * d * bits_w // 8, dtype=torch.uint8, device="cuda")
    wn = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wc, wn, R, wmode, cb_w, 0.0)
    for T in (2000, 257):
        print(f"noalloc codebook mode={mode} bits_w={bits_w} T={T}", flush=True)
        x = to_dev(workloads.f32_to_bf16_bits(workloads.small_case(7400 + T, T, d, "t3")), "bf16")
        y_ref = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
        y = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        rtq.rotated_qlinear(x, R, wc, wn, y_ref, mode, cb_a, cb_w)
        rtq.rotated_qlinear_noalloc(x, R, wc, wn, y, mode, cb_a, cb_w)
        torch.cuda.synchronize()
        assert _same_bits(y, y_ref)


def test_noalloc_rejects_inputs_beyond_the_scratch():
    d, N = 16384, 64
    R = rtq.Rpbh.from_seed(63, d)
    T = rtq.NOALLOC_SCRATCH_BYTES // d + 1
    x = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    ws = torch.ones(N, dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rtq.RtqError, match="static scratch"):
        rtq.rotated_qlinear_noalloc(x, R, wq, ws, y)
