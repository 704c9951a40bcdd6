"""End-to-end GPU parity of the rotated quantised linear layer (offline weight rotate-quantise +
online rotate-quantise-product) against the oracle, at small shapes that span several tiles and a
ragged tail, and at the DiT shapes on sampled rows/columns the oracle computes one by one."""
import math

import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
import _dit_cases as dit_cases
from _helpers import (bf16_host, codebook_mismatches_allowed, dense_pi, int8_mismatches_allowed, rel_fro, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _gpu_weights_int8(w_dev, R, scale_dtype):
    N, d = w_dev.shape
    codes = torch.empty((N, d), dtype=torch.int8, device="cuda")
    scale = torch.empty(N, dtype=scale_dtype, device="cuda")
    rtq.quantize_rows(w_dev, codes, scale, R, rtq.RTQ_INT8)
    return codes, scale


def test_tiny_fp32_layer_end_to_end():
    # d_in=256, d_out=512, 128 tokens, fp32; outlier columns/channels; RPBH with 4 blocks.
    inp = workloads.tiny_inputs()
    x, w = inp["x"], inp["w"]
    d = 256
    R = rtq.Rpbh.from_seed(inp["rpbh_seed"], d)
    wq, ws = _gpu_weights_int8(to_dev(w), R, torch.float32)
    y = torch.empty((128, 512), dtype=torch.float32, device="cuda")
    rtq.rotated_qlinear(to_dev(x), R, wq, ws, y)
    torch.cuda.synchronize()
    pi = dense_pi(inp["rpbh_seed"], d)
    wo = oracle.weights_int8(w, pi, False)
    assert np.array_equal(ws.cpu().numpy(), wo["scale"])
    assert int8_mismatches_allowed(wq.cpu().numpy(), wo["q"], wo["pre"])[1] == 0
    ref = oracle.qlinear_int8(x, pi, wo)["y"]
    assert rel_fro(y.cpu().numpy(), ref) <= 1e-4
    # method sanity (not parity): the rotated W8A8 layer is closer to W x than plain W8A8
    exact = oracle.matmul_f64(x, w)
    qa, sa, _ = oracle.quantize_int8(x, False)
    qw, sw, _ = oracle.quantize_int8(w, False)
    plain = oracle.rescale_int8(oracle.gemm_int8(qa, qw), sa, sw)
    assert rel_fro(y.cpu().numpy(), exact) < 0.5 * rel_fro(plain, exact)


@pytest.mark.parametrize("T,N,d", [(300, 384, 4096), (129, 130, 1024)])
def test_w8a8_bf16_layer_small(T, N, d):
    xf = workloads.small_case(600 + d, T, d, "t3")
    wf = workloads.small_case(601 + d, N, d, "w")
    xh, wh = workloads.f32_to_bf16_bits(xf), workloads.f32_to_bf16_bits(wf)
    xf, wf = workloads.bf16_bits_to_f32(xh), workloads.bf16_bits_to_f32(wh)
    seed = 41
    R = rtq.Rpbh.from_seed(seed, d)
    wq, ws = _gpu_weights_int8(to_dev(wh, "bf16"), R, torch.bfloat16)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wq, ws, y)
    torch.cuda.synchronize()
    pi = dense_pi(seed, d)
    wo = oracle.weights_int8(wf, pi, True)
    got_ws = workloads.bf16_bits_to_f32(bf16_host(ws))
    assert np.array_equal(got_ws, wo["scale"])
    assert int8_mismatches_allowed(wq.cpu().numpy(), wo["q"], wo["pre"])[1] == 0
    ref = oracle.qlinear_int8(xf, pi, wo)["y"]
    got = workloads.bf16_bits_to_f32(bf16_host(y))
    assert rel_fro(got, ref) <= 2e-2
    # codes agree, so y differs only by fp32-vs-fp64 epilogue rounding: <= 1 bf16 ulp per element
    refb = oracle.bf16_bits_to_f32(oracle.to_bf16_bits(ref))
    ulp = np.spacing(np.abs(refb).astype(np.float32)) * 65536
    assert np.mean(np.abs(got - refb) <= ulp) > 0.999


@pytest.mark.parametrize("bits_w,T,N,d", [(4, 200, 256, 4096), (2, 70, 130, 16384), (4, 33, 65, 256)])
def test_codebook_layer_small(bits_w, T, N, d):
    xf = workloads.small_case(700 + d, T, d, "t3")
    wf = workloads.small_case(701 + d, N, d, "w")
    xh, wh = workloads.f32_to_bf16_bits(xf), workloads.f32_to_bf16_bits(wf)
    xf, wf = workloads.bf16_bits_to_f32(xh), workloads.bf16_bits_to_f32(wh)
    seed = 43
    R = rtq.Rpbh.from_seed(seed, d)
    cb_a = rtq.Codebook.for_dim(d, 4)
    cb_w = rtq.Codebook.for_dim(d, bits_w)
    wcodes = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wcodes, wnorm, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK, 4), dtype=torch.uint8, device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wcodes, wnorm, y, rtq.RTQ_CODEBOOK, cb_a, cb_w, workspace=ws)
    torch.cuda.synchronize()
    pi = dense_pi(seed, d)
    ocb_a, ocb_w = oracle.lloyd_max(4, d), oracle.lloyd_max(bits_w, d)
    wo = oracle.weights_codebook(wf, pi, ocb_w, bits_w)
    got_codes = oracle.unpack(wcodes.cpu().numpy(), d, bits_w)
    assert codebook_mismatches_allowed(got_codes, wo["codes"], wo["u"], ocb_w["boundaries"], d)[1] == 0
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(wnorm)), wo["norm"])
    out = oracle.qlinear_codebook(xf, pi, wo, ocb_a, ocb_w, 4)
    # the workspace holds the activation codes and norms
    a_codes = oracle.unpack(ws[:T * d // 2].view(T, d // 2).cpu().numpy(), d, 4)
    assert codebook_mismatches_allowed(a_codes, out["act"]["codes"], out["act"]["u"], ocb_a["boundaries"], d)[1] == 0
    off = ((T * d // 2 + 255) // 256) * 256
    a_norm = ws[off:off + 4 * T].view(torch.float32).cpu().numpy()
    assert np.array_equal(a_norm, out["act"]["norm"])
    got = workloads.bf16_bits_to_f32(bf16_host(y))
    assert rel_fro(got, out["y"]) <= 2e-2


# ---------------------------------------------------------------- DiT shapes, sampled

def test_w8a8_dit_shape_sampled():
    # 4608 tokens x 4096 -> 16384, bf16 in/out, weights = the DiT MLP-up linear, launched exactly as
    # the benchmark does (rotated_qlinear on the full tensors, with the K-split workspace: three
    # whole rounds of tiles, then stream-K runs over the last 384).  64 tokens x 256 channels are
    # compared, covering every output tile (each tile's first and last row and column).
    d, N = workloads.DIT_HIDDEN, workloads.DIT_MLP
    xh, wh = workloads.dit_activations_bf16(d), workloads.dit_weight_bf16("mlp_up")
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    wq, ws = _gpu_weights_int8(to_dev(wh, "bf16"), R, torch.bfloat16)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(rtq.rotated_qlinear_workspace(T, d), dtype=torch.uint8, device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wq, ws, y, workspace=work)
    torch.cuda.synchronize()
    ref = dit_cases.w8a8_sample()
    rows, cols, wo, ao = ref["rows"], ref["cols"], ref["wo"], ref["ao"]
    # weight codes and scales of the sampled rows
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(ws))[cols], wo["scale"])
    w_codes = wq.cpu().numpy()[cols]
    assert int8_mismatches_allowed(w_codes, wo["q"], wo["pre"])[1] == 0
    # activation codes and scales (workspace) of the sampled tokens
    a_codes = work[:T * d].view(T, d).cpu().numpy().view(np.int8)[rows]
    a_scale = work[T * d:T * d + 4 * T].view(torch.float32).cpu().numpy()[rows]
    assert np.array_equal(a_scale, ao["scale"])
    assert int8_mismatches_allowed(a_codes, ao["q"], ao["pre"])[1] == 0
    got = workloads.bf16_bits_to_f32(bf16_host(y))[np.ix_(rows, cols)]
    assert rel_fro(got, ref["y"]) <= 2e-2
    # element by element: where a token's and a channel's codes equal the oracle's, the two sides
    # round the same exact accumulator to bf16 (fp32 vs fp64 epilogue): at most one bf16 ulp apart
    same = np.all(a_codes == ao["q"], axis=1)[:, None] & np.all(w_codes == wo["q"], axis=1)[None, :]
    assert same.mean() > 0.9
    assert np.all(dit_cases.bf16_within_one_ulp(got, ref["y"])[same])


@pytest.mark.parametrize("variant", ["w4a4", "w2a4"])
def test_codebook_dit_shape_sampled(variant):
    # the codebook layers on the fp16-LUT product (RTQ_CODEBOOK), full launches; 64 tokens x 256
    # channels covering every output tile
    ref = dit_cases.codebook_sample(variant)
    d, N, bits_w, bits_a = ref["d"], ref["N"], ref["bits_w"], ref["bits_a"]
    _, _, _, _, wgen = dit_cases.CODEBOOK_VARIANTS[variant]
    xh, wh = workloads.dit_activations_bf16(d), wgen()
    T = xh.shape[0]
    R = rtq.Rpbh.from_seed(workloads.RPBH_SEED[d], d)
    cb_a, cb_w = rtq.Codebook.for_dim(d, bits_a), rtq.Codebook.for_dim(d, bits_w)
    wcodes = torch.empty((N, d * bits_w // 8), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), wcodes, wnorm, R, rtq.RTQ_CODEBOOK, cb_w, 0.0)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    work = torch.empty(rtq.rotated_qlinear_workspace(T, d, rtq.RTQ_CODEBOOK, bits_a), dtype=torch.uint8,
                       device="cuda")
    rtq.rotated_qlinear(to_dev(xh, "bf16"), R, wcodes, wnorm, y, rtq.RTQ_CODEBOOK, cb_a, cb_w, workspace=work)
    torch.cuda.synchronize()
    rows, cols, wo, ao = ref["rows"], ref["cols"], ref["wo"], ref["ao"]
    ocb_a, ocb_w = ref["ocb_a"], ref["ocb_w"]
    got_w = oracle.unpack(wcodes.cpu().numpy()[cols], d, bits_w)
    assert codebook_mismatches_allowed(got_w, wo["codes"], wo["u"], ocb_w["boundaries"], d)[1] == 0
    assert np.array_equal(workloads.bf16_bits_to_f32(bf16_host(wnorm))[cols], wo["norm"])
    a_codes = oracle.unpack(work[:T * d // 2].view(T, d // 2).cpu().numpy()[rows], d, bits_a)
    assert codebook_mismatches_allowed(a_codes, ao["codes"], ao["u"], ocb_a["boundaries"], d)[1] == 0
    off = ((T * d // 2 + 255) // 256) * 256
    assert np.array_equal(work[off:off + 4 * T].view(torch.float32).cpu().numpy()[rows], ao["norm"])
    got = workloads.bf16_bits_to_f32(bf16_host(y))[np.ix_(rows, cols)]
    assert rel_fro(got, ref["y"]) <= 2e-2
    # fp16 centroid copies (2^-11 relative) and fp32 sums: every sampled element stays close
    scale = np.abs(ref["y"]).max()
    assert np.max(np.abs(got - ref["y"])) <= 1e-2 * scale
