"""GPU parity of the quantised products (INT8 MFMA and codebook-LUT MFMA) against the oracle.

INT8 accumulators must be bit-exact; rescaled outputs within the stated relative Frobenius bounds
(1e-4 fp32 output; 2e-2 bf16 output, the layer's tolerance) and, where both sides round the same
fp32/fp64 value to bf16, within one bf16 ulp elementwise."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import bf16_host, rel_fro, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _codes(seed, rows, d, lo=-127, hi=127):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=(rows, d)).astype(np.int8)


@pytest.mark.parametrize("T,N,d", [(130, 200, 256), (1, 1, 64), (257, 129, 128), (64, 384, 4096),
                                   (33, 70, 16384)])
def test_int8_accumulators_bit_exact(T, N, d):
    a = _codes(1 + T, T, d)
    w = _codes(2 + N, N, d)
    a_s = np.ones(T, np.float32)
    w_s = np.ones(N, np.float32)
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
    rtq.qgemm(to_dev(a), to_dev(a_s), to_dev(w), to_dev(w_s), acc, d)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), oracle.gemm_int8(a, w))


def test_int8_accumulator_extremes():
    # |acc| reaches 127^2 * d at d = 16384 (264,257,536 < 2^31)
    d = 16384
    a = np.full((3, d), 127, np.int8)
    a[1] = -127
    w = np.full((2, d), 127, np.int8)
    w[1] = -127
    acc = torch.empty((3, 2), dtype=torch.int32, device="cuda")
    rtq.qgemm(to_dev(a), to_dev(np.ones(3, np.float32)), to_dev(w), to_dev(np.ones(2, np.float32)), acc, d)
    assert np.array_equal(acc.cpu().numpy().astype(np.int64), oracle.gemm_int8(a, w))
    assert acc[0, 0].item() == 127 * 127 * d


@pytest.mark.parametrize("yt", ["f32", "bf16"])
def test_int8_rescale_epilogue(yt):
    T, N, d = 150, 300, 512
    a = _codes(7, T, d)
    w = _codes(8, N, d)
    rng = np.random.default_rng(9)
    a_s = (rng.random(T) * 0.1 + 0.01).astype(np.float32)
    w_sb = oracle.to_bf16_bits(rng.random(N) * 1e-3 + 1e-4)
    w_s = oracle.bf16_bits_to_f32(w_sb)
    y = torch.empty((T, N), dtype=torch.float32 if yt == "f32" else torch.bfloat16, device="cuda")
    rtq.qgemm(to_dev(a), to_dev(a_s), to_dev(w), to_dev(w_sb, "bf16"), y, d)
    ref = oracle.rescale_int8(oracle.gemm_int8(a, w), a_s, w_s)
    if yt == "f32":
        got = y.cpu().numpy()
        assert rel_fro(got, ref) <= 1e-6
    else:
        got = oracle.bf16_bits_to_f32(bf16_host(y))
        refb = oracle.bf16_bits_to_f32(oracle.to_bf16_bits(ref))
        assert rel_fro(got, ref) <= 2e-2
        # same value rounded on both sides: at most one bf16 ulp apart
        ulp = np.spacing(np.abs(refb).astype(np.float32)) * 65536
        assert np.all(np.abs(got - refb) <= ulp)


@pytest.mark.parametrize("bits_w", [4, 2])
def test_codebook_gemm_matches_oracle(bits_w):
    T, N, d = 140, 260, 1024
    rng = np.random.default_rng(10 + bits_w)
    qa = rng.integers(0, 16, size=(T, d)).astype(np.uint8)
    qw = rng.integers(0, 1 << bits_w, size=(N, d)).astype(np.uint8)
    cb_a = rtq.Codebook.for_dim(d, 4)
    cb_w = rtq.Codebook.for_dim(d, bits_w)
    ca = oracle.lloyd_max(4, d)["centroids"]
    cw = oracle.lloyd_max(bits_w, d)["centroids"]
    s_a = (rng.random(T) * 10 + 1).astype(np.float32)
    r_wb = oracle.to_bf16_bits(rng.random(N) + 0.5)
    r_w = oracle.bf16_bits_to_f32(r_wb)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.qgemm(to_dev(oracle.pack(qa, 4)), to_dev(s_a), to_dev(oracle.pack(qw, bits_w)), to_dev(r_wb, "bf16"), y, d,
              rtq.RTQ_CODEBOOK, cb_a, cb_w)
    ref = oracle.gemm_codebook(qa, qw, ca, cw, s_a, r_w)
    got = oracle.bf16_bits_to_f32(bf16_host(y))
    err = rel_fro(got, ref)
    # fp16 copies of the centroids (2^-11 relative rounding), fp32 sums and the bf16 output
    assert err <= 2e-2, err
    assert np.max(np.abs(got - ref)) <= 1e-2 * np.abs(ref).max()


def test_int8_full_shape_sampled():
    # W8A8 DiT shape, 4608 x 4096 -> 16384 (1152 tiles: 4.5 rounds), launched whole and in the
    # configuration the benchmark times (with the workspace: 3 whole rounds, then stream-K runs of
    # 1.5 tiles over the last 384).
    T, N, d = 4608, 16384, 4096
    a = _codes(21, T, d)
    w = _codes(22, N, d)
    rng = np.random.default_rng(23)
    rows = np.sort(rng.choice(T, 48, replace=False))
    cols = np.sort(rng.choice(N, 48, replace=False))
    rows = np.concatenate([rows, [0, T - 1]])
    cols = np.concatenate([cols, [0, N - 1]])
    ref = oracle.gemm_int8(a[rows], w[cols])
    ws = rtq.new_qgemm_workspace()
    for workspace in (None, ws):
        acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
        rtq.qgemm(to_dev(a), to_dev(np.ones(T, np.float32)), to_dev(w), to_dev(np.ones(N, np.float32)), acc, d,
                  workspace=workspace)
        torch.cuda.synchronize()
        got = acc.cpu().numpy()[np.ix_(rows, cols)].astype(np.int64)
        assert np.array_equal(got, ref)


# ---------------------------------------------------------------- K-split of the last round

@pytest.mark.parametrize("T,N,d", [(130, 200, 256), (257, 129, 128), (64, 384, 4096), (33, 70, 16384),
                                   (300, 700, 2048), (4608, 4096, 8192), (3328, 5376, 4096), (4608, 4096, 1024),
                                   (2304, 8448, 2048), (4608, 8192, 4096), (4100, 4100, 1024)])
def test_int8_ksplit_accumulators_bit_exact(T, N, d):
    # with a workspace a last round that leaves most compute units idle is shared along d; the
    # pieces add exactly in int32.  On 256 CUs: d < 1024 never shares; with no full round, one
    # tile at d = 4096 / 16384 splits 4 / 8 ways and 300 x 700 x 2048 is 6 tiles split 2 ways.
    # After a full round, stream-K: every block runs an equal run of K stages across tile edges,
    # a tile meeting at most two runs.  4608 x 4096 x 8192 is 288 tiles (runs of 1.125 tiles);
    # 3328 x 5376 is 273 tiles, dealt unevenly over the 8 XCDs (35 on the first, 34 on the
    # others); 4608 x 4096 x 1024 has runs of 18 stages; 2304 x 8448 is 297 tiles; 4608 x 8192 is
    # 576 tiles: one whole round, then 320 tiles shared; 4100 x 4100 is 289 tiles with ragged
    # last rows and columns (N % 8 != 0: per-element stores).
    a = _codes(11 + T, T, d)
    w = _codes(12 + N, N, d)
    ws = rtq.new_qgemm_workspace()
    ws[:-_counter_bytes()] = 0x5A   # partial tiles: any contents; the counters start at zero
    acc = torch.empty((T, N), dtype=torch.int32, device="cuda")
    ones_t, ones_n = to_dev(np.ones(T, np.float32)), to_dev(np.ones(N, np.float32))
    da, dw = to_dev(a), to_dev(w)
    rows = np.arange(T) if T * N <= 1 << 17 else np.sort(np.random.default_rng(3).choice(T, 40, replace=False))
    ref = oracle.gemm_int8(a[rows], w)
    for _ in range(3):   # the same workspace again: each launch leaves its counters at zero
        acc.fill_(0)
        rtq.qgemm(da, ones_t, dw, ones_n, acc, d, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)
        assert not ws[-_counter_bytes():].any()


@pytest.mark.parametrize("yt", ["f32", "bf16"])
@pytest.mark.parametrize("T,N,d", [(300, 700, 2048), (3328, 5376, 4096), (4100, 4100, 1024)])
def test_ksplit_outputs_equal_unsplit(yt, T, N, d):
    # exact int32 sums, then the same epilogue: split and unsplit products agree bit for bit
    # (6 tiles split 2 ways; 273 and 289 tiles shared by stream-K runs, the latter with ragged
    # edges and N % 8 != 0)
    a = _codes(21, T, d)
    w = _codes(22, N, d)
    rng = np.random.default_rng(23)
    a_s = to_dev((rng.random(T) * 0.1 + 0.01).astype(np.float32))
    w_s = to_dev(oracle.to_bf16_bits(rng.random(N) * 0.1 + 0.01), "bf16")
    dt = torch.float32 if yt == "f32" else torch.bfloat16
    y0 = torch.empty((T, N), dtype=dt, device="cuda")
    y1 = torch.empty((T, N), dtype=dt, device="cuda")
    rtq.qgemm(to_dev(a), a_s, to_dev(w), w_s, y0, d)
    ws = rtq.new_qgemm_workspace()
    rtq.qgemm(to_dev(a), a_s, to_dev(w), w_s, y1, d, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0.view(torch.int16) if yt == "bf16" else y0.view(torch.int32),
                       y1.view(torch.int16) if yt == "bf16" else y1.view(torch.int32))


def _counter_bytes():
    # the split region ends with two 8-byte arrival counters per block slot
    nbytes = rtq.qgemm_workspace()
    return 16 * (nbytes // (2 * (256 * 256 * 4 + 8)))


def test_split_counters_left_zero_and_layer_workspace_any_contents():
    # rtq_qgemm_ws: a zero-filled workspace stays reusable, since the block that finishes a shared
    # tile resets its counter; partial tiles may hold anything.  rtq_rotated_qlinear: its workspace
    # may hold anything at all (the quantiser launch zeroes the product's counters), here int32
    # partial-tile-like data with the counter words set to publication-like values (1, 2, 4, 5 ...).
    T, N, d = 4608, 4096, 4096                    # 288 tiles: all shared by stream-K runs
    a = to_dev(_codes(31, T, d))
    w = to_dev(_codes(32, N, d))
    ones_t, ones_n = to_dev(np.ones(T, np.float32)), to_dev(np.ones(N, np.float32))
    acc0 = torch.empty((T, N), dtype=torch.int32, device="cuda")
    rtq.qgemm(a, ones_t, w, ones_n, acc0, d)
    ws = rtq.new_qgemm_workspace()
    ws[:-_counter_bytes()].view(torch.int32).copy_(torch.randint(-1000, 1000, ((ws.numel() - _counter_bytes()) // 4,),
                                                                 dtype=torch.int32, device="cuda"))
    for _ in range(3):
        acc1 = torch.full((T, N), -1, dtype=torch.int32, device="cuda")
        rtq.qgemm(a, ones_t, w, ones_n, acc1, d, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(acc0, acc1)
        assert not ws[-_counter_bytes():].any()
    # the layer: any workspace contents
    R = rtq.Rpbh.from_seed(33, d)
    xh = to_dev(workloads.f32_to_bf16_bits(workloads.small_case(3301, T, d, "t3")), "bf16")
    wq = torch.empty((N, d), dtype=torch.int8, device="cuda")
    wsc = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(workloads.f32_to_bf16_bits(workloads.small_case(3302, N, d, "w")), "bf16"), wq, wsc, R,
                      rtq.RTQ_INT8)
    need = rtq.rotated_qlinear_workspace(T, d)
    y0 = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    rtq.rotated_qlinear(xh, R, wq, wsc, y0, workspace=torch.zeros(need, dtype=torch.uint8, device="cuda"))
    junk = torch.randint(-1000, 1000, ((need + 3) // 4,), dtype=torch.int32, device="cuda")
    junk_ws = junk.view(torch.uint8)[:need]
    cw = junk_ws[-_counter_bytes():].view(torch.int64)
    cw.copy_(torch.arange(cw.numel(), device="cuda", dtype=torch.int64) % 8)
    for _ in range(2):
        y1 = torch.full((T, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        rtq.rotated_qlinear(xh, R, wq, wsc, y1, workspace=junk_ws)
        torch.cuda.synchronize()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
        cw.fill_(5)
