"""GPU parity on the quantiser's edge cases, against the oracle.

  * Tiny rows: the INT8 kernels divide without a division per element while the row's max |x'|
    is at least 2^-103 and take IEEE division below that (subnormal quotients could round
    differently); the asymmetric kernels switch at hi - lo < 2^-100.  Rows scaled down to and
    into the bf16 subnormal range, mixed with ordinary rows in one launch, must still match.
  * Exact ties: rows whose rotated values land exactly on k + 1/2 in units of the scale (INT8,
    round half to even) or exactly on a codebook boundary (the code of the lower cell).  The
    input is x = Pi^T y for a chosen rotated row y, built so that x is exact in bf16 and Pi x = y
    exactly; no allowance is taken there: codes must be equal.
  * Codebooks whose boundaries crowd one cell of the kernels' boundary grid: 64-level codes are
    then found by binary search over the row's thresholds (rows of >= 64 blocks), or by counting.
Readings (OrbitQuant article, sections 2.1-2.2; round half to even and ties to the lower cell are
the standardised rounding of its section 6.3)."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import (bf16_host, codebook_mismatches_allowed, codes_of, dense_pi, int8_mismatches_allowed,
                      int8_table, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SEED = 77


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _bf16_rows(xf):
    xh = workloads.f32_to_bf16_bits(xf)
    return xh, workloads.bf16_bits_to_f32(xh)


def _tiny_rows(d, seed):
    """Ordinary Student-t rows interleaved with the same rows scaled by 2^-e, e from 100 to 131
    (the last ones are bf16 subnormals), and an all-zero row."""
    base = workloads.small_case(seed, 12, d, "t3")
    rows = []
    for i, e in enumerate([0, 100, 0, 103, 106, 0, 112, 118, 0, 124, 128, 131]):
        rows.append(base[i] * np.float32(2.0 ** -e))
    rows.append(np.zeros(d, np.float32))
    return _bf16_rows(np.stack(rows))


@pytest.mark.parametrize("d", [256, 4096, 16384])
@pytest.mark.parametrize("scale_bf16", [False, True])
def test_int8_tiny_rows(d, scale_bf16):
    xh, xf = _tiny_rows(d, 900 + d)
    rows = xh.shape[0]
    R = rtq.Rpbh.from_seed(SEED, d)
    q = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.bfloat16 if scale_bf16 else torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), q, s, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    qo, so, pre = oracle.quantize_int8(rot, scale_bf16)
    got_s = workloads.bf16_bits_to_f32(bf16_host(s)) if scale_bf16 else s.cpu().numpy()
    assert np.array_equal(got_s, so)
    assert int8_mismatches_allowed(q.cpu().numpy(), qo, pre)[1] == 0


@pytest.mark.parametrize("d", [256, 4096, 16384])
def test_int8_asym_tiny_rows(d):
    xh, xf = _tiny_rows(d, 950 + d)
    rows = xh.shape[0]
    R = rtq.Rpbh.from_seed(SEED, d)
    q = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    z = torch.empty(rows, dtype=torch.int32, device="cuda")
    cs = torch.empty(rows, dtype=torch.int32, device="cuda")
    rtq.quantize_rows_asym(to_dev(xh, "bf16"), q, s, z, cs, R)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    qo, so, zo, csum, pre = oracle.quantize_int8_asym(rot, False)
    assert np.array_equal(s.cpu().numpy(), so)
    assert np.array_equal(z.cpu().numpy(), zo)
    qg = q.cpu().numpy()
    # codes: equal, or one step apart at a rounding boundary of the pre-offset quotient
    assert int8_mismatches_allowed(qg.astype(np.int32) - zo[:, None], qo.astype(np.int32) - zo[:, None], pre)[1] == 0
    assert np.array_equal(cs.cpu().numpy().astype(np.int64), qg.astype(np.int64).sum(axis=1))


@pytest.mark.parametrize("d", [256, 4096, 16384])
def test_codebook_tiny_rows(d):
    # weights (eps = 0: the direction of a tiny row is still quantised) and activations (eps =
    # 1e-8 swamps a tiny norm: u ~ 0)
    xh, xf = _tiny_rows(d, 980 + d)
    rows = xh.shape[0]
    R = rtq.Rpbh.from_seed(SEED, d)
    cbo = oracle.lloyd_max(4, d)
    cb = rtq.Codebook.for_dim(d, 4)
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    for weight in (True, False):
        eps = 0.0 if weight else 1e-8
        c = torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty(rows, dtype=torch.bfloat16 if weight else torch.float32, device="cuda")
        rtq.quantize_rows(to_dev(xh, "bf16"), c, s, R, rtq.RTQ_CODEBOOK, cb, eps)
        torch.cuda.synchronize()
        co, so, u = oracle.quantize_codebook(rot, cbo["boundaries"], weight, eps)
        got_s = workloads.bf16_bits_to_f32(bf16_host(s)) if weight else s.cpu().numpy()
        assert np.array_equal(got_s, so), weight
        got = oracle.unpack(c.cpu().numpy(), d, 4)
        assert codebook_mismatches_allowed(got, co, u, cbo["boundaries"], d)[1] == 0, weight


# ---------------------------------------------------------------- exact ties

def _tie_rows_int8(d, rows, seed):
    """Rotated rows y with max |y| = 1016 = 127 * 8 (scale 8 exactly) alone in its block and, in
    the other blocks, up to 4 entries of +-(8k + 4), whose quotients k + 1/2 are ties; the input
    x = Pi^T y has half-integer entries of magnitude at most 127 (exact in bf16)."""
    rng = np.random.default_rng(seed)
    y = np.zeros((rows, d), np.float64)
    nb = d // 64
    for r in range(rows):
        big = rng.integers(nb)
        y[r, big * 64 + rng.integers(64)] = 1016.0 * (1 if rng.random() < 0.5 else -1)
        for b in range(nb):
            if b == big:
                continue
            slots = rng.choice(64, rng.integers(1, 5), replace=False)
            k = rng.integers(0, 16, size=len(slots))
            sg = np.where(rng.random(len(slots)) < 0.5, -1.0, 1.0)
            y[r, b * 64 + slots] = sg * (8 * k + 4)
    x = (y @ dense_pi(SEED, d)).astype(np.float32)           # rows of Pi^T y
    assert np.all(np.abs(x) <= 127) and np.all(x * 2 == np.round(x * 2))
    assert np.array_equal(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)), x)
    return y, x


@pytest.mark.parametrize("d", [256, 4096, 16384])
@pytest.mark.parametrize("xt", ["bf16", "f32"])
def test_int8_exact_ties_round_half_even(d, xt):
    rows = 6
    y, xf = _tie_rows_int8(d, rows, 400 + d)
    R = rtq.Rpbh.from_seed(SEED, d)
    xd = to_dev(workloads.f32_to_bf16_bits(xf), "bf16") if xt == "bf16" else to_dev(xf)
    q = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(xd, q, s, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    assert np.all(workloads.bf16_bits_to_f32(bf16_host(s)) == 8.0)
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    assert np.array_equal(rot.astype(np.float64), y)   # the oracle sees the ties exactly
    qo, so, pre = oracle.quantize_int8(rot, True)
    expect = np.rint(y / 8.0)                          # numpy rint: half to even
    assert np.array_equal(qo.astype(np.float64), expect)
    assert np.array_equal(q.cpu().numpy(), qo)         # no allowance at exact ties


# custom 4-bit codebook whose boundaries are short binary fractions, so rotated values can sit on them
TIE_BOUNDS = np.array([-0.5, -0.375, -0.25, -0.1875, -0.125, -0.0625, -0.03125, 0.0, 0.03125, 0.0625, 0.125,
                       0.1875, 0.25, 0.375, 0.5], np.float32)
TIE_CENTS = np.array([-0.625, -0.4375, -0.3125, -0.21875, -0.15625, -0.09375, -0.046875, -0.015625, 0.015625,
                      0.046875, 0.09375, 0.15625, 0.21875, 0.3125, 0.4375, 0.625], np.float32)


def _tie_rows_codebook(d, rows, seed):
    """Rotated rows y with one nonzero entry per block (so x = Pi^T y is +-y_b / 8 on the block's
    64 columns) and norm ||y|| a power of two, so u = y / ||y|| is exactly 0, +-1/16, +-1/8, +-1/4
    or +-1/2: boundaries of TIE_BOUNDS."""
    rng = np.random.default_rng(seed)
    nb = d // 64
    y = np.zeros((rows, d), np.float64)
    for r in range(rows):
        if nb == 4:
            mags = [2.0, 2.0, 2.0, 2.0]                    # ||y|| = 4: u = +-1/2
        elif nb == 64:
            mags = [2.0] * 48 + [4.0] * 4 + [0.0] * 12     # ||y|| = 16: u = +-1/8, +-1/4, 0
        else:
            mags = [2.0] * 192 + [4.0] * 16 + [0.0] * 48   # ||y|| = 32: u = +-1/16, +-1/8, 0
        mags = rng.permutation(np.array(mags))
        for b in range(nb):
            y[r, b * 64 + rng.integers(64)] = mags[b] * (1 if rng.random() < 0.5 else -1)
    x = y @ dense_pi(SEED, d)
    return y, x.astype(np.float32)


@pytest.mark.parametrize("d", [256, 4096, 16384])
@pytest.mark.parametrize("mode", ["packed", "int8"])
def test_codebook_exact_ties_take_the_lower_cell(d, mode):
    rows = 5
    y, xf = _tie_rows_codebook(d, rows, 500 + d)
    assert np.array_equal(workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(xf)), xf)
    R = rtq.Rpbh.from_seed(SEED, d)
    cb = rtq.Codebook(4, to_dev(TIE_CENTS), to_dev(TIE_BOUNDS))
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    assert np.array_equal(rot.astype(np.float64), y)
    for weight in (True, False):
        eps = 0.0 if weight else 1e-8
        co, so, u = oracle.quantize_codebook(rot, TIE_BOUNDS, weight, eps)
        assert np.isin(u, TIE_BOUNDS).mean() > 0.7           # most values sit exactly on a boundary
        s = torch.empty(rows, dtype=torch.bfloat16 if weight else torch.float32, device="cuda")
        if mode == "packed":
            c = torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda")
            rtq.quantize_rows(to_dev(workloads.f32_to_bf16_bits(xf), "bf16"), c, s, R, rtq.RTQ_CODEBOOK, cb, eps)
            torch.cuda.synchronize()
            got = oracle.unpack(c.cpu().numpy(), d, 4)
        else:
            c = torch.empty((rows, d), dtype=torch.int8, device="cuda")
            rtq.quantize_rows(to_dev(workloads.f32_to_bf16_bits(xf), "bf16"), c, s, R, rtq.RTQ_CODEBOOK_I8, cb, eps)
            torch.cuda.synchronize()
            got = codes_of(c.cpu().numpy(), int8_table(TIE_CENTS)[1])
        got_s = workloads.bf16_bits_to_f32(bf16_host(s)) if weight else s.cpu().numpy()
        assert np.array_equal(got_s, so)
        assert np.array_equal(got.astype(np.int64), co.astype(np.int64)), (weight, int((got != co).sum()))


# ---------------------------------------------------------------- crowded 64-level boundaries

@pytest.mark.parametrize("d", [1024, 4096, 16384])
def test_six_bit_codes_without_the_grid(d):
    # Lloyd-Max 64-level boundaries with boundary 32 moved to within 0.3 grid cells of boundary
    # 31 (the one at 0): one cell would hold two boundaries, so the kernels leave the grid and
    # search the row's thresholds (binary search for rows of >= 64 blocks, counting below)
    cbo = oracle.lloyd_max(6, d)
    bounds = cbo["boundaries"].copy()
    tmax = max(abs(float(bounds[0])), abs(float(bounds[-1])))
    assert bounds[31] == 0.0
    bounds[32] = np.float32(0.3 * tmax / 100.0)
    assert np.all(np.diff(bounds) > 0)
    cents = cbo["centroids"]
    rows = 24
    xh, xf = _bf16_rows(workloads.small_case(1200 + d, rows, d, "t3"))
    R = rtq.Rpbh.from_seed(SEED, d)
    cb = rtq.Codebook(6, to_dev(cents), to_dev(bounds))
    c = torch.empty((rows, d), dtype=torch.int8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    rtq.quantize_rows(to_dev(xh, "bf16"), c, s, R, rtq.RTQ_CODEBOOK_I8, cb, 1e-8)
    torch.cuda.synchronize()
    _, rot = oracle.rotate(xf, dense_pi(SEED, d))
    co, so, u = oracle.quantize_codebook(rot, bounds, False, 1e-8)
    assert np.array_equal(s.cpu().numpy(), so)
    got = codes_of(c.cpu().numpy(), int8_table(cents)[1])
    assert codebook_mismatches_allowed(got, co, u, bounds, d)[1] == 0
    # the moved boundary is really used: some values fall between boundaries 31 and 32
    assert np.any(co == 32)
