"""Pins of the CPU oracle to facts outside itself (closed forms, invariants,
textbook/library special cases, published reference streams, brute force).

Each test names the page passage (title + section) whose statement it pins.
  [OQ]  OrbitQuant article (hotelren.com/news/3376620)
  [CR1] "INT8旋转量化是什么？图像生成模型轻量化全解" (cloud.baidu.com/article/9430339)
  [CR2] "量化旋转主模型是什么？一文读懂低比特图像生成模型" (cloud.baidu.com/article/9432521)
"""
import itertools
import math

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats
import torch

import oracle
import workloads

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ---------------------------------------------------------------- generator

def test_splitmix64_reference_stream():
    # Reference outputs of SplitMix64 (Steele/Lea/Flood 2014; Vigna's
    # public-domain splitmix64.c): seed 1234567 and seed 0.
    assert list(oracle.splitmix64(1234567, 5)) == [
        6457827717110365317, 3203168211198807973, 9817491932198370423,
        4593380528125082431, 16408922859458223821]
    assert int(oracle.splitmix64(0, 1)[0]) == 0xE220A8397B1DCDAF


def test_descriptor_is_permutation_and_rademacher():
    # [OQ] 2.3: P_pi a permutation matrix, D_i diagonal with +-1 entries.
    for d in (64, 256, 4096, 16384):
        perm, signs = oracle.rpbh_descriptor(workloads.RPBH_SEED.get(d, 7), d)
        assert np.array_equal(np.sort(perm), np.arange(d))
        assert set(np.unique(signs)) <= {-1, 1}
        if d >= 4096:
            assert abs(signs.astype(np.float64).mean()) < 5.0 / math.sqrt(d)
            assert (perm != np.arange(d)).mean() > 0.99


def test_fisher_yates_uniform_over_small_group():
    # A uniformly random permutation ([OQ] 2.3 "random permutation"): every
    # one of the 24 permutations of 4 items appears about equally often.
    counts = {}
    n = 24000
    for seed in range(n):
        p, _ = oracle.rpbh_descriptor(seed, 4)
        counts[tuple(p)] = counts.get(tuple(p), 0) + 1
    assert len(counts) == 24
    chi2 = sum((c - n / 24) ** 2 / (n / 24) for c in counts.values())
    assert chi2 < scipy.stats.chi2.ppf(0.999, 23)


def test_signs_match_descriptor_stream_layout():
    # The descriptor consumes d-1 draws for the shuffle then d draws for the
    # signs (top bit); check against the published stream directly.
    d = 64
    stream = oracle.splitmix64(99, 2 * d - 1)
    _, signs = oracle.rpbh_descriptor(99, d)
    expect = np.where((stream[d - 1:] >> np.uint64(63)) == 1, -1, 1)
    assert np.array_equal(signs, expect)


# ---------------------------------------------------------------- dense Pi

def test_identity_descriptor_gives_sylvester_hadamard():
    # d = h = 64, pi = identity, all signs +1: Pi is H_64 / 8 (textbook
    # Sylvester matrix, scipy.linalg.hadamard).
    pi = oracle.rpbh_dense(64, 64, np.arange(64, dtype=np.int32), np.ones(64, np.int8))
    assert np.array_equal(pi, scipy.linalg.hadamard(64) / 8.0)
    # Pi e_0 = (1/8) 1 and H H^T = 64 I
    assert np.array_equal(pi[:, 0], np.full(64, 1 / 8.0))


def test_dense_pi_equals_its_factorisation():
    # [OQ] 2.3: Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi, built here
    # from library pieces: block_diag, hadamard, diag, and the gather
    # permutation matrix (row j is e_{perm[j]}).
    d, h = 256, 64
    perm, signs = oracle.rpbh_descriptor(1003, d)
    blocks = [scipy.linalg.hadamard(h) @ np.diag(signs[i * h:(i + 1) * h].astype(np.float64)) / 8.0
              for i in range(d // h)]
    P = np.eye(d)[perm]
    expect = scipy.linalg.block_diag(*blocks) @ P
    assert np.array_equal(oracle.rpbh_dense(d, h, perm, signs), expect)
    # and P_pi acts as a gather
    x = np.arange(d, dtype=np.float64)
    assert np.array_equal(P @ x, x[perm])


@pytest.mark.parametrize("d", [64, 256, 1024])
def test_pi_is_exactly_orthogonal(d):
    # Orthogonality ([CR2] 4: an orthogonal rotation; [OQ] 2.2 needs
    # Pi^T Pi = I for the cancellation).  Entries are +-1/8, so the products
    # are exact in fp64.
    perm, signs = oracle.rpbh_descriptor(11 + d, d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    assert np.array_equal(pi.T @ pi, np.eye(d))
    assert np.array_equal(pi @ pi.T, np.eye(d))


def test_rotation_preserves_norm_and_singular_values():
    # [CR2] 4: an orthogonal transform keeps singular values.
    d = 256
    perm, signs = oracle.rpbh_descriptor(5, d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    x = workloads.small_case(17, 32, d)
    x64, _ = oracle.rotate(x, pi)
    assert np.allclose(np.linalg.norm(x64, axis=1), np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-13)
    w = workloads.small_case(18, 48, d, "w")
    w64, _ = oracle.rotate(w, pi)
    s0 = np.linalg.svd(w.astype(np.float64), compute_uv=False)
    s1 = np.linalg.svd(w64, compute_uv=False)
    assert np.allclose(s0, s1, rtol=1e-10)


def _textbook_block_fwht(v, h=64):
    """Plain radix-2 butterflies per h-block, in fp64 (a different algorithm
    from the dense product; used only to pin the dense product)."""
    v = np.array(v, np.float64).copy()
    rows, d = v.shape
    v = v.reshape(rows, d // h, h)
    span = 1
    while span < h:
        for start in range(0, h, 2 * span):
            a = v[:, :, start:start + span].copy()
            b = v[:, :, start + span:start + 2 * span].copy()
            v[:, :, start:start + span] = a + b
            v[:, :, start + span:start + 2 * span] = a - b
        span *= 2
    return v.reshape(rows, d) / math.sqrt(h)


@pytest.mark.parametrize("d", [256, 4096])
def test_fast_transform_equals_dense_bit_exactly_on_integers(d):
    # [OQ] 2.3: the O(d log h) block transform computes the same Pi x as the
    # dense matrix.  On small integers all partial sums are exact.
    perm, signs = oracle.rpbh_descriptor(23, d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    rng = np.random.default_rng(0)
    x = rng.integers(-1000, 1001, size=(4, d)).astype(np.float32)
    _, dense32 = oracle.rotate(x, pi)
    fast = _textbook_block_fwht(x[:, perm] * signs[None, :].astype(np.float64))
    assert np.array_equal(dense32, fast.astype(np.float32))
    # random real inputs agree to fp64 rounding
    xr = workloads.small_case(3, 4, d)
    d64, _ = oracle.rotate(xr, pi)
    fr = _textbook_block_fwht(xr[:, perm].astype(np.float64) * signs[None, :])
    assert np.max(np.abs(d64 - fr)) <= 1e-12 * np.max(np.abs(fr))


def test_inverse_rotation_undoes_rotation():
    d = 256
    perm, signs = oracle.rpbh_descriptor(31, d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    x = workloads.small_case(4, 8, d)
    x64, _ = oracle.rotate(x, pi)
    back64, _ = oracle.rotate(x64.astype(np.float32), pi, inverse=True)
    # the fp32 round trip of x' bounds the error
    assert np.max(np.abs(back64 - x)) <= 1e-6 * np.max(np.abs(x))


def test_rotation_cancels_inside_the_product():
    # [OQ] 2.2: W Pi^T Pi x = W x -- with quantisation off the rotated
    # product equals the plain one up to the fp32 rounding of x' and W'.
    inp = workloads.tiny_inputs()
    d = 256
    perm, signs = oracle.rpbh_descriptor(inp["rpbh_seed"], d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    x, w = inp["x"], inp["w"]
    x64, x32 = oracle.rotate(x, pi)
    w64, w32 = oracle.rotate(w, pi)
    ref = oracle.matmul_f64(x, w)
    exact = x64 @ w64.T
    assert np.linalg.norm(exact - ref) <= 1e-12 * np.linalg.norm(ref)
    y32 = oracle.matmul_f64(x32, w32)
    rel = np.linalg.norm(y32 - ref) / np.linalg.norm(ref)
    assert rel < 1e-6


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch_and_ties_to_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(3.0),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2.0 ** -130, 3.0e38, 0.0, -0.0],
                 np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),
    ])
    got = oracle.to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0)
    assert oracle.bf16_bits_to_f32(oracle.to_bf16_bits(np.array([1.0 + 2 ** -8])))[0] == 1.0
    assert oracle.bf16_bits_to_f32(oracle.to_bf16_bits(np.array([1.0 + 3 * 2 ** -8])))[0] == 1.0 + 2 ** -6


def test_bf16_of_double_rounds_once():
    # a double just above a bf16 tie must round up even though its fp32
    # rounding would land exactly on the tie.
    x = 1.0 + 2 ** -8 + 2 ** -40
    assert oracle.bf16_bits_to_f32(oracle.to_bf16_bits(np.array([x])))[0] == 1.0 + 2 ** -7


# ---------------------------------------------------------------- INT8

def test_int8_error_bound_and_extremes():
    # [CR2] 4: q = round(v / s); with s = absmax/127 every element is within
    # s/2 of s*q, the absmax element maps to +-127, and |q| <= 127.
    v = workloads.small_case(41, 64, 512)
    v[3] = 0.0
    for bf16_scale in (False, True):
        q, s, _ = oracle.quantize_int8(v, bf16_scale)
        err = np.abs(v.astype(np.float64) - s[:, None].astype(np.float64) * q)
        assert np.all(err <= s[:, None].astype(np.float64) / 2 * (1 + 1e-6))
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        assert s[3] == 0.0 and not q[3].any()
        nz = np.arange(64) != 3
        amax_idx = np.argmax(np.abs(v), axis=1)
        top = np.abs(q[np.arange(64), amax_idx]).astype(np.int32)
        if bf16_scale:
            # a bf16 scale can round below absmax/127 by < 2^-9 relative,
            # so the largest element lands on 127 (never past it).
            assert np.all(top[nz] >= 126)
        else:
            assert np.all(top[nz] == 127)


def test_int8_codes_by_brute_force_round_half_even():
    # Python's round() is round-half-to-even; fp32 division via numpy.
    rng = np.random.default_rng(2)
    v = (rng.standard_normal((8, 64)) * 3).astype(np.float32)
    v[0, :4] = np.float32(127.0) * np.array([1.0, 0.5, 2.5 / 127, -3.5 / 127], np.float32)  # ties
    q, s, pre = oracle.quantize_int8(v, False)
    for r in range(8):
        amax = max(abs(float(a)) for a in v[r])
        sr = np.float32(np.float32(amax) / np.float32(127.0))
        assert sr == s[r]
        for j in range(64):
            t = np.float32(v[r, j] / sr)
            assert pre[r, j] == t
            assert q[r, j] == max(-127, min(127, round(float(t))))


# ---------------------------------------------------------------- codebook

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 6])
def test_lloyd_max_optimality_conditions(bits):
    # [OQ] 4.2: Lloyd-Max codebook for a Gaussian.  Centroids are the
    # conditional means of their cells, boundaries the midpoints
    # (conditions checked with scipy's normal pdf/sf, not the oracle's).
    cb = oracle.lloyd_max(bits, 1)
    c, t = cb["c_unit"], cb["t_unit"]
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(len(c)):
        a, b = edges[k], edges[k + 1]
        mass = scipy.stats.norm.cdf(b) - scipy.stats.norm.cdf(a) if b <= 0 else \
            scipy.stats.norm.sf(a) - scipy.stats.norm.sf(b)
        mean = (scipy.stats.norm.pdf(a) - scipy.stats.norm.pdf(b)) / mass
        assert abs(mean - c[k]) < 1e-12
    assert np.allclose(t, (c[:-1] + c[1:]) / 2, atol=1e-15, rtol=0)
    assert np.array_equal(c, -c[::-1])          # exact symmetry
    assert np.all(np.diff(c) > 0)


def test_lloyd_max_one_bit_closed_form():
    cb = oracle.lloyd_max(1, 1)
    assert np.allclose(cb["c_unit"], [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], rtol=0, atol=1e-15)
    mse = 2 * scipy.integrate.quad(lambda x: (x - math.sqrt(2 / math.pi)) ** 2 * scipy.stats.norm.pdf(x),
                                   0, np.inf, epsabs=1e-14)[0]
    assert abs(mse - (1 - 2 / math.pi)) < 1e-10


def test_lloyd_max_two_bit_is_the_mse_minimum_by_search():
    # Brute force: over symmetric 4-level quantisers with inner boundary t,
    # the best reconstruction levels are the cell means; the MSE is smallest
    # at the oracle's boundary.
    cb = oracle.lloyd_max(2, 1)
    t_or = cb["t_unit"][2]

    def mse(t):
        m1 = (scipy.stats.norm.pdf(0) - scipy.stats.norm.pdf(t)) / (scipy.stats.norm.cdf(t) - 0.5)
        m2 = scipy.stats.norm.pdf(t) / scipy.stats.norm.sf(t)
        f1 = scipy.integrate.quad(lambda x: (x - m1) ** 2 * scipy.stats.norm.pdf(x), 0, t, epsabs=1e-14)[0]
        f2 = scipy.integrate.quad(lambda x: (x - m2) ** 2 * scipy.stats.norm.pdf(x), t, np.inf, epsabs=1e-14)[0]
        return 2 * (f1 + f2)

    grid = np.linspace(0.5, 1.5, 201)
    vals = np.array([mse(t) for t in grid])
    best = grid[np.argmin(vals)]
    assert abs(best - t_or) <= 0.0051
    assert mse(t_or) <= vals.min() + 1e-12


@pytest.mark.parametrize("d", [256, 4096, 16384])
def test_lloyd_max_scales_as_one_over_sqrt_d(d):
    # [OQ] 1 / 4.2: the codebook is for N(0, 1/d) = N(0,1)/sqrt(d).
    cb1 = oracle.lloyd_max(4, 1)
    cbd = oracle.lloyd_max(4, d)
    assert np.array_equal(cbd["centroids"], (cb1["c_unit"] / math.sqrt(d)).astype(np.float32))
    assert np.all(np.diff(cbd["boundaries"]) > 0)
    assert cbd["boundaries"][7] == 0.0


def test_codebook_search_is_nearest_centroid():
    # Counting boundaries below u (numpy searchsorted 'left') equals the
    # nearest-centroid rule away from exact midpoints.
    cb = oracle.lloyd_max(4, 256)
    v = workloads.small_case(5, 32, 256)
    codes, nrm, u = oracle.quantize_codebook(v, cb["boundaries"], False)
    ss = np.searchsorted(cb["boundaries"], u, side="left")
    assert np.array_equal(codes, ss)
    near = np.argmin(np.abs(u[..., None].astype(np.float64) - cb["centroids"].astype(np.float64)), axis=-1)
    far = np.min(np.abs(u[..., None] - cb["boundaries"]), axis=-1) > 1e-6 / 16
    assert np.array_equal(codes[far], near[far])
    # norms: s = ||x'|| in fp32, u = x'/(s+eps)
    assert np.allclose(nrm, np.linalg.norm(v.astype(np.float64), axis=1), rtol=1e-7)


def test_codebook_weight_norm_is_bf16_and_zero_row():
    cb = oracle.lloyd_max(2, 256)
    v = workloads.small_case(6, 8, 256, "w")
    v[2] = 0
    codes, nrm, u = oracle.quantize_codebook(v, cb["boundaries"], True)
    assert np.array_equal(oracle.bf16_bits_to_f32(oracle.to_bf16_bits(nrm)), nrm)
    assert nrm[2] == 0 and np.all(u[2] == 0)
    # u = 0 sits on the middle boundary (0): ties go to the lower cell
    assert np.all(codes[2] == 1)


def test_rotation_evens_out_coordinates():
    # [OQ] 1: after the rotation every coordinate is close to N(0, 1/d).
    # A 64-point block mixes 64 inputs, so a finite excess kurtosis shrinks
    # by ~64x (Laplace: 6 -> ~3.05); outlier channels are flattened by a
    # large factor even though block-local mixing cannot fully even them.
    d = 4096
    perm, signs = oracle.rpbh_descriptor(workloads.RPBH_SEED[d], d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    kurt = lambda u: np.mean(u ** 4) / np.mean(u ** 2) ** 2
    lap = np.random.default_rng(12).laplace(size=(32, d)).astype(np.float32)
    u = oracle.rotate(lap, pi)[0]
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    assert abs(np.mean(u ** 2) * d - 1) < 1e-9
    assert kurt(lap) > 5.5 and 2.9 < kurt(u) < 3.2
    x = workloads.small_case(7, 48, d)
    r = oracle.rotate(x, pi)[0]
    assert kurt(x) > 20 * kurt(r)


def test_permutation_needed_when_outliers_share_a_block():
    # [OQ] 2.3 / 3.3: without P_pi, outliers packed into one block stay
    # there; with RPBH the per-block energy is even.
    d = 1024
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, d)).astype(np.float32)
    x[:, :8] *= 40
    _, signs = oracle.rpbh_descriptor(9, d)
    perm, _ = oracle.rpbh_descriptor(9, d)
    plain = oracle.rpbh_dense(d, 64, np.arange(d, dtype=np.int32), signs)
    rpbh = oracle.rpbh_dense(d, 64, perm, signs)
    e_plain = (oracle.rotate(x, plain)[0] ** 2).reshape(16, d // 64, 64).sum(-1)
    e_rpbh = (oracle.rotate(x, rpbh)[0] ** 2).reshape(16, d // 64, 64).sum(-1)
    ratio = lambda e: (e.max(1) / e.mean(1)).mean()
    # all outlier energy in one of 16 blocks -> max/mean close to 16
    assert ratio(e_plain) > 12
    assert ratio(e_rpbh) < ratio(e_plain) / 2


# ---------------------------------------------------------------- packing

def test_pack_examples_and_roundtrip():
    c4 = np.array([[1, 2, 3, 4, 15, 0, 7, 8]], np.uint8)
    assert list(oracle.pack(c4, 4)[0]) == [0x21, 0x43, 0x0F, 0x87]
    c2 = np.array([[1, 2, 3, 0, 0, 0, 0, 3]], np.uint8)
    assert list(oracle.pack(c2, 2)[0]) == [0b00111001, 0b11000000]
    for bits in (2, 4):
        allc = np.array(list(itertools.product(range(1 << bits), repeat=2)), np.uint8).reshape(4, -1)
        assert np.array_equal(oracle.unpack(oracle.pack(allc, bits), allc.shape[1], bits), allc)


def test_pack_bit_stream_for_three_and_six_bits():
    # 3- and 6-bit codes (the W3A3 / W4A6 variants, OrbitQuant article 3.2-3.3) continue the
    # LSB-first rule as one little-endian bit stream per row: element j in bits [j*b, j*b + b).
    # Worked by hand: 3-bit codes 1..7,0 -> sum c_j 2^(3j) = 0x1F58D1 -> bytes D1 58 1F;
    # 6-bit codes 1, 2, 3, 63 -> 0xFC3081 -> bytes 81 30 FC.
    c3 = np.array([[1, 2, 3, 4, 5, 6, 7, 0]], np.uint8)
    assert list(oracle.pack(c3, 3)[0]) == [0xD1, 0x58, 0x1F]
    c6 = np.array([[1, 2, 3, 63]], np.uint8)
    assert list(oracle.pack(c6, 6)[0]) == [0x81, 0x30, 0xFC]
    # every pair of codes in every position of a 24-bit group survives the round trip
    for bits in (3, 6):
        per = 24 // bits
        rng = np.random.default_rng(bits)
        c = rng.integers(0, 1 << bits, size=(64, 8 * per)).astype(np.uint8)
        assert np.array_equal(oracle.unpack(oracle.pack(c, bits), c.shape[1], bits), c)
        # one set code at each position lights exactly its own bits
        for j in range(per):
            one = np.zeros((1, per), np.uint8)
            one[0, j] = (1 << bits) - 1
            word = int.from_bytes(bytes(oracle.pack(one, bits)[0]), "little")
            assert word == ((1 << bits) - 1) << (bits * j)
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((1, 4), np.uint8), 3)      # 12 bits: not whole bytes


# ---------------------------------------------------------------- products

def test_int8_gemm_matches_integer_matmul():
    rng = np.random.default_rng(3)
    a = rng.integers(-127, 128, size=(5, 192)).astype(np.int8)
    w = rng.integers(-127, 128, size=(7, 192)).astype(np.int8)
    acc = oracle.gemm_int8(a, w)
    assert np.array_equal(acc, a.astype(np.int64) @ w.astype(np.int64).T)
    full = np.full((2, 16384), 127, np.int8)
    assert oracle.gemm_int8(full, -full)[0, 0] == -127 * 127 * 16384


def test_int8_rescale_is_the_dequantised_product():
    # y = (s_a q_a) . (s_w q_w) = s_a s_w sum_j q_a q_w ([CR2] section 4: W ~ s q).  With power-of-two
    # scales every product and sum below is exact in fp64, so the oracle's rescale of the integer
    # product must equal the product of the dequantised operands bit for bit; T != N and distinct
    # scales per row and column catch a transposed or swapped scale.
    rng = np.random.default_rng(12)
    T, N, d = 5, 9, 128
    qa = rng.integers(-127, 128, size=(T, d)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, d)).astype(np.int8)
    sa = np.ldexp(1.0, rng.integers(-12, -2, size=T)).astype(np.float32)
    sw = np.ldexp(1.0, rng.integers(-20, -8, size=N)).astype(np.float32)
    y = oracle.rescale_int8(oracle.gemm_int8(qa, qw), sa, sw)
    deq_a = qa.astype(np.float64) * sa.astype(np.float64)[:, None]
    deq_w = qw.astype(np.float64) * sw.astype(np.float64)[:, None]
    assert y.shape == (T, N)
    assert np.array_equal(y, deq_a @ deq_w.T)
    # a row of zero codes gives zero outputs; a zero scale gives zero outputs
    qa[1] = 0
    sw[3] = 0.0
    y = oracle.rescale_int8(oracle.gemm_int8(qa, qw), sa, sw)
    assert np.all(y[1] == 0.0) and np.all(y[:, 3] == 0.0)


def test_codebook_gemm_matches_float_matmul():
    rng = np.random.default_rng(4)
    cb_a = oracle.lloyd_max(4, 256)["centroids"]
    cb_w = oracle.lloyd_max(2, 256)["centroids"]
    qa = rng.integers(0, 16, size=(6, 256)).astype(np.uint8)
    qw = rng.integers(0, 4, size=(5, 256)).astype(np.uint8)
    s = rng.random(6).astype(np.float32)
    r = rng.random(5).astype(np.float32)
    y = oracle.gemm_codebook(qa, qw, cb_a, cb_w, s, r)
    ref = (cb_a[qa].astype(np.float64) @ cb_w[qw].astype(np.float64).T) * s[:, None] * r[None, :]
    assert np.allclose(y, ref, rtol=1e-13, atol=0)


def test_rotation_lowers_int8_error_on_outliers():
    # [CR1] 2 and 4: rotating before INT8 spreads outlier energy, so the
    # quantised product is closer to W x than without the rotation.
    inp = workloads.tiny_inputs()
    d = 256
    perm, signs = oracle.rpbh_descriptor(inp["rpbh_seed"], d)
    pi = oracle.rpbh_dense(d, 64, perm, signs)
    x, w = inp["x"], inp["w"]
    ref = oracle.matmul_f64(x, w)
    wq = oracle.weights_int8(w, pi, False)
    rot = oracle.qlinear_int8(x, pi, wq)["y"]
    qa, sa, _ = oracle.quantize_int8(x, False)
    qw, sw, _ = oracle.quantize_int8(w, False)
    plain = oracle.rescale_int8(oracle.gemm_int8(qa, qw), sa, sw)
    e_rot = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
    e_plain = np.linalg.norm(plain - ref) / np.linalg.norm(ref)
    assert e_rot < 0.5 * e_plain


def test_transform_ablation_error_ordering():
    # [OQ] 2.3 / 3.3: with outlier channels packed into one block, block Hadamard without P_pi
    # leaves them concentrated, so its W8A8 error stays above RPBH's; RPBH is as good as a dense
    # Haar rotation (the ">25x faster" transform buys nothing worse here), and any rotation beats
    # none.
    d = 1024
    rng = np.random.default_rng(8)
    x = rng.standard_normal((32, d)).astype(np.float32)
    x[:, :8] *= 40
    w = (rng.standard_normal((256, d)) * 0.02).astype(np.float32)
    perm, signs = oracle.rpbh_descriptor(9, d)
    transforms = {
        "block_hadamard": oracle.rpbh_dense(d, 64, np.arange(d, dtype=np.int32), signs),
        "rpbh": oracle.rpbh_dense(d, 64, perm, signs),
        "haar": workloads.haar_orthogonal(9, d).astype(np.float64),
    }
    ref = oracle.matmul_f64(x, w)
    qa, sa, _ = oracle.quantize_int8(x, False)
    qw, sw, _ = oracle.quantize_int8(w, False)
    err = {"none": np.linalg.norm(oracle.rescale_int8(oracle.gemm_int8(qa, qw), sa, sw) - ref)}
    for name, pi in transforms.items():
        err[name] = np.linalg.norm(oracle.qlinear_int8(x, pi, oracle.weights_int8(w, pi, False))["y"] - ref)
    assert err["none"] > 2 * err["block_hadamard"]
    assert err["block_hadamard"] > 1.3 * err["rpbh"]
    assert err["rpbh"] < 1.25 * err["haar"]


def test_haar_input_is_orthogonal():
    # the dense comparison rotation is orthogonal (Q^T Q = I to fp32 rounding)
    q = workloads.haar_orthogonal(5, 256).astype(np.float64)
    assert np.abs(q.T @ q - np.eye(256)).max() < 1e-6


@pytest.mark.parametrize("bits,mse", [(3, 0.034548), (4, 0.009501)])
def test_lloyd_max_mse_matches_max_table(bits, mse):
    # Max (1960), "Quantizing for minimum distortion" (outside the pages): the minimum mean-square
    # error of an L-level quantiser of N(0,1); recomputed here by quadrature over the oracle's cells.
    cb = oracle.lloyd_max(bits, 1)
    c, t = cb["c_unit"], cb["t_unit"]
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    err = sum(scipy.integrate.quad(lambda x, ck=c[k]: (x - ck) ** 2 * scipy.stats.norm.pdf(x),
                                   edges[k], edges[k + 1])[0] for k in range(len(c)))
    assert abs(err - mse) < 2e-6


# ---------------------------------------------------------------- asymmetric INT8 (zero points)

def _asym_cases():
    rng = np.random.default_rng(31)
    v = rng.standard_normal((6, 512)).astype(np.float32)
    v[1] = np.abs(v[1]) + 0.5          # all positive
    v[2] = -np.abs(v[2]) * 3           # all negative
    v[3] = 0.0                         # zero row
    v[4] = 0.75                        # constant row
    v[5] = rng.exponential(1.0, 512).astype(np.float32) - 0.2   # skewed
    return v


@pytest.mark.parametrize("scale_bf16", [False, True])
def test_int8_asym_reconstruction_bounds(scale_bf16):
    # [CR1] 3 / [CR3]: scale and zero point per row; v ~ s (q - z).  Zero is an exact code, the
    # row minimum (or 0) maps to -128, codes stay in [-128, 127], and every element the clamp
    # leaves alone is within s/2 of its reconstruction; clamped ends are within s.
    v = _asym_cases()
    q, s, z, csum, pre = oracle.quantize_int8_asym(v, scale_bf16)
    assert q.dtype == np.int8 and np.all(z >= -128) and np.all(z <= 127)
    assert np.array_equal(csum, q.astype(np.int64).sum(1))
    if scale_bf16:
        assert np.array_equal(oracle.bf16_bits_to_f32(oracle.to_bf16_bits(s)), s)
    for r in range(v.shape[0]):
        if s[r] == 0:
            assert not v[r].any() and z[r] == 0 and not q[r].any()
            continue
        rec = s[r] * (q[r].astype(np.float64) - z[r])
        err = np.abs(rec - v[r])
        unclamped = np.rint(pre[r]) + z[r] == q[r]
        assert np.all(err[unclamped] <= s[r] / 2 * (1 + 1e-6))
        assert np.all(err <= s[r] * (1 + 1e-6))
        lo = min(float(v[r].min()), 0.0)
        assert q[r][v[r] == v[r].min()].min() == -128 or lo == 0.0
    assert z[1] == -128                                     # lo = 0 for a positive row: 0 -> -128
    assert z[2] == 127 and q[2].max() <= 127                # hi = 0 for a negative row: 0 -> 127
    # the constant row 0.75: range [0, 0.75], every element at the top code, reconstructed exactly
    assert np.all(q[4] == 127) and z[4] == -128 and np.allclose(s[4] * 255, 0.75, rtol=2 ** -8 if scale_bf16 else 1e-6)


def test_int8_asym_product_equals_integer_definition_and_expansion():
    rng = np.random.default_rng(32)
    qa = rng.integers(-128, 128, size=(5, 192)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(7, 192)).astype(np.int8)
    za = rng.integers(-128, 128, size=5).astype(np.int32)
    zw = rng.integers(-128, 128, size=7).astype(np.int32)
    acc = oracle.gemm_int8_asym(qa, za, qw, zw)
    a64, w64 = qa.astype(np.int64), qw.astype(np.int64)
    assert np.array_equal(acc, (a64 - za[:, None]) @ (w64 - zw[:, None]).T)
    # the four-term form the product's epilogue uses
    d = qa.shape[1]
    expand = a64 @ w64.T - zw[None, :] * a64.sum(1)[:, None] - za[:, None] * w64.sum(1)[None, :] + \
        d * za[:, None].astype(np.int64) * zw[None, :]
    assert np.array_equal(acc, expand)


def test_int8_asym_beats_symmetric_on_skewed_rows():
    # a zero point spends all 256 levels on [lo, hi]: on one-sided rows the step halves
    rng = np.random.default_rng(33)
    v = (rng.exponential(1.0, size=(8, 1024))).astype(np.float32)
    qs, ss, _ = oracle.quantize_int8(v, False)
    qa, sa, za, _, _ = oracle.quantize_int8_asym(v, False)
    e_sym = np.linalg.norm(ss[:, None] * qs - v)
    e_asym = np.linalg.norm(sa[:, None] * (qa.astype(np.float64) - za[:, None]) - v)
    assert e_asym < 0.6 * e_sym
