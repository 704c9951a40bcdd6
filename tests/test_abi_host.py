"""CPU tests of librtq's C ABI: exported symbols, host-only helpers against the oracle, and
argument validation (which runs before any HIP call, so no GPU is needed)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
from _helpers import tile_codes, tile_packed, untile_codes, untile_packed

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rtq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = rtq.load_library()
    names = _declared()
    assert set(names) == set(rtq.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", rtq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(rtq_\w+)", out))
    assert set(names) <= exported


def test_library_is_built_for_gfx950():
    sec = subprocess.run(["readelf", "-S", rtq.LIB_PATH], capture_output=True, text=True).stdout
    assert ".hip_fatbin" in sec
    blob = open(rtq.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


@pytest.mark.parametrize("d", [64, 256, 4096, 16384])
def test_rpbh_make_matches_oracle_generator(d):
    for seed in (0, 1, 2003, 2013, 0xFFFFFFFFFFFFFFFF):
        p1, s1 = rtq.rpbh_make(seed, d)
        p2, s2 = oracle.rpbh_descriptor(seed, d)
        assert np.array_equal(p1, p2) and np.array_equal(s1, s2)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [256, 4096, 16384, 1000])
def test_lloyd_max_matches_oracle_within_one_ulp(d, bits):
    c, t = rtq.lloyd_max(d, bits)
    ref = oracle.lloyd_max(bits, d)
    ulp_c = np.spacing(np.abs(ref["centroids"]))
    assert np.all(np.abs(c - ref["centroids"]) <= ulp_c)
    tb = ref["boundaries"]
    ulp_t = np.spacing(np.maximum(np.abs(tb), np.float32(1e-30)))
    assert np.all(np.abs(t - tb) <= ulp_t)
    # in practice they agree bit for bit
    assert np.array_equal(c, ref["centroids"]) and np.array_equal(t, tb)


_R = rtq._Rpbh
_C = rtq._Codebook


A = 0x10000  # a fake, 16-byte aligned "device" address: never dereferenced by the host checks


def test_host_helper_errors():
    lib = rtq.load_library()
    perm = np.empty(64, np.int32)
    signs = np.empty(64, np.int8)
    assert lib.rtq_rpbh_make(1, 64, 32, perm.ctypes.data, signs.ctypes.data) == rtq.RTQ_ERR_UNSUPPORTED
    assert lib.rtq_rpbh_make(1, 100, 64, perm.ctypes.data, signs.ctypes.data) == rtq.RTQ_ERR_INVALID_ARG
    assert lib.rtq_rpbh_make(1, 64, 64, None, signs.ctypes.data) == rtq.RTQ_ERR_INVALID_ARG
    assert "NULL" in rtq.last_error()
    c = np.empty(16, np.float32)
    t = np.empty(15, np.float32)
    assert lib.rtq_lloyd_max(256, 9, c.ctypes.data, t.ctypes.data) == rtq.RTQ_ERR_INVALID_ARG
    assert lib.rtq_lloyd_max(0, 4, c.ctypes.data, t.ctypes.data) == rtq.RTQ_ERR_INVALID_ARG
    assert lib.rtq_lloyd_max(256, 4, c.ctypes.data, t.ctypes.data) == rtq.RTQ_OK
    assert rtq.last_error() == ""


def test_quantize_rows_validation():
    lib = rtq.load_library()
    R = _R(256, 64, A, A)
    cb = _C(4, A, A)
    q = lib.rtq_quantize_rows
    ok_args = dict(x=A, xt=rtq.RTQ_BF16, rows=8, d=256, R=ctypes.byref(R), mode=rtq.RTQ_INT8, cb=None, eps=0.0,
                   codes=A, scale=A, st=rtq.RTQ_F32)

    def call(**kw):
        a = dict(ok_args, **kw)
        return q(a["x"], a["xt"], a["rows"], a["d"], a["R"], a["mode"], a["cb"], ctypes.c_float(a["eps"]),
                 a["codes"], a["scale"], a["st"], None)

    assert call(d=100) == rtq.RTQ_ERR_INVALID_ARG                      # d % 64
    assert call(d=192, R=None) == rtq.RTQ_ERR_UNSUPPORTED              # 3 blocks: not a power of two
    assert call(d=32768, R=None) == rtq.RTQ_ERR_UNSUPPORTED            # beyond 16384
    assert call(d=512) == rtq.RTQ_ERR_INVALID_ARG                      # descriptor d mismatch
    assert call(x=None) == rtq.RTQ_ERR_INVALID_ARG
    assert call(x=A + 8) == rtq.RTQ_ERR_MISALIGNED
    assert call(codes=A + 4) == rtq.RTQ_ERR_MISALIGNED
    assert call(xt=rtq.RTQ_I32) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(rows=-1) == rtq.RTQ_ERR_INVALID_ARG
    assert call(cb=ctypes.byref(cb)) == rtq.RTQ_ERR_INVALID_ARG         # INT8 takes no codebook
    assert call(mode=rtq.RTQ_CODEBOOK) == rtq.RTQ_ERR_INVALID_ARG       # codebook missing
    assert call(mode=rtq.RTQ_CODEBOOK, cb=ctypes.byref(_C(5, A, A))) == rtq.RTQ_ERR_UNSUPPORTED   # no 5-bit codes
    assert call(mode=rtq.RTQ_CODEBOOK, cb=ctypes.byref(_C(6, A, A))) == rtq.RTQ_ERR_UNSUPPORTED   # 6-bit: int8 values only
    # 3- and 6-bit codes come from the bf16 rotate-quantise kernels only
    assert call(mode=rtq.RTQ_CODEBOOK, cb=ctypes.byref(_C(3, A, A)), xt=rtq.RTQ_F32) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK, cb=ctypes.byref(_C(3, A, A)), R=None) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK_I8, cb=ctypes.byref(_C(6, A, A)), R=None) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK, cb=ctypes.byref(cb), eps=-1.0) == rtq.RTQ_ERR_INVALID_ARG
    assert call(mode=7) == rtq.RTQ_ERR_INVALID_ARG
    # tiled codebook layouts: the same checks as their row-major modes
    assert call(mode=rtq.RTQ_CODEBOOK_TILED) == rtq.RTQ_ERR_INVALID_ARG        # codebook missing
    assert call(mode=rtq.RTQ_CODEBOOK_TILED, cb=ctypes.byref(_C(6, A, A))) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK_TILED, cb=ctypes.byref(_C(3, A, A)), R=None) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK_I8_TILED, cb=ctypes.byref(_C(6, A, A)), R=None) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK_I8_TILED, cb=ctypes.byref(_C(5, A, A))) == rtq.RTQ_ERR_UNSUPPORTED
    assert call(mode=rtq.RTQ_CODEBOOK_TILED, cb=ctypes.byref(cb), rows=0) == rtq.RTQ_OK
    assert call(mode=rtq.RTQ_CODEBOOK_I8_TILED, cb=ctypes.byref(cb), rows=0) == rtq.RTQ_OK
    R_bad_h = _R(256, 32, A, A)
    assert call(R=ctypes.byref(R_bad_h)) == rtq.RTQ_ERR_UNSUPPORTED
    R_misaligned = _R(256, 64, A + 2, A)
    assert call(R=ctypes.byref(R_misaligned)) == rtq.RTQ_ERR_MISALIGNED
    # zero rows: valid, nothing launched, no GPU needed
    assert call(rows=0) == rtq.RTQ_OK


def test_qgemm_and_qlinear_validation():
    lib = rtq.load_library()
    cb4 = _C(4, A, A)
    cb2 = _C(2, A, A)
    g = lib.rtq_qgemm
    base = [A, A, 16, A, A, rtq.RTQ_BF16, 32, 256, rtq.RTQ_INT8, None, None, A, rtq.RTQ_BF16, None]

    def call(idx_vals):
        a = list(base)
        for i, v in idx_vals.items():
            a[i] = v
        return g(*a)

    assert call({6: 0}) == rtq.RTQ_ERR_INVALID_ARG                       # N = 0
    assert call({7: 100}) == rtq.RTQ_ERR_INVALID_ARG                     # d % 64
    assert call({11: A + 1}) == rtq.RTQ_ERR_MISALIGNED                   # y
    assert call({9: ctypes.byref(cb4)}) == rtq.RTQ_ERR_INVALID_ARG        # codebooks with INT8
    assert call({8: rtq.RTQ_CODEBOOK}) == rtq.RTQ_ERR_INVALID_ARG         # codebooks missing
    assert call({8: rtq.RTQ_CODEBOOK, 9: ctypes.byref(cb2), 10: ctypes.byref(cb2)}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK, 9: ctypes.byref(cb4), 10: ctypes.byref(cb2), 12: rtq.RTQ_I32}) == \
        rtq.RTQ_ERR_UNSUPPORTED
    cb3, cb6 = _C(3, A, A), _C(6, A, A)
    assert call({8: rtq.RTQ_CODEBOOK, 9: ctypes.byref(cb4), 10: ctypes.byref(cb3)}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK_I8, 9: ctypes.byref(cb4), 10: ctypes.byref(cb6)}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK_I8, 9: ctypes.byref(cb6), 10: ctypes.byref(cb3), 2: 0}) == rtq.RTQ_OK
    assert call({2: 0}) == rtq.RTQ_OK                                    # T = 0 is a no-op
    # codebook products give bf16 output only: fp32 output is refused in both codebook modes
    assert call({8: rtq.RTQ_CODEBOOK, 9: ctypes.byref(cb4), 10: ctypes.byref(cb4), 12: rtq.RTQ_F32, 2: 0}) == \
        rtq.RTQ_ERR_UNSUPPORTED
    assert "bf16" in rtq.last_error()
    assert call({8: rtq.RTQ_CODEBOOK_I8, 9: ctypes.byref(cb4), 10: ctypes.byref(cb4), 12: rtq.RTQ_F32, 2: 0}) == \
        rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK_I8, 9: ctypes.byref(cb4), 10: ctypes.byref(cb4), 2: 0}) == rtq.RTQ_OK
    # the tiled codebook product takes the CODEBOOK_I8 arguments; CODEBOOK_TILED is a weight layout only
    assert call({8: rtq.RTQ_CODEBOOK_I8_TILED, 9: ctypes.byref(cb4), 10: ctypes.byref(cb2), 2: 0}) == rtq.RTQ_OK
    assert call({8: rtq.RTQ_CODEBOOK_I8_TILED, 9: ctypes.byref(cb4), 10: ctypes.byref(cb4), 12: rtq.RTQ_F32,
                 2: 0}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK_I8_TILED, 9: ctypes.byref(cb4), 10: ctypes.byref(cb6), 2: 0}) == \
        rtq.RTQ_ERR_UNSUPPORTED
    assert call({8: rtq.RTQ_CODEBOOK_TILED, 9: ctypes.byref(cb4), 10: ctypes.byref(cb4), 2: 0}) == \
        rtq.RTQ_ERR_UNSUPPORTED
    assert "RTQ_CODEBOOK_I8_TILED" in rtq.last_error()
    # output-row limits of the INT8-core product: one 256-row block of y spans at most 2^31 bytes
    assert call({6: (1 << 21) + 8, 12: rtq.RTQ_F32, 2: 0}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({6: (1 << 21) + 8, 12: rtq.RTQ_I32, 2: 0}) == rtq.RTQ_ERR_UNSUPPORTED
    assert call({6: 1 << 21, 12: rtq.RTQ_F32, 2: 0}) == rtq.RTQ_OK
    assert call({6: (1 << 21) + 8, 12: rtq.RTQ_BF16, 2: 0}) == rtq.RTQ_OK
    assert call({6: (1 << 22) + 8, 12: rtq.RTQ_BF16, 2: 0}) == rtq.RTQ_ERR_UNSUPPORTED
    # workspace sizing and checks of the fused call
    ws = lib.rtq_rotated_qlinear_workspace
    split = lib.rtq_qgemm_workspace()
    # two int32 256 x 256 partial tiles and two counters per block slot (a multiple of 8 XCDs)
    per_slot = 2 * (256 * 256 * 4 + 8)
    assert split % 16 == 0 and split % per_slot == 0 and (split // per_slot) % 8 == 0 and split >= 8 * per_slot
    split256 = (split + 255) // 256 * 256
    assert ws(4608, 4096, rtq.RTQ_INT8, 8) == 4608 * 4096 + 4608 * 4 + (256 - (4608 * 4) % 256) % 256 + split256
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 4) == 4608 * 4096 + 18432 + split256
    assert ws(4608, 4096, rtq.RTQ_INT8_TILED, 8) == ws(4608, 4096, rtq.RTQ_INT8, 8)
    assert ws(100, 256, rtq.RTQ_INT8_TILED, 8) == 256 * 256 + 512 + split256     # rows padded to 256
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK, 4) == 4608 * 2048 + 18432
    assert ws(10, 4096, rtq.RTQ_CODEBOOK, 3) == 0
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 3) == ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 6) == \
        ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 4)
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 5) == 0
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_I8_TILED, 4) == ws(4608, 4096, rtq.RTQ_CODEBOOK_I8, 4)
    assert ws(100, 256, rtq.RTQ_CODEBOOK_I8_TILED, 2) == 256 * 256 + 512 + split256   # rows padded to 256
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_I8_TILED, 5) == 0
    assert ws(4608, 4096, rtq.RTQ_CODEBOOK_TILED, 4) == 0                        # not a layer mode
    R = _R(256, 64, A, A)
    ql = lib.rtq_rotated_qlinear
    args = [A, rtq.RTQ_BF16, 16, ctypes.byref(R), A, A, rtq.RTQ_BF16, 32, rtq.RTQ_INT8, None, None, A, rtq.RTQ_BF16,
            A, 1 << 20, None]
    a = list(args); a[14] = 16
    assert ql(*a) == rtq.RTQ_ERR_INVALID_ARG and "workspace too small" in rtq.last_error()
    a = list(args); a[12] = rtq.RTQ_I32
    assert ql(*a) == rtq.RTQ_ERR_UNSUPPORTED
    a = list(args); a[2] = 0
    assert ql(*a) == rtq.RTQ_OK
    # codebook layers: bf16 output only
    a = list(args); a[8] = rtq.RTQ_CODEBOOK_I8; a[9] = ctypes.byref(cb4); a[10] = ctypes.byref(cb4)
    a[12] = rtq.RTQ_F32; a[2] = 0
    assert ql(*a) == rtq.RTQ_ERR_UNSUPPORTED


def test_noalloc_layer_rejects_inputs_beyond_its_scratch():
    # the allocation-free layer checks its size limit on the host, before any HIP call
    lib = rtq.load_library()
    cb4 = _C(4, A, A)
    R = _R(4096, 64, A, A)
    f = lib.rtq_rotated_qlinear_noalloc
    args = [A, rtq.RTQ_BF16, 0, ctypes.byref(R), A, A, rtq.RTQ_BF16, 32, rtq.RTQ_INT8, None, None, A, rtq.RTQ_BF16,
            None]
    limit = rtq.NOALLOC_SCRATCH_BYTES
    # INT8 codes: T * 4096 bytes plus 4 T bytes of scales (each 256-aligned)
    t_max = max(t for t in range(limit // 4096 - 64, limit // 4096 + 1)
                if ((t * 4096 + 255) // 256 + (4 * t + 255) // 256) * 256 <= limit)
    a = list(args); a[2] = t_max + 1
    assert f(*a) == rtq.RTQ_ERR_INVALID_ARG and "static scratch" in rtq.last_error()
    # packed 4-bit codes take half the bytes per token (no call that passes the checks is made
    # here: its fake pointers would reach a kernel)
    a = list(args); a[2] = 2 * t_max + 64; a[8] = rtq.RTQ_CODEBOOK; a[9] = ctypes.byref(cb4); a[10] = ctypes.byref(cb4)
    assert f(*a) == rtq.RTQ_ERR_INVALID_ARG and "static scratch" in rtq.last_error()
    a = list(args); a[3] = None
    assert f(*a) == rtq.RTQ_ERR_INVALID_ARG


def test_rotate_validation():
    lib = rtq.load_library()
    R = _R(256, 64, A, A)
    r = lib.rtq_rpbh_rotate
    assert r(A, rtq.RTQ_F32, A, rtq.RTQ_F32, 4, None, 0, None) == rtq.RTQ_ERR_INVALID_ARG
    assert r(A, rtq.RTQ_F32, A, rtq.RTQ_F32, 4, ctypes.byref(R), 2, None) == rtq.RTQ_ERR_INVALID_ARG
    assert r(A, rtq.RTQ_F32, A, rtq.RTQ_I32, 4, ctypes.byref(R), 0, None) == rtq.RTQ_ERR_UNSUPPORTED
    assert r(A, rtq.RTQ_F32, A, rtq.RTQ_F32, 0, ctypes.byref(R), 0, None) == rtq.RTQ_OK


def test_product_path_has_no_oracle_or_fallback():
    # The product package never imports the oracle and has no CPU compute path.
    pkg = os.path.join(ROOT, "rotation_then_quantize_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.c" not in text and "liboracle" not in text, f


def test_asym_validation():
    lib = rtq.load_library()
    R = _R(256, 64, A, A)
    q = lib.rtq_quantize_rows_asym
    ok = [A, rtq.RTQ_BF16, 8, 256, ctypes.byref(R), A, A, rtq.RTQ_F32, A, A, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return q(*a)

    assert call(a1=rtq.RTQ_F32) == rtq.RTQ_ERR_UNSUPPORTED          # bf16 rows only
    assert call(a4=None) == rtq.RTQ_ERR_UNSUPPORTED                 # rotation required
    assert call(a8=None) == rtq.RTQ_ERR_INVALID_ARG                 # zero points missing
    assert call(a9=A + 2) == rtq.RTQ_ERR_MISALIGNED
    assert call(a2=0) == rtq.RTQ_OK
    g = lib.rtq_qgemm_asym
    base = [A, A, A, A, 16, A, A, rtq.RTQ_BF16, A, A, 32, 256, A, rtq.RTQ_BF16, None, 0, None]

    def gcall(**kw):
        a = list(base)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)

    assert gcall(a2=None) == rtq.RTQ_ERR_INVALID_ARG
    assert gcall(a9=A + 1) == rtq.RTQ_ERR_MISALIGNED
    assert gcall(a11=100) == rtq.RTQ_ERR_INVALID_ARG
    assert gcall(a4=0) == rtq.RTQ_OK
    ws = lib.rtq_rotated_qlinear_asym_workspace
    split256 = (lib.rtq_qgemm_workspace() + 255) // 256 * 256
    assert ws(4608, 4096) == 4608 * 4096 + 3 * 18432 + split256
    ql = lib.rtq_rotated_qlinear_asym
    args = [A, rtq.RTQ_BF16, 16, ctypes.byref(R), A, A, rtq.RTQ_BF16, A, A, 32, A, rtq.RTQ_BF16, A, 1 << 20, None]
    a = list(args); a[13] = 16
    assert ql(*a) == rtq.RTQ_ERR_INVALID_ARG and "workspace too small" in rtq.last_error()
    a = list(args); a[1] = rtq.RTQ_F32
    assert ql(*a) == rtq.RTQ_ERR_UNSUPPORTED
    a = list(args); a[2] = 0
    assert ql(*a) == rtq.RTQ_OK


def test_tile_helpers_follow_the_declared_layouts():
    # the tests' host-side tilers against the byte offsets rtq.h defines for the two tiled layouts
    rng = np.random.default_rng(5)
    rows, d = 300, 256
    q = rng.integers(-127, 128, size=(rows, d)).astype(np.int8)
    t = tile_codes(q)
    assert t.size == rtq.tiled_rows(rows) * d
    for r, j in [(0, 0), (5, 17), (255, 255), (256, 64), (299, 130), (4, 200)]:
        # block ((r/256)*(d/64) + j/64) * 16384, row (r%256) * 64, chunk ((j%64)/16) ^ ((r>>2)&3)
        off = ((r // 256) * (d // 64) + j // 64) * 16384 + (r % 256) * 64 + \
            ((((j % 64) // 16) ^ ((r >> 2) & 3)) * 16) + j % 16
        assert t[off] == q[r, j]
    assert not untile_codes(t, rtq.tiled_rows(rows), d)[rows:].any()
    assert np.array_equal(untile_codes(t, rows, d), q)
    for bits in (2, 3, 4):
        wrow = d * bits // 8
        c = rng.integers(0, 256, size=(rows, wrow)).astype(np.uint8)
        tp = tile_packed(c, bits)
        assert tp.size == rtq.tiled_code_bytes(rows, d, rtq.RTQ_CODEBOOK_TILED, bits)
        for r, b in [(0, 0), (7, 3), (255, wrow - 1), (256, 8 * bits), (299, 5 * bits + 1)]:
            # block ((r/256)*(d/64) + b/(8 bits)) of 256 * 8 bits bytes, row (r%256), byte b % (8 bits)
            rb = 8 * bits
            off = (((r // 256) * (d // 64) + b // rb) * 256 + r % 256) * rb + b % rb
            assert tp[off] == c[r, b]
        assert np.array_equal(untile_packed(tp, rows, d, bits), c)
