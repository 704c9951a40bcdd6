"""GPU parity of the INT8-core product over seeded random shapes: every operand format (row-major
and tiled INT8 codes; 2-, 3- and 4-bit codebook weights with int8 activation values, row-major and
tiled), with and without the K-split workspace, ragged T and N, d from 64 to 4096.  The raw int32
accumulators (`RTQ_I32`) must equal the oracle's int64 product of the same codes (through the
int8 codebook tables, computed here from the oracle's centroids) exactly; at shapes whose full
product would be slow on the CPU, 48 sampled rows (the first and last always among them)."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
from _helpers import int8_table, tile_codes, tile_packed, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _shapes():
    rng = np.random.default_rng(20261203)
    out = []
    for k in range(28):
        big = k % 7 == 6                      # a few shapes past one round of 256 x 256 tiles
        T = int(rng.integers(2000, 4700)) if big else int(rng.integers(1, 1500))
        N = int(rng.integers(2000, 4700)) if big else int(rng.integers(1, 1500))
        d = int(rng.choice([1024, 2048, 4096])) if big else int(rng.choice([64, 128, 256, 512, 1024, 2048]))
        fmt = ["int8", "int8_tiled", "cb4", "cb4_tiled", "cb2", "cb2_tiled", "cb3", "cb3_tiled"][k % 8]
        ws = bool(rng.integers(0, 2)) or big
        out.append((k, T, N, d, fmt, ws))
    return out


@pytest.mark.parametrize("k,T,N,d,fmt,ws", _shapes())
def test_product_accumulators_random_shapes(k, T, N, d, fmt, ws):
    rng = np.random.default_rng(1000 + k)
    tiled = fmt.endswith("_tiled")
    bits = 8 if fmt.startswith("int8") else int(fmt[2])
    rows = np.arange(T) if T * N * d <= 1 << 31 else np.unique(
        np.concatenate([[0, T - 1], rng.choice(T, 46, replace=False)]))
    if bits == 8:
        a = rng.integers(-127, 128, size=(T, d)).astype(np.int8)
        w = rng.integers(-127, 128, size=(N, d)).astype(np.int8)
        ref = oracle.gemm_int8(a[rows], w)
        w_dev = to_dev(tile_codes(w)) if tiled else to_dev(w)
        mode = rtq.RTQ_INT8_TILED if tiled else rtq.RTQ_INT8
        cba = cbw = None
    else:
        ocb_a, ocb_w = oracle.lloyd_max(4, d), oracle.lloyd_max(bits, d)
        _, ta = int8_table(ocb_a["centroids"])
        _, tw = int8_table(ocb_w["centroids"])
        a = ta[rng.integers(0, 16, size=(T, d), dtype=np.uint8)].astype(np.int8)
        cw = rng.integers(0, 1 << bits, size=(N, d), dtype=np.uint8)
        ref = oracle.gemm_int8(a[rows], tw[cw].astype(np.int8))
        packed = oracle.pack(cw, bits)
        w_dev = to_dev(tile_packed(packed, bits)) if tiled else to_dev(packed)
        mode = rtq.RTQ_CODEBOOK_I8_TILED if tiled else rtq.RTQ_CODEBOOK_I8
        cba, cbw = rtq.Codebook.for_dim(d, 4), rtq.Codebook.for_dim(d, bits)
    a_dev = to_dev(tile_codes(a)) if tiled else to_dev(a)
    acc = torch.full((T, N), -7, dtype=torch.int32, device="cuda")
    work = rtq.new_qgemm_workspace() if ws else None
    print(f"shape {k}: T={T} N={N} d={d} {fmt} ws={ws}", flush=True)
    rtq.qgemm(a_dev, to_dev(np.ones(T, np.float32)), w_dev, to_dev(np.ones(N, np.float32)), acc, d, mode, cba, cbw,
              workspace=work, n_tokens=T, n_out=N)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy()[rows].astype(np.int64), ref)
