"""GPU parity of the offline weight rotate-quantise of one DiT block's four linears, at full row
count (OrbitQuant article, section 2.1: W' = W Pi^T, then a per-row INT8 scale and codes; the INT8
rule of "量化旋转主模型是什么？一文读懂低比特图像生成模型", section 4).

Each linear is quantised whole, in the launch the benchmark times (bf16 weights in, int8 codes and
bf16 row scales out).  64 rows spread over the whole matrix (the first and last row, then one row
from each of 62 equal slices, so every part of the launch's row range is met) go through the
oracle: scales bit-exact, codes equal up to the boundary allowance.  Every row is also checked
against two properties that hold at any size: its largest code is +-127 (the absmax element; the
stored bf16 scale keeps max|x'|/s within [126.75, 127.25]), and the dequantised row has the norm
of the input row to within the rounding bound (s/2) sqrt(d), since the rotation is orthogonal."""
import numpy as np
import pytest

import oracle
import rotation_then_quantize_amd as rtq
import workloads
from _helpers import bf16_host, dense_pi, int8_mismatches_allowed, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rtq.load_library()


def _spread_rows(n, count, seed):
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, n, count - 1, dtype=np.int64)
    picks = [rng.integers(edges[i], edges[i + 1]) for i in range(count - 2)]
    return np.unique(np.concatenate([[0, n - 1], picks]))


@pytest.mark.parametrize("name,n_out,d_in", workloads.DIT_LINEARS)
def test_offline_linear_full_rows(name, n_out, d_in):
    wh = workloads.dit_weight_bf16(name)
    assert wh.shape == (n_out, d_in)
    seed = workloads.RPBH_SEED[d_in]
    R = rtq.Rpbh.from_seed(seed, d_in)
    print(f"offline {name}: {n_out} x {d_in}", flush=True)
    q = torch.empty((n_out, d_in), dtype=torch.int8, device="cuda")
    s = torch.empty(n_out, dtype=torch.bfloat16, device="cuda")
    rtq.quantize_rows(to_dev(wh, "bf16"), q, s, R, rtq.RTQ_INT8)
    torch.cuda.synchronize()
    qh = q.cpu().numpy()
    sh = workloads.bf16_bits_to_f32(bf16_host(s)).astype(np.float64)
    rows = _spread_rows(n_out, 64, 31 + d_in)
    wo = oracle.weights_int8(workloads.bf16_bits_to_f32(wh[rows]), dense_pi(seed, d_in), True)
    assert np.array_equal(sh[rows].astype(np.float32), wo["scale"])
    assert int8_mismatches_allowed(qh[rows], wo["q"], wo["pre"])[1] == 0
    # every row: the absmax element takes the end code, and the dequantised norm matches
    assert np.all(np.abs(qh.astype(np.int32)).max(axis=1) == 127)
    wf = workloads.bf16_bits_to_f32(wh).astype(np.float64)
    norm_in = np.sqrt(np.einsum("ij,ij->i", wf, wf))
    qf = qh.astype(np.float64)
    norm_q = sh * np.sqrt(np.einsum("ij,ij->i", qf, qf))
    assert np.all(np.abs(norm_q - norm_in) <= 0.5 * sh * np.sqrt(d_in) + 1e-6 * norm_in)
