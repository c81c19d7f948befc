"""GPU parity on activation rows whose absmax beta lies below 127 / FLT_MAX
(about 3.7e-37), where 127 / beta is not a finite binary32: subnormal rows,
tiny normal rows, and a row with exact zeros.  The quantiser takes such a row
to the power-of-two scale where beta lies in [1, 2) (8-bit absmax activations,
LIT-380 record, Key takeaways, bullet 1; the reading is scale-invariant), so
q must match the oracle bit for bit on every path that quantises: the
standalone quantisers (row-major and tiled), the GEMVs that quantise 1 to 4
tokens themselves (per-tile and persistent; i2, b3, b1), 16 tokens (quantiser
then GEMV) and 2048 tokens (quantiser then GEMM)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}
# power-of-two row scales: subnormal, tiny normal, below and above 2^-96, ordinary
SCALES = [2.0 ** -133, 2.0 ** -124, 2.0 ** -110, 1.0, 2.0 ** -140, 2.0 ** -97, 2.0 ** -126, 2.0 ** 60]


def log(*a):
    print(*a, flush=True)


def tiny_rows(M, K, seed, xk):
    """N(0, 1) rows scaled by the powers of two above (cycled); row 1 (if any)
    is the hand row [1e-38, 3e-39, -5e-39, 0, ...]; returned as fp32 or as
    bfloat16 bit patterns."""
    x = synth.activations_f32(M, K, seed).astype(np.float64)
    for m in range(M):
        x[m] *= SCALES[m % len(SCALES)]
    x = x.astype(np.float32)
    if M > 1:
        x[1] = 0.0
        x[1, :4] = [1e-38, 3e-39, -5e-39, 0.0]
        x[1, 4:K:3] = np.float32(2e-39)
    if xk == "bf16":
        xb = synth.to_bf16_bits(x)
        return xb, synth.bf16_bits_to_f32(xb)
    return x, x


def test_rows_are_tiny():
    x, xf = tiny_rows(8, 300, seed=1, xk="f32")
    beta = np.abs(xf).max(axis=1)
    assert (beta < np.float32(127) / np.finfo(np.float32).max).sum() >= 4


@pytest.mark.parametrize("xk", ["f32", "bf16"])
@pytest.mark.parametrize("M,K", [(8, 3200), (3, 77), (96, 3200), (70, 640)])
def test_quantize_act_tiny_beta(M, K, xk):
    log("quantize_act tiny beta", M, K, xk)
    x, xf = tiny_rows(M, K, seed=M + K, xk=xk)
    q_ref, b_ref = oracle.quantize_act(xf)
    Xq, beta = bl.quantize_act(to_dev(x))
    assert np.array_equal(to_host(beta).view(np.uint32), b_ref.view(np.uint32))
    assert np.array_equal(to_host(Xq)[:, :K], q_ref)
    for layout in (bl.LAYOUT_I2, bl.LAYOUT_B3):
        Xt, bt = bl.quantize_act_tiled(to_dev(x), layout)
        assert np.array_equal(to_host(bt).view(np.uint32), b_ref.view(np.uint32))
        y = to_host(bl.forward(to_dev(oracle.pack(np.eye(16, K, dtype=np.int8), layout)), layout,
                               to_dev(np.array([1.0], np.float32)), Xt, 16, K, beta=bt, y_dtype=torch.int32))
        # with T = I (16 rows) the accumulators are q[:, :16] itself
        assert np.array_equal(y, q_ref[:, :16].astype(np.int32))


def _forward_case(layout, M, N, K, xk, want_kernel=None):
    xdt = bl.BF16 if xk == "bf16" else bl.F32
    kname = bl.bitlinear_product_kernel(M, N, K, LAYOUTS[layout], xdt)
    log("forward tiny beta", layout, M, N, K, xk, kname)
    if want_kernel:
        assert kname.startswith(want_kernel), kname
    t = synth.binary_weights(N, K, seed=N + K) if layout == "b1" else synth.ternary_weights(N, K, seed=N + K)
    x, xf = tiny_rows(M, K, seed=3 * M + K, xk=xk)
    gamma = np.float32(0.0173)
    ref = oracle.forward(t, gamma, xf)
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    g = to_dev(np.array([gamma], np.float32))
    xd = to_dev(x)
    acc = to_host(bl.forward(P, LAYOUTS[layout], g, xd, N, K, y_dtype=torch.int32))
    assert np.array_equal(acc, ref["acc"]), f"acc mismatch at {np.argwhere(acc != ref['acc'])[:5]}"
    assert_f32_parity(to_host(bl.forward(P, LAYOUTS[layout], g, xd, N, K)), ref["y"])
    yb = to_host(bl.forward(P, LAYOUTS[layout], g, xd, N, K, y_dtype=torch.bfloat16))
    assert_bf16_parity(yb, ref["y"], oracle.f32_to_bf16(ref["y"]))


@pytest.mark.parametrize("xk", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["i2", "b3", "b1"])
@pytest.mark.parametrize("M", [1, 2, 4])
def test_fused_gemv_tiny_beta(layout, M, xk):
    # per-tile kernel with the quantiser inside
    _forward_case(layout, M, 3200, 3200, xk, want_kernel="bl::k_gemv_fq<")
    # persistent kernel with the quantiser inside
    _forward_case(layout, M, 8640, 3200, xk, want_kernel="bl::k_gemv_persist_fq<")


@pytest.mark.parametrize("xk", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["i2", "b3"])
def test_gemv16_tiny_beta(layout, xk):
    _forward_case(layout, 16, 3200, 3200, xk)


@pytest.mark.parametrize("xk", ["f32", "bf16"])
def test_gemm2048_tiny_beta(xk):
    _forward_case("i2", 2048, 512, 640, xk, want_kernel="bl::k_gemm_mfma")
