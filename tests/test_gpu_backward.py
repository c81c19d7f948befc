"""GPU parity of the straight-through-estimator backward: dX = gamma * dY @ T
from the packed weights (i2, and b3 / b1 through their i2 rewrite) and
dW = dY^T @ Xhat from the forward's int8 activations and beta, against the
oracle's binary64 products.  Both GPU results are fp32 sums in an unspecified
order, so the bar is the summation bound: |got - want| <= (n + 2) * 2^-24 *
sum |terms| per element (n the contraction length), plus bit-exact zeros
where every term is zero.  Batches below 32 tokens (dW), or with fewer than
256 tiles of 128 x 128 (dX), take the small-batch kernels (dX splitting the
weight rows over workgroups when it has few of them); the rest the tiled
ones, with 16-byte stores on aligned rows and single ones otherwise."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}


def log(*a):
    print(*a, flush=True)


def assert_sum_bound(got, want, abs_terms, n):
    got = np.asarray(got, np.float64)
    assert got.shape == want.shape
    assert np.isfinite(got).all()
    bound = (n + 2) * 2.0 ** -24 * abs_terms
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} elements beyond the bound; first at {np.argwhere(bad)[0]}"
    assert np.all(got[abs_terms == 0] == 0)


def weights(layout, N, K, seed):
    return synth.binary_weights(N, K, seed) if layout == "b1" else synth.ternary_weights(N, K, seed)


@pytest.mark.parametrize("layout", ["i2", "b3", "b1"])
@pytest.mark.parametrize("M,N,K", [(1, 3200, 3200), (4, 130, 333), (16, 8640, 3200), (17, 100, 64), (3, 48, 1),
                                   (300, 257, 700), (1024, 1000, 3200), (1100, 130, 3900), (1030, 70, 4001),
                                   (5, 1000, 130), (2, 520, 4100)])
def test_backward_dx(layout, M, N, K):
    log("backward dx", layout, M, N, K)
    t = weights(layout, N, K, seed=M + 3 * N + K)
    gamma = np.float32(0.0173)
    dy = synth.activations_f32(M, N, seed=M + N)
    want = oracle.backward_dx(t, gamma, dy)
    abs_terms = float(gamma) * (np.abs(dy.astype(np.float64)) @ np.abs(t.astype(np.float64)))
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    got = to_host(bl.backward_dx(P, LAYOUTS[layout], to_dev(np.array([gamma], np.float32)), to_dev(dy), K))
    assert_sum_bound(got, want, abs_terms, N)


@pytest.mark.parametrize("M,N,K", [(1, 3200, 3200), (4, 130, 333), (16, 8640, 3200), (17, 100, 65), (5, 1, 7),
                                   (300, 257, 700), (2048, 640, 1024), (33, 100, 65), (40, 129, 1030), (3, 70, 1000), (1, 70, 333), (1, 9, 1030)])
def test_backward_dw(M, N, K):
    log("backward dw", M, N, K)
    x = synth.activations_bf16(M, K, seed=M + K)
    q, beta = oracle.quantize_act(x)
    dy = synth.activations_f32(M, N, seed=2 * M + N)
    want = oracle.backward_dw(q, beta, dy)
    abs_terms = np.abs(dy.astype(np.float64)).T @ np.abs(oracle.dequantize_act(q, beta).astype(np.float64))
    # the forward's own quantiser output feeds the backward
    Xq, beta_d = bl.quantize_act(to_dev(x))
    assert np.array_equal(to_host(Xq)[:, :K], q) and np.array_equal(to_host(beta_d), beta)
    got = to_host(bl.backward_dw(Xq, beta_d, to_dev(dy), K))
    assert_sum_bound(got, want, abs_terms, M)


@pytest.mark.parametrize("M", [6, 3, 1])
def test_backward_strided_and_zero_rows(M):
    """Row strides wider than the rows; a zero gradient row and a zero
    activation token give exact zeros."""
    N, K = 200, 300
    t = synth.ternary_weights(N, K, seed=61)
    gamma = np.float32(0.05)
    dyw = synth.activations_f32(M, N + 13, seed=62)
    if M > 2:
        dyw[2] = 0.0
    dy = np.ascontiguousarray(dyw[:, :N])
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    out = torch.full((M, K + 5), float("nan"), dtype=torch.float32, device="cuda")
    bl.backward_dx(P, bl.LAYOUT_I2, to_dev(np.array([gamma], np.float32)), to_dev(dyw)[:, :N], K, out=out[:, :K])
    got = to_host(out)
    assert np.isnan(got[:, K:]).all()  # columns past K untouched
    want = oracle.backward_dx(t, gamma, dy)
    abs_terms = float(gamma) * (np.abs(dy.astype(np.float64)) @ np.abs(t.astype(np.float64)))
    assert_sum_bound(got[:, :K], want, abs_terms, N)
    if M > 2:
        assert np.all(got[2, :K] == 0)
    x = synth.activations_bf16(M, K, seed=63)
    x[min(4, M - 1)] = 0
    q, beta = oracle.quantize_act(x)
    Xq, beta_d = bl.quantize_act(to_dev(x))
    got = to_host(bl.backward_dw(Xq, beta_d, to_dev(dyw)[:, :N], K))
    want = oracle.backward_dw(q, beta, dy)
    abs_terms = np.abs(dy.astype(np.float64)).T @ np.abs(oracle.dequantize_act(q, beta).astype(np.float64))
    assert_sum_bound(got, want, abs_terms, M)


@pytest.mark.parametrize("xk", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 3200, 3200), (4, 700, 1000), (16, 8640, 3200), (300, 640, 1000)])
def test_forward_quant_outputs_feed_backward_dw(M, N, K, xk):
    """bitlinear_forward_ex returns the quantiser's int8 activations and beta
    next to Y: they equal the oracle's, Y equals the plain forward's bit for
    bit, and bitlinear_backward_dw takes them without a second quantiser pass."""
    log("forward_ex quant outputs -> backward_dw", M, N, K, xk)
    t = synth.ternary_weights(N, K, seed=M + N + K)
    x = (synth.activations_bf16 if xk == "bf16" else synth.activations_f32)(M, K, seed=M * K)
    xf = synth.bf16_bits_to_f32(x) if xk == "bf16" else x
    gamma = np.float32(0.0173)
    ref = oracle.forward(t, gamma, xf)
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    g = to_dev(np.array([gamma], np.float32))
    xd = to_dev(x)
    y, Xq, beta = bl.forward_with_quant(P, bl.LAYOUT_I2, g, xd, N, K)
    assert np.array_equal(to_host(Xq)[:, :K], ref["q"]) and not to_host(Xq)[:, K:].any()
    assert np.array_equal(to_host(beta).view(np.uint32), ref["beta"].view(np.uint32))
    y_plain = to_host(bl.forward(P, bl.LAYOUT_I2, g, xd, N, K))
    assert np.array_equal(to_host(y).view(np.uint32), y_plain.view(np.uint32))
    assert np.array_equal(to_host(y).view(np.uint32), ref["y"].view(np.uint32))
    dy = synth.activations_f32(M, N, seed=M + 2 * N)
    want = oracle.backward_dw(ref["q"], ref["beta"], dy)
    xhat = oracle.dequantize_act(ref["q"], ref["beta"]).astype(np.float64)
    abs_terms = np.abs(dy.astype(np.float64)).T @ np.abs(xhat)
    got = to_host(bl.backward_dw(Xq, beta, to_dev(dy), K))
    assert_sum_bound(got, want, abs_terms, M)
