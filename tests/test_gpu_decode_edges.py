"""GPU parity of the decode forward (at most 4 tokens) on activation rows
that are awkward for the quantiser: a zero token, a single dominant element,
values at rounding ties, negative zeros, row strides that break 16-byte
alignment, a base pointer one element in, K not a multiple of the vector
width; and the forward replayed from a HIP graph.  Accumulators exact,
fp32 / bf16 outputs bit-identical to the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}


def log(*a):
    print(*a, flush=True)


def weights(layout, N, K, seed):
    return synth.binary_weights(N, K, seed) if layout == "b1" else synth.ternary_weights(N, K, seed)


def check(layout, t, x, xd, N, K, y_kinds=("i32", "f32", "bf16")):
    ref = oracle.forward(t, np.float32(0.0173), x)
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([0.0173], np.float32))
    for yk in y_kinds:
        ydt = {"i32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16}[yk]
        y = to_host(bl.forward(P, LAYOUTS[layout], gamma, xd, N, K, y_dtype=ydt))
        if yk == "i32":
            assert np.array_equal(y, ref["acc"]), f"acc mismatch at {np.argwhere(y != ref['acc'])[:5]}"
        elif yk == "f32":
            assert_f32_parity(y, ref["y"])
        else:
            assert_bf16_parity(y, ref["y"], oracle.f32_to_bf16(ref["y"]))


def test_decode_zero_and_extreme_rows():
    """A zero token (beta = 0, q = 0), a token with one huge element (every
    other q rounds to 0), ties at .5 after scaling, and -0.0 inputs."""
    M, N, K = 4, 700, 2048
    t = synth.ternary_weights(N, K, seed=5)
    x = synth.activations_f32(M, K, seed=6)
    x[0] = 0.0
    x[1] = 1e-3
    x[1, 17] = -3e4
    x[2] = np.where(np.arange(K) % 2 == 0, 0.5, -1.5).astype(np.float32)  # beta 1.5: x*s = 42.33.., -127
    x[2, ::7] = 127.0 / 254.0 * 1.5  # scaled to exactly 63.5 up to the rounding of s
    x[3] = -0.0
    check("i2", t, x, to_dev(x), N, K)


def test_decode_unaligned_rows():
    """A row stride that breaks 16-byte alignment, a base pointer one element
    in, K not a multiple of the vector width (the quantiser's scalar path)."""
    N = 1000
    # stride 3203 bf16 elements: rows not 16-byte aligned
    M, K, ldx = 3, 3200, 3203
    xw = synth.activations_bf16(M, ldx, seed=7)
    x = np.ascontiguousarray(xw[:, :K])
    t = synth.ternary_weights(N, K, seed=8)
    check("i2", t, x, to_dev(xw)[:, :K], N, K)
    # base pointer one element in
    xw = synth.activations_f32(2, K + 4, seed=9)
    x = np.ascontiguousarray(xw[:, 1:K + 1])
    xd = to_dev(xw)[:, 1:K + 1]
    assert xd.data_ptr() % 16 != 0
    check("b3", t, x, xd, N, K)
    # K % 8 != 0 for bf16
    K = 3203
    t = synth.ternary_weights(N, K, seed=10)
    x = synth.activations_bf16(4, K, seed=11)
    check("i2", t, x, to_dev(x), N, K)


def test_decode_graph_replay():
    """A decode forward (quantiser + persistent GEMV) captured in a HIP graph and replayed with other eager
    work between replays gives the eager result every time."""
    M, N, K = 2, 8640, 3200
    t = synth.ternary_weights(N, K, seed=12)
    x = to_dev(synth.activations_bf16(M, K, seed=13))
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.02], np.float32))
    want = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, x, N, K))
    out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        bl.forward(P, bl.LAYOUT_I2, gamma, x, N, K, out=out)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            bl.forward(P, bl.LAYOUT_I2, gamma, x, N, K, out=out)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        bl.forward(P, bl.LAYOUT_I2, gamma, x[:1], N, K)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32)), r
