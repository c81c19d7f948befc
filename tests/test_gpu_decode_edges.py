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


# ---------------------------------------------------------------------------
# 1-4 tokens of aligned fp32 / bf16 rows: the GEMV quantises them itself
# (one launch).  Its beta and q must be the quantiser's, bit for bit.
# ---------------------------------------------------------------------------
FQ_CASES = [  # (layout, M, N, K)
    ("i2", 1, 3200, 3200), ("i2", 4, 3200, 8640), ("i2", 2, 17, 64), ("i2", 3, 700, 1001), ("i2", 4, 1024, 100),
    ("i2", 1, 50, 16), ("b3", 1, 3200, 3200), ("b3", 4, 333, 1001), ("b3", 2, 100, 80), ("b1", 1, 3200, 3200),
    ("b1", 3, 500, 1000), ("b1", 4, 64, 128),
    ("b3", 4, 3200, 8640), ("b1", 4, 3200, 8640),
    # wide layers: the persistent kernel with the quantiser inside
    ("i2", 1, 8640, 3200), ("i2", 4, 8640, 3200), ("i2", 3, 9000, 77), ("b3", 2, 8640, 1001), ("b3", 4, 8640, 3200),
    ("b1", 1, 8640, 3200), ("b1", 3, 9000, 77),
]


@pytest.mark.parametrize("xk", ["bf16", "f32"])
@pytest.mark.parametrize("layout,M,N,K", FQ_CASES)
def test_fused_quant_gemv(layout, M, N, K, xk):
    xdt = bl.BF16 if xk == "bf16" else bl.F32
    kname = bl.bitlinear_product_kernel(M, N, K, LAYOUTS[layout], xdt)
    log("fused quant gemv", layout, M, N, K, xk, kname)
    assert kname.startswith(("bl::k_gemv_fq<", "bl::k_gemv_persist_fq<")), kname
    t = weights(layout, N, K, seed=M * 7 + N + K)
    x = (synth.activations_bf16 if xk == "bf16" else synth.activations_f32)(M, K, seed=N + 3 * K)
    # rows padded to 16 bytes (the one-launch path needs aligned rows)
    ld = -(-K * x.itemsize // 16) * 16 // x.itemsize
    xw = np.zeros((M, ld), x.dtype)
    xw[:, :K] = x
    xd = to_dev(xw)[:, :K]
    assert xd.data_ptr() % 16 == 0 and (xd.stride(0) * xd.element_size()) % 16 == 0
    check(layout, t, x, xd, N, K)
    # the two-launch path (quantiser, then the GEMV on int8) gives the same bits
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([0.0173], np.float32))
    Xq, beta = bl.quantize_act(xd)
    y2 = to_host(bl.forward(P, LAYOUTS[layout], gamma, Xq, N, K, beta=beta, algo=bl.ALGO_GEMV_MFMA))
    y1 = to_host(bl.forward(P, LAYOUTS[layout], gamma, xd, N, K))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_fused_quant_gemv_rows():
    """Zero, dominant and tie rows, -0.0, and rows in a strided (but aligned)
    view, through the one-launch path."""
    M, N, K = 4, 300, 1000
    t = synth.ternary_weights(N, K, seed=21)
    xw = synth.activations_bf16(M, 1024, seed=22)  # row stride 1024 values: 2048 bytes
    xw[0] = 0
    xw[1, 5] = 3e4
    xw[3] = np.float32(-0.0)
    xd = to_dev(xw)[:, :K]
    assert bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_I2, bl.BF16).startswith("bl::k_gemv_fq<")
    check("i2", t, np.ascontiguousarray(xw[:, :K]), xd, N, K)


def test_fused_quant_gemv_graph_replay():
    """The one-launch decode forward captured in a HIP graph and replayed with
    eager work between replays gives the eager result every time."""
    M, N, K = 3, 3200, 3200
    t = synth.ternary_weights(N, K, seed=23)
    x = to_dev(synth.activations_bf16(M, K, seed=24))
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
