"""The allocation-free forward (bitlinear_forward_noalloc) through the C ABI:
two calls in a row, the second with a smaller input, each compared with
bitlinear_forward on the same inputs (bit-identical) and with the oracle.
The cases use the scratch array for what bitlinear_forward keeps in its
workspace: the staged int8 activations and beta, for the GEMV (16 tokens;
unaligned rows) and for the GEMM on binary weights."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu


def _noalloc(P, layout, gamma, X, N, K, y_dtype=torch.float32):
    M = X.shape[0]
    Y = torch.empty((M, N), dtype=y_dtype, device=X.device)
    ydt = {torch.float32: bl.F32, torch.int32: bl.I32, torch.bfloat16: bl.BF16}[y_dtype]
    xdt = bl.F32 if X.dtype == torch.float32 else bl.BF16
    st = bl.bitlinear_forward_noalloc(P.data_ptr(), layout, gamma.data_ptr(), M, N, K, X.data_ptr(), xdt,
                                      X.stride(0), None, Y.data_ptr(), ydt, Y.stride(0),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == bl.OK, bl.bitlinear_status_string(st)
    return Y


CASES = [  # (name, layout, M, N, K, x kind) -- in call order: larger, then smaller
    ("i2_16x3200x3200_bf16", bl.LAYOUT_I2, 16, 3200, 3200, "bf16"),
    ("i2_5x700x1001_f32", bl.LAYOUT_I2, 5, 700, 1001, "f32"),
    ("b1_gemm_300x512x1000_bf16", bl.LAYOUT_B1, 300, 512, 1000, "bf16"),
    ("b1_gemm_40x256x300_bf16", bl.LAYOUT_B1, 40, 256, 300, "bf16"),
]


@pytest.mark.parametrize("pair", [(0, 1), (2, 3)], ids=["gemv_staged", "gemm_b1_staged"])
def test_noalloc_matches_forward_two_calls(pair):
    results = []
    for idx in pair:
        name, layout, M, N, K, xk = CASES[idx]
        print("noalloc", name, flush=True)
        assert bl.bitlinear_forward_workspace_bytes(M, N, K, layout, bl.BF16 if xk == "bf16" else bl.F32) > 0
        t = synth.binary_weights(N, K, seed=M + N) if layout == bl.LAYOUT_B1 else synth.ternary_weights(N, K, seed=M + N)
        x = (synth.activations_bf16 if xk == "bf16" else synth.activations_f32)(M, K, seed=K + M)
        xw = np.zeros((M, K + 3), x.dtype)  # row stride K + 3: unaligned rows (the staged quantiser)
        xw[:, :K] = x
        xd = to_dev(xw)[:, :K]
        P = to_dev(oracle.pack(t, layout))
        g = to_dev(np.array([0.0173], np.float32))
        y = to_host(_noalloc(P, layout, g, xd, N, K))
        acc = to_host(_noalloc(P, layout, g, xd, N, K, torch.int32))
        want = to_host(bl.forward(P, layout, g, xd, N, K))
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), name
        ref = oracle.forward(t, np.float32(0.0173), synth.bf16_bits_to_f32(x) if xk == "bf16" else x)
        assert np.array_equal(acc, ref["acc"]), name
        assert_f32_parity(y, ref["y"])
        results.append(y)
    torch.cuda.synchronize()


def test_noalloc_rejects_beyond_scratch():
    # 1024 tokens x 131072 columns of staged int8 activations exceed the 64 MiB array
    st = bl.bitlinear_forward_noalloc(0x10000, bl.LAYOUT_I2, 0x20000, 1024, 16, 131072, 0x40000000, bl.BF16, 131072,
                                      None, 0x80000000, bl.F32, 16, None)
    assert st == bl.ERR_SCRATCH
