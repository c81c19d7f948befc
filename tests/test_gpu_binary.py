"""GPU parity of the binary-weight variant (weights -1 or +1 with the same
absmean scale; the 1-bit b1 packed layout) against the CPU oracle: the sign
quantiser and gamma bit-exact, b1 packing byte-exact, the forward's int32
accumulators exact and its fp32 / bf16 outputs bit-identical, through the
matrix-core GEMV (row-major and tiled activations, per-tile and persistent
kernels) and through the GEMM, which decodes the bits itself; the load-time
b1 -> i2 transcode byte-exact."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu


def log(*a):
    print(*a, flush=True)


def weight_cases():
    yield "tiny_512x256", synth.latent_weights(512, 256, seed=11)
    yield "ragged_17x129", synth.latent_weights(17, 129, seed=12)
    yield "signed_zeros", np.array([[0.0, -0.0, 1e-45, -1e-45, 0.25, -0.25, 3.0, -3.0]], np.float32)
    yield "zeros", np.zeros((3, 40), np.float32)
    yield "rows_3200x8640", synth.latent_weights(3200, 8640, seed=13)


@pytest.mark.parametrize("name,w", list(weight_cases()), ids=[c[0] for c in weight_cases()])
def test_binarize_weights(name, w):
    log("binarize_weights", name, w.shape)
    T, gamma = bl.binarize_weights(to_dev(w))
    t_ref, g_ref = oracle.quantize_weights_binary(w)
    assert to_host(gamma).view(np.uint32)[0] == np.array(g_ref, np.float32).view(np.uint32)
    assert np.array_equal(to_host(T), t_ref)


def test_binarize_weights_strided():
    w = synth.latent_weights(40, 300, seed=14)
    T, gamma = bl.binarize_weights(to_dev(w)[:, :200])
    t_ref, g_ref = oracle.quantize_weights_binary(np.ascontiguousarray(w[:, :200]))
    assert to_host(gamma)[0] == g_ref
    assert np.array_equal(to_host(T), t_ref)


@pytest.mark.parametrize("N,K", [(1, 1), (16, 128), (17, 129), (33, 127), (48, 257), (100, 1000), (512, 256)])
def test_pack_b1(N, K):
    t = synth.binary_weights(N, K, seed=N * 5 + K)
    P = bl.pack(to_dev(t), bl.LAYOUT_B1)
    assert np.array_equal(to_host(P), oracle.pack(t, bl.LAYOUT_B1))


def run_case(M, N, K, algo, seed, x_kind="bf16", y_kinds=("i32", "f32", "bf16")):
    t = synth.binary_weights(N, K, seed=seed)
    w_scale = np.float32(0.0171)
    P = to_dev(oracle.pack(t, bl.LAYOUT_B1))
    gamma = to_dev(np.array([w_scale], np.float32))
    x = synth.activations_bf16(M, K, seed=seed + 1) if x_kind == "bf16" else synth.activations_f32(M, K, seed + 1)
    ref = oracle.forward(t, w_scale, x)
    xd = to_dev(x)
    for yk in y_kinds:
        ydt = {"i32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16}[yk]
        y = to_host(bl.forward(P, bl.LAYOUT_B1, gamma, xd, N, K, y_dtype=ydt, algo=algo))
        if yk == "i32":
            assert np.array_equal(y, ref["acc"]), f"acc mismatch at {np.argwhere(y != ref['acc'])[:5]}"
        elif yk == "f32":
            assert_f32_parity(y, ref["y"])
        else:
            assert_bf16_parity(y, ref["y"], oracle.f32_to_bf16(ref["y"]))


@pytest.mark.parametrize("algo", [bl.ALGO_GEMV_MFMA, bl.ALGO_AUTO], ids=["mfma_gemv", "auto"])
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (1, 50, 100), (2, 333, 257), (3, 64, 1000), (4, 130, 3200),
                                   (5, 17, 65), (8, 200, 640), (11, 48, 1), (16, 512, 512), (16, 100, 333)])
def test_forward_small(algo, M, N, K):
    """Ragged K: the padding bits of the last k-block are -1 weights that must
    meet zero activations."""
    log("b1 forward", algo, M, N, K)
    run_case(M, N, K, algo, seed=M * 10009 + N * 37 + K)


@pytest.mark.parametrize("algo", [bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA], ids=["mfma_gemv", "gemm"])
@pytest.mark.parametrize("M,N,K", [(17, 40, 100), (64, 96, 512), (130, 257, 700), (256, 128, 64)])
def test_forward_many_tokens(algo, M, N, K):
    log("b1 forward many tokens", algo, M, N, K)
    run_case(M, N, K, algo, seed=M * 137 + N + K)


def test_forward_gemm_prefill_rows():
    """The GEMM at a prefill shape with several workgroup tiles and a ragged
    k tail (the -1 pad weights masked in the last stage)."""
    log("b1 gemm", 2048, 3200, 330)
    run_case(2048, 3200, 330, bl.ALGO_AUTO, seed=21, y_kinds=("i32", "f32"))


@pytest.mark.parametrize("M,N,K", [(16, 512, 256), (7, 100, 333), (40, 260, 700), (1, 48, 3200)])
def test_forward_tiled_input(M, N, K):
    log("b1 forward tiled", M, N, K)
    t = synth.binary_weights(N, K, seed=N + 3 * K)
    x = synth.activations_bf16(M, K, seed=M * 5 + K)
    ref = oracle.forward(t, np.float32(0.02), x)
    P = to_dev(oracle.pack(t, bl.LAYOUT_B1))
    gamma = to_dev(np.array([0.02], np.float32))
    Xt, beta = bl.quantize_act_tiled(to_dev(x), bl.LAYOUT_B1)
    acc = to_host(bl.forward(P, bl.LAYOUT_B1, gamma, Xt, N, K, beta=beta, y_dtype=torch.int32))
    assert np.array_equal(acc, ref["acc"])
    assert_f32_parity(to_host(bl.forward(P, bl.LAYOUT_B1, gamma, Xt, N, K, beta=beta)), ref["y"])


@pytest.mark.parametrize("x_kind", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (16, 8200, 3200), (16, 9000, 9984), (3, 2048, 9920),
                                   (16, 28672, 1000)])
def test_forward_gemv_float_input(x_kind, M, N, K):
    """Float activations of at most 16 tokens: the per-tile and the persistent
    GEMV kernels."""
    log("b1 forward gemv float input", x_kind, M, N, K)
    run_case(M, N, K, bl.ALGO_GEMV_MFMA, seed=M + N + 5 * K, x_kind=x_kind, y_kinds=("i32", "f32"))


def test_forward_max_k():
    """K = BITLINEAR_MAX_K with every weight of row 0 at +1 and a token whose
    every q is 127: the largest accumulator, 127 * K."""
    M, N, K = 3, 40, bl.MAX_K
    t = synth.binary_weights(N, K, seed=22)
    t[0] = 1
    x = synth.activations_bf16(M, K, seed=23)
    x[1] = synth.to_bf16_bits(np.full(K, 0.75, np.float32))
    ref = oracle.forward(t, np.float32(0.03), x)
    assert ref["acc"][1, 0] == 127 * K
    P = to_dev(oracle.pack(t, bl.LAYOUT_B1))
    gamma = to_dev(np.array([0.03], np.float32))
    for algo in (bl.ALGO_AUTO, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        acc = to_host(bl.forward(P, bl.LAYOUT_B1, gamma, to_dev(x), N, K, y_dtype=torch.int32, algo=algo))
        assert np.array_equal(acc, ref["acc"]), algo


def test_binary_chain_end_to_end():
    """Latent weights -> binarize -> pack b1 -> forward, against the oracle's
    own chain on the same latent weights and activations (decode and prefill
    token counts)."""
    N, K = 1000, 1500
    w = synth.latent_weights(N, K, seed=24)
    T, gamma = bl.binarize_weights(to_dev(w))
    P = bl.pack(T, bl.LAYOUT_B1)
    t_ref, g_ref = oracle.quantize_weights_binary(w)
    for M in (1, 16, 300):
        x = synth.activations_bf16(M, K, seed=25 + M)
        ref = oracle.forward(t_ref, g_ref, x)
        assert_f32_parity(to_host(bl.forward(P, bl.LAYOUT_B1, gamma, to_dev(x), N, K)), ref["y"])


@pytest.mark.parametrize("M,N,K", [(1, 50, 100), (5, 17, 65), (16, 100, 333), (16, 256, 128)])
def test_forward_gemm_few_tokens(M, N, K):
    """The GEMM at 1-16 tokens (the bits decoded in the GEMM at any M)."""
    log("b1 gemm few tokens", M, N, K)
    assert bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_B1, bl.BF16, bl.ALGO_GEMM_MFMA).startswith("bl::k_gemm_mfma_b1<")
    run_case(M, N, K, bl.ALGO_GEMM_MFMA, seed=M * 7 + N + K, y_kinds=("i32", "f32"))


@pytest.mark.parametrize("M,N,K", [(40, 300, 200), (300, 130, 1000), (2048, 512, 129)])
def test_forward_gemm_int8_rows_with_junk_past_k(M, N, K):
    """Caller-quantised int8 rows whose bytes past K (up to the row stride)
    hold junk: the GEMM reads them with the row, and the -1 pad weights of the
    last k-block must not meet them (masked operand bytes)."""
    log("b1 gemm int8 junk", M, N, K)
    t = synth.binary_weights(N, K, seed=M + N + K)
    x = synth.activations_bf16(M, K, seed=M + 2 * K)
    ref = oracle.forward(t, np.float32(0.02), x)
    q, beta = oracle.quantize_act(synth.bf16_bits_to_f32(x))
    ldx = (K + 15) // 16 * 16 + 16
    xq = np.random.default_rng(K).integers(-127, 128, size=(M, ldx), dtype=np.int64).astype(np.int8)
    xq[:, :K] = q
    P = to_dev(oracle.pack(t, bl.LAYOUT_B1))
    gamma = to_dev(np.array([0.02], np.float32))
    Xd = to_dev(xq)[:, :K]
    assert bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_B1, bl.I8, bl.ALGO_GEMM_MFMA).startswith("bl::k_gemm_mfma_b1<")
    acc = to_host(bl.forward(P, bl.LAYOUT_B1, gamma, Xd, N, K, beta=to_dev(beta), y_dtype=torch.int32,
                             algo=bl.ALGO_GEMM_MFMA))
    assert np.array_equal(acc, ref["acc"])


@pytest.mark.parametrize("layout", [bl.LAYOUT_B3, bl.LAYOUT_B1], ids=["b3", "b1"])
@pytest.mark.parametrize("N,K", [(1, 1), (17, 129), (64, 1000), (3200, 8640)])
def test_transcode_i2(layout, N, K):
    """The load-time i2 rewrite: byte-exact against packing the same weights
    as i2, and a forward on it equals the oracle."""
    log("transcode i2", layout, N, K)
    t = (synth.binary_weights if layout == bl.LAYOUT_B1 else synth.ternary_weights)(N, K, seed=N + K)
    P2 = bl.transcode_i2(to_dev(oracle.pack(t, layout)), layout, N, K)
    assert np.array_equal(to_host(P2), oracle.pack(t, bl.LAYOUT_I2))
    if N * K <= 64 * 1000:
        x = synth.activations_bf16(300, K, seed=K)
        ref = oracle.forward(t, np.float32(0.02), x)
        acc = to_host(bl.forward(P2, bl.LAYOUT_I2, to_dev(np.array([0.02], np.float32)), to_dev(x), N, K,
                                 y_dtype=torch.int32))
        assert np.array_equal(acc, ref["acc"])
