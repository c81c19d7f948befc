"""GPU parity: every entry point of libbitlinear against the CPU oracle,
element by element, on seeded inputs that span several tiles, ragged tails and
the degenerate cases.  Integer, byte and index outputs must be bit-exact; the
fp32 output within 1e-5 relative (and, by construction, bit-identical); the
bf16 output within 2e-2 relative (and identical).  Calls go through the C ABI
(the ctypes binding)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import (DEV, assert_bf16_parity, assert_f32_parity, f32_bits, to_dev,  # noqa: E402
                         to_host)

pytestmark = pytest.mark.gpu

LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3}


def log(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------
# weight ternarisation
# ---------------------------------------------------------------------------
def weight_cases():
    yield "tiny_512x256", synth.latent_weights(512, 256, seed=1)
    yield "ragged_17x65", synth.latent_weights(17, 65, seed=2)
    yield "one", np.array([[0.37]], np.float32)
    yield "ties", np.array([[0.5, 1.5, -0.5, -1.5, 0.0, 1.0, -1.0, 0.5]], np.float32)
    yield "zeros", np.zeros((3, 40), np.float32)
    r = synth.rng(3)
    w = (r.standard_normal((33, 97)) * np.exp2(r.integers(-140, 40, (33, 97)))).astype(np.float32)
    yield "wide_exponents", w
    yield "subnormal", (r.standard_normal((8, 70)) * 1e-42).astype(np.float32)
    yield "constant", np.where(r.random((20, 30)) < 0.5, -0.02, 0.02).astype(np.float32)
    yield "rows_3200x3200", synth.latent_weights(3200, 3200, seed=4)


@pytest.mark.parametrize("name,w", list(weight_cases()), ids=[c[0] for c in weight_cases()])
def test_quantize_weights(name, w):
    log("quantize_weights", name, w.shape)
    T, gamma = bl.quantize_weights(to_dev(w))
    torch.cuda.synchronize()
    t_ref, g_ref = oracle.quantize_weights(w)
    assert to_host(gamma).view(np.uint32)[0] == np.array(g_ref, np.float32).view(np.uint32)
    assert np.array_equal(to_host(T), t_ref)


def test_quantize_weights_strided():
    w = synth.latent_weights(40, 200, seed=5)
    wd = to_dev(w)[:, :150]  # row stride 200, K = 150
    T, gamma = bl.quantize_weights(wd)
    t_ref, g_ref = oracle.quantize_weights(np.ascontiguousarray(w[:, :150]))
    assert to_host(gamma)[0] == g_ref
    assert np.array_equal(to_host(T), t_ref)


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["i2", "b3"])
@pytest.mark.parametrize("N,K", [(1, 1), (16, 64), (17, 65), (33, 80), (48, 257), (100, 1000), (512, 256)])
def test_pack(layout, N, K):
    t = synth.ternary_weights(N, K, seed=N * 7 + K)
    P = bl.pack(to_dev(t), LAYOUTS[layout])
    assert np.array_equal(to_host(P), oracle.pack(t, LAYOUTS[layout]))


def test_pack_strided():
    t = synth.ternary_weights(20, 300, seed=9)
    P = bl.pack(to_dev(t)[:, :250], bl.LAYOUT_I2)
    assert np.array_equal(to_host(P), oracle.pack(np.ascontiguousarray(t[:, :250]), bl.LAYOUT_I2))


# ---------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------
def act_cases():
    yield "f32_16x256", synth.activations_f32(16, 256, seed=11)
    yield "bf16_16x3200", synth.activations_bf16(16, 3200, seed=12)
    yield "bf16_ragged_5x77", synth.activations_bf16(5, 77, seed=13)
    yield "bf16_1x1", synth.activations_bf16(1, 1, seed=14)
    yield "student_t_64x8640", synth.activations_student_t_bf16(64, 8640, seed=15)
    x = synth.activations_f32(6, 300, seed=16)
    x[0] = 0.0                                       # zero row
    x[1, :7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0]
    x[1, 7:] = 0.0                                   # exact ties
    x[2] = (x[2] * 1e-40).astype(np.float32)         # subnormal row
    x[3] = np.float32(-3.0)                          # constant row
    yield "f32_edges", x
    # 64 tokens or more: a wave per row (k_quant_act_rows), the same bits
    yield "bf16_prefill_2048x3200", synth.activations_student_t_bf16(2048, 3200, seed=17)
    yield "f32_100x2048", synth.activations_f32(100, 2048, seed=18)
    yield "bf16_70x12288", synth.activations_bf16(70, 12288, seed=19)
    yield "bf16_65x12296_vec_path", synth.activations_bf16(65, 12296, seed=20)
    x = synth.activations_f32(67, 300, seed=21)      # 67 rows: the last workgroup partly empty
    x[0] = 0.0
    x[1, :7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0]
    x[1, 7:] = 0.0
    x[2] = (x[2] * 1e-40).astype(np.float32)
    x[3] = np.float32(-3.0)
    x[4] = np.float32(-0.0)
    x[66, 5] = np.float32(3e38)
    yield "f32_edges_67x300", x
    xb = synth.activations_bf16(64, 1000, seed=22)
    xb[7] = 0x8000                                   # bf16 -0.0 row
    xb[9, 3] = 0x7f7f                                # bf16 largest finite
    yield "bf16_edges_64x1000", xb
    # prefill-sized row counts that leave the last workgroup partly empty,
    # with edge rows among the last ones
    yield "bf16_1501x3200_ragged", synth.activations_student_t_bf16(1501, 3200, seed=23)
    x = synth.activations_f32(2053, 1000, seed=24)
    for r in (0, 2049, 2052):
        x[r] = 0.0
        x[r, :7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0]
    x[2050] = (x[2050] * 1e-40).astype(np.float32)  # subnormal row
    x[2051] = np.float32(-0.0)
    x[5] = (x[5] * 1e-38).astype(np.float32)        # beta below 127 / FLT_MAX
    yield "f32_edges_2053x1000", x


@pytest.mark.parametrize("name,x", list(act_cases()), ids=[c[0] for c in act_cases()])
def test_quantize_act(name, x):
    log("quantize_act", name, x.shape)
    Xq, beta = bl.quantize_act(to_dev(x))
    q_ref, b_ref = oracle.quantize_act(x)
    K = x.shape[1]
    xq = to_host(Xq)
    assert np.array_equal(xq[:, :K], q_ref)
    assert not xq[:, K:].any()
    assert np.array_equal(f32_bits(to_host(beta)), f32_bits(b_ref))


def untile(xt: np.ndarray, M: int, K: int, layout: str) -> np.ndarray:
    """Read q[m][k] back out of the tiled activation layout (the byte formula of
    bitlinear_act_tiled_bytes), and check that every other byte is zero."""
    S, F = (256, 4) if layout == "i2" else (320, 5)
    nsteps = -(-K // S)
    G = -(-M // 16)
    m = np.arange(G * 16)[:, None]
    k = np.arange(nsteps * S)[None, :]
    s, r = k // S, k % S
    g, r2 = r // (S // 4), r % (S // 4)
    d, e = r2 // 16, r2 % 16
    off = ((((m // 16) * nsteps + s) * F + d) * 64 + g * 16 + (m % 16)) * 16 + e
    full = xt[off]
    assert off.size == xt.size and np.unique(off).size == off.size
    assert not full[M:, :].any() and not full[:, K:].any()
    return full[:M, :K]


@pytest.mark.parametrize("layout", ["i2", "b3"])
@pytest.mark.parametrize("M,K,kind", [(16, 256, "f32"), (5, 3200, "bf16"), (20, 333, "bf16"), (1, 80, "f32"),
                                      (33, 8192, "bf16"), (3, 28672, "bf16"), (5, 65500, "f32"), (2, 65536, "bf16")])
def test_quantize_act_tiled(layout, M, K, kind):
    log("quantize_act_tiled", layout, M, K, kind)
    x = synth.activations_f32(M, K, seed=M + K) if kind == "f32" else synth.activations_bf16(M, K, seed=M + K)
    Xt, beta = bl.quantize_act_tiled(to_dev(x), LAYOUTS[layout])
    q_ref, b_ref = oracle.quantize_act(x)
    assert np.array_equal(untile(to_host(Xt), M, K, layout), q_ref)
    assert np.array_equal(f32_bits(to_host(beta)), f32_bits(b_ref))


@pytest.mark.parametrize("layout", ["i2", "b3"])
@pytest.mark.parametrize("M,N,K", [(16, 512, 256), (7, 100, 333), (40, 260, 700), (1, 48, 3200)])
def test_forward_tiled_input(layout, M, N, K):
    log("forward tiled", layout, M, N, K)
    t = synth.ternary_weights(N, K, seed=N + K)
    x = synth.activations_bf16(M, K, seed=M * 3 + K)
    ref = oracle.forward(t, np.float32(0.03), x)
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([0.03], np.float32))
    Xt, beta = bl.quantize_act_tiled(to_dev(x), LAYOUTS[layout])
    acc = to_host(bl.forward(P, LAYOUTS[layout], gamma, Xt, N, K, beta=beta, y_dtype=torch.int32))
    assert np.array_equal(acc, ref["acc"])
    y = to_host(bl.forward(P, LAYOUTS[layout], gamma, Xt, N, K, beta=beta))
    assert_f32_parity(y, ref["y"])


# ---------------------------------------------------------------------------
# forward: every kernel, several tiles, ragged tails
# ---------------------------------------------------------------------------
FWD_SHAPES = [  # (M, N, K)
    (1, 16, 64), (1, 50, 100), (2, 333, 257), (3, 64, 1000), (4, 130, 3200), (5, 17, 65),
    (8, 200, 640), (11, 48, 1), (16, 512, 256), (16, 100, 333),
]
ALGOS_SMALL = [("addsub", bl.ALGO_GEMV_ADDSUB, "i2"), ("mfma_gemv", bl.ALGO_GEMV_MFMA, "i2"),
               ("mfma_gemv", bl.ALGO_GEMV_MFMA, "b3"), ("gemm", bl.ALGO_GEMM_MFMA, "i2"),
               ("gemm", bl.ALGO_GEMM_MFMA, "b3"), ("auto", bl.ALGO_AUTO, "i2"), ("auto", bl.ALGO_AUTO, "b3")]


def run_forward_case(M, N, K, algo, layout, seed, x_kind="bf16", y_kinds=("i32", "f32", "bf16")):
    t = synth.ternary_weights(N, K, seed=seed)
    w_scale = np.float32(0.0123)
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([w_scale], np.float32))
    if x_kind == "bf16":
        x = synth.activations_bf16(M, K, seed=seed + 1)
    else:
        x = synth.activations_f32(M, K, seed=seed + 1)
    ref = oracle.forward(t, w_scale, x)
    xd = to_dev(x)
    for yk in y_kinds:
        ydt = {"i32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16}[yk]
        Y = bl.forward(P, LAYOUTS[layout], gamma, xd, N, K, y_dtype=ydt, algo=algo)
        y = to_host(Y)
        if yk == "i32":
            assert np.array_equal(y, ref["acc"]), f"acc mismatch at {np.argwhere(y != ref['acc'])[:5]}"
        elif yk == "f32":
            assert_f32_parity(y, ref["y"])
        else:
            assert_bf16_parity(y, ref["y"], oracle.f32_to_bf16(ref["y"]))


@pytest.mark.parametrize("algo_name,algo,layout", ALGOS_SMALL, ids=[f"{a}-{l}-{c}" for a, c, l in ALGOS_SMALL])
@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_forward_small(algo_name, algo, layout, M, N, K):
    log("forward", algo_name, layout, M, N, K)
    run_forward_case(M, N, K, algo, layout, seed=M * 10007 + N * 31 + K)


@pytest.mark.parametrize("algo_name,algo,layout", [("mfma_gemv", bl.ALGO_GEMV_MFMA, "i2"),
                                                   ("mfma_gemv", bl.ALGO_GEMV_MFMA, "b3"),
                                                   ("gemm", bl.ALGO_GEMM_MFMA, "i2"),
                                                   ("gemm", bl.ALGO_GEMM_MFMA, "b3")])
@pytest.mark.parametrize("M,N,K", [(17, 40, 100), (64, 96, 512), (130, 257, 700), (256, 128, 64), (40, 2000, 300)])
def test_forward_many_tokens(algo_name, algo, layout, M, N, K):
    log("forward", algo_name, layout, M, N, K)
    run_forward_case(M, N, K, algo, layout, seed=M * 131 + N + K)


@pytest.mark.parametrize("M,N,K", [(1100, 5000, 200), (4000, 4000, 130), (2048, 3200, 320), (150, 6000, 300),
                                   (100, 9000, 200), (1000, 8640, 330), (2048, 8640, 200)],
                         ids=["tile128x256", "tile256x256_odd_kb", "prefill_rows", "tile32x128_skinny",
                              "tile32x128_one_block", "tile160x256_ragged", "tile160x256_prefill_rows"])
def test_gemm_tile_shapes(M, N, K):
    """Sizes whose workgroup-tile choice differs (128x256, 256x256, 160x256 and
    32x128 tiles, ragged in M and N; an odd number of k-blocks ends in a half
    stage)."""
    log("forward gemm tiles", M, N, K, bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMM_MFMA))
    run_forward_case(M, N, K, bl.ALGO_GEMM_MFMA, "i2", seed=M + 7 * N + K, y_kinds=("i32", "f32"))
    if M * N <= 1100 * 5000:  # base-3 weights, decoded inside the GEMM
        run_forward_case(M, N, K, bl.ALGO_GEMM_MFMA, "b3", seed=M + 7 * N + K + 1, y_kinds=("i32",))


# (M, N, K) for the base-3 GEMM, whose stage is two 80-weight k-blocks:
# one block (a half stage), exactly one stage, an odd block count (the last
# stage half empty), K inside a block (pad bytes), K < 16, many stages, and
# each b3 tile shape (32 x 128, 64 x 128, 128 x 128, 128 x 256), ragged in M
# and N.
# The GEMM decodes b3 itself at every token count (no weight rewrite): the
# last four shapes meet a weight tile with many token blocks.
B3_GEMM_SHAPES = [(33, 200, 80, "b3"), (40, 130, 160, "b3"), (64, 257, 240, "b3"), (64, 300, 1001, "b3"),
                  (17, 16, 7, "b3"), (64, 2000, 3200, "b3"), (129, 13500, 170, "b3"), (200, 26500, 250, "b3"),
                  (64, 20000, 100, "b3"), (50, 20000, 250, "b3"),
                  (100, 96, 1001, "b3"), (300, 520, 3200, "b3"), (700, 9000, 333, "b3"), (2048, 3200, 320, "b3")]


@pytest.mark.parametrize("M,N,K,kernel", B3_GEMM_SHAPES)
def test_gemm_b3(M, N, K, kernel):
    kname = bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_B3, bl.BF16, bl.ALGO_GEMM_MFMA)
    log("forward gemm b3", M, N, K, kname)
    assert kname.startswith(f"bl::k_gemm_mfma_{kernel}<")
    run_forward_case(M, N, K, bl.ALGO_GEMM_MFMA, "b3", seed=3 * M + N + 11 * K, y_kinds=("i32", "f32"))


@pytest.mark.parametrize("K", [80, 240, 1001])
def test_gemm_b3_int8_tight_rows(K):
    """Pre-quantised rows only 16-byte padded: the last stage's 160-byte
    activation reads run into the next row or past the buffer, where the
    weights are zero (pad bytes, or a missing k-block's zero word)."""
    M, N = 50, 300
    assert bl.bitlinear_product_kernel(M, N, K, bl.LAYOUT_B3, bl.I8, bl.ALGO_GEMM_MFMA).startswith("bl::k_gemm_mfma_b3<")
    t = synth.ternary_weights(N, K, seed=K + 5)
    x = synth.activations_bf16(M, K, seed=K + 6)
    ref = oracle.forward(t, np.float32(0.02), x)
    Xq, beta = bl.quantize_act(to_dev(x))
    ld = (K + 15) // 16 * 16
    xt = torch.zeros((M, ld), dtype=torch.int8, device="cuda")
    xt[:, :K] = Xq[:, :K]
    assert xt.stride(0) == ld
    P = to_dev(oracle.pack(t, bl.LAYOUT_B3))
    gamma = to_dev(np.array([0.02], np.float32))
    acc = to_host(bl.forward(P, bl.LAYOUT_B3, gamma, xt, N, K, beta=beta, y_dtype=torch.int32,
                             algo=bl.ALGO_GEMM_MFMA))
    assert np.array_equal(acc, ref["acc"])
    # the same with garbage (not zero) bytes between K and the row stride
    xt[:, K:] = 77
    acc = to_host(bl.forward(P, bl.LAYOUT_B3, gamma, xt, N, K, beta=beta, y_dtype=torch.int32,
                             algo=bl.ALGO_GEMM_MFMA))
    assert np.array_equal(acc, ref["acc"])


@pytest.mark.parametrize("layout", ["i2", "b3"])
@pytest.mark.parametrize("M,N,K", [(20, 16400, 300), (64, 16390, 70), (16, 8200, 100), (5, 16384, 1000)])
def test_forward_wide_short(layout, M, N, K):
    """Many row tiles and few k-steps: a workgroup owns several tiles and may
    have fewer waves than tiles."""
    log("forward wide", layout, M, N, K)
    run_forward_case(M, N, K, bl.ALGO_GEMV_MFMA, layout, seed=M + N + K, y_kinds=("i32", "f32"))


@pytest.mark.parametrize("layout", ["i2", "b3"])
@pytest.mark.parametrize("x_kind", ["bf16", "f32"])
@pytest.mark.parametrize("M,N,K", [(1, 300, 1024), (7, 1000, 2000), (16, 8200, 3200), (16, 9000, 9984),
                                   (3, 2048, 9920)])
def test_forward_gemv_float_input(layout, x_kind, M, N, K):
    """bf16/fp32 activations of at most 16 tokens through the matrix-core GEMV
    (per-tile and persistent kernels, K near 10^4)."""
    log("forward gemv float input", layout, x_kind, M, N, K)
    run_forward_case(M, N, K, bl.ALGO_GEMV_MFMA, layout, seed=M + N + 3 * K, x_kind=x_kind, y_kinds=("i32", "f32"))


def test_forward_gemv_strided_f32():
    """Rows of a wider fp32 matrix (the stack's o and down inputs): row stride
    larger than K."""
    M, N, K, ldx = 16, 640, 800, 1200
    t = synth.ternary_weights(N, K, seed=91)
    xw = synth.activations_f32(M, ldx, seed=92)
    ref = oracle.forward(t, np.float32(0.02), np.ascontiguousarray(xw[:, :K]))
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.02], np.float32))
    xd = to_dev(xw)[:, :K]
    acc = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, xd, N, K, y_dtype=torch.int32, algo=bl.ALGO_GEMV_MFMA))
    assert np.array_equal(acc, ref["acc"])
    y = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, xd, N, K, algo=bl.ALGO_GEMV_MFMA))
    assert_f32_parity(y, ref["y"])


def test_forward_f32_input_tiny():
    run_forward_case(16, 512, 256, bl.ALGO_AUTO, "i2", seed=77, x_kind="f32")


def test_forward_int8_input():
    M, N, K = 6, 80, 300
    t = synth.ternary_weights(N, K, seed=81)
    x = synth.activations_bf16(M, K, seed=82)
    ref = oracle.forward(t, np.float32(0.02), x)
    Xq, beta = bl.quantize_act(to_dev(x))
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.02], np.float32))
    for algo in (bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        Y = bl.forward(P, bl.LAYOUT_I2, gamma, Xq, N, K, beta=beta, algo=algo)
        assert_f32_parity(to_host(Y), ref["y"])


def test_forward_degenerate():
    # zero activations row and all-zero weights
    M, N, K = 4, 32, 128
    x = synth.activations_bf16(M, K, seed=91)
    x[2] = 0
    t = np.zeros((N, K), np.int8)
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.0], np.float32))
    for algo in (bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        y = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, to_dev(x), N, K, algo=algo))
        assert not y.any() and not np.signbit(y).any()
    # all +1 weights: the product is the row sum of q
    t = np.ones((N, K), np.int8)
    ref = oracle.forward(t, np.float32(1.0), x)
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([1.0], np.float32))
    for algo in (bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        acc = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, to_dev(x), N, K, y_dtype=torch.int32, algo=algo))
        assert np.array_equal(acc, ref["acc"])


@pytest.mark.parametrize("layout", ["i2", "b3"])
def test_forward_max_k(layout):
    """K = BITLINEAR_MAX_K: the row-major staging (K beyond the tiled
    quantiser's range), and the largest accumulator the contract allows,
    127 * K = 16,646,144 < 2^24, which float(acc) still represents exactly."""
    M, N, K = 3, 40, bl.MAX_K
    t = synth.ternary_weights(N, K, seed=101)
    t[0] = 1                                        # row 0: all +1
    x = synth.activations_bf16(M, K, seed=102)
    x[1] = synth.to_bf16_bits(np.full(K, 0.75, np.float32))  # token 1: every q = 127
    ref = oracle.forward(t, np.float32(0.03), x)
    assert ref["acc"][1, 0] == 127 * K
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([0.03], np.float32))
    algos = [bl.ALGO_AUTO, bl.ALGO_GEMV_MFMA] + ([bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMM_MFMA] if layout == "i2" else [])
    for algo in algos:
        acc = to_host(bl.forward(P, LAYOUTS[layout], gamma, to_dev(x), N, K, y_dtype=torch.int32, algo=algo))
        assert np.array_equal(acc, ref["acc"]), algo
        y = to_host(bl.forward(P, LAYOUTS[layout], gamma, to_dev(x), N, K, algo=algo))
        assert_f32_parity(y, ref["y"])


def test_forward_max_m():
    """M = BITLINEAR_MAX_M tokens: 4096 token groups for the GEMV, 256-token
    tiles for the GEMM."""
    M, N, K = bl.MAX_M, 48, 72
    t = synth.ternary_weights(N, K, seed=103)
    x = synth.activations_bf16(M, K, seed=104)
    ref = oracle.forward(t, np.float32(0.01), x)
    gamma = to_dev(np.array([0.01], np.float32))
    for layout, algo in (("i2", bl.ALGO_AUTO), ("i2", bl.ALGO_GEMV_MFMA), ("b3", bl.ALGO_AUTO)):
        P = to_dev(oracle.pack(t, LAYOUTS[layout]))
        acc = to_host(bl.forward(P, LAYOUTS[layout], gamma, to_dev(x), N, K, y_dtype=torch.int32, algo=algo))
        assert np.array_equal(acc, ref["acc"]), (layout, algo)


def test_forward_strided_output_and_input():
    M, N, K = 16, 96, 200
    t = synth.ternary_weights(N, K, seed=95)
    x = synth.activations_bf16(M, 256, seed=96)
    ref = oracle.forward(t, np.float32(0.5), np.ascontiguousarray(x[:, :K]))
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.5], np.float32))
    xd = to_dev(x)[:, :K]
    out = torch.full((M, 128), -7.0, dtype=torch.float32, device=DEV)
    for algo in (bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        bl.forward(P, bl.LAYOUT_I2, gamma, xd, N, K, algo=algo, out=out[:, :N])
        o = to_host(out)
        assert_f32_parity(o[:, :N], ref["y"])
        assert np.all(o[:, N:] == -7.0)


def test_forward_deterministic():
    M, N, K = 16, 1024, 3200
    t = synth.ternary_weights(N, K, seed=97)
    x = to_dev(synth.activations_bf16(M, K, seed=98))
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.01], np.float32))
    for algo in (bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA):
        a = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, x, N, K, algo=algo))
        b = to_host(bl.forward(P, bl.LAYOUT_I2, gamma, x, N, K, algo=algo))
        assert np.array_equal(f32_bits(a), f32_bits(b))
