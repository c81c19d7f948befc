"""The C ABI without a GPU: the library loads, exports every function declared
in include/bitlinear.h, and rejects invalid arguments on the host before any
HIP call.  Pointer arguments here are fake addresses that are never touched."""
import os
import re

import pytest

from ternary_weight_linear_forward_amd import bitlinear as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

A = 0x10000  # 16-byte aligned fake device addresses, far apart
B = 0x20000000
C = 0x40000000
D = 0x60000000
E = 0x80000000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    declared = header_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(bl._lib, name), name
    assert sorted(declared) == sorted(bl.EXPORTED)


def test_status_strings_and_version():
    assert bl.bitlinear_status_string(bl.OK) == "ok"
    for s in range(1, 6):
        assert bl.bitlinear_status_string(s) not in ("ok", "unknown status")
    assert bl.bitlinear_status_string(99) == "unknown status"
    assert bl.bitlinear_version() >= 100


def test_size_queries():
    assert bl.bitlinear_packed_bytes(3200, 3200, bl.LAYOUT_I2) == 3200 * 3200 // 4
    assert bl.bitlinear_packed_bytes(28672, 8192, bl.LAYOUT_B3) == 28672 * 103 * 16
    assert bl.bitlinear_packed_bytes(17, 65, bl.LAYOUT_I2) == 2 * 2 * 256
    assert bl.bitlinear_packed_bytes(3200, 3200, bl.LAYOUT_B1) == 3200 * 25 * 16
    assert bl.bitlinear_packed_bytes(17, 129, bl.LAYOUT_B1) == 2 * 2 * 256
    assert bl.bitlinear_packed_bytes(0, 4, bl.LAYOUT_I2) == -1
    assert bl.bitlinear_packed_bytes(4, bl.MAX_K + 1, bl.LAYOUT_I2) == -1
    assert bl.bitlinear_packed_bytes(4, 4, 7) == -1
    assert bl.bitlinear_quantize_weights_workspace_bytes(10, 10) == 2048
    assert bl.bitlinear_quantize_weights_workspace_bytes(1 << 21, 1 << 20) == -1
    assert bl.bitlinear_forward_workspace_bytes(16, 100, 100, bl.LAYOUT_I2, bl.I8) == 0
    assert bl.bitlinear_forward_workspace_bytes(16, 100, 100, bl.LAYOUT_I2, bl.BF16) >= 16 * 100 + 64
    assert bl.bitlinear_forward_workspace_bytes(16, 100, 100, bl.LAYOUT_I2, bl.I32) == -1


def qw(**kw):
    a = dict(W=A, N=64, K=64, ldw=64, T=B, gamma=C, ws=D, ws_bytes=2048, stream=None)
    a.update(kw)
    return bl.bitlinear_quantize_weights(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), bl.ERR_INVALID_ARG), (dict(T=None), bl.ERR_INVALID_ARG), (dict(gamma=None), bl.ERR_INVALID_ARG),
    (dict(N=0), bl.ERR_INVALID_ARG), (dict(K=-1), bl.ERR_INVALID_ARG), (dict(ldw=63), bl.ERR_INVALID_ARG),
    (dict(N=1 << 21, K=1 << 20, ldw=1 << 20), bl.ERR_INVALID_ARG),
    (dict(ldw=(1 << 40) + 64), bl.ERR_INVALID_ARG),             # stride bound
    (dict(ws=None), bl.ERR_WORKSPACE), (dict(ws_bytes=2047), bl.ERR_WORKSPACE),
    (dict(ws=D + 8), bl.ERR_INVALID_ARG), (dict(W=A + 2), bl.ERR_INVALID_ARG),
    (dict(T=A + 64), bl.ERR_INVALID_ARG),       # T overlaps W
    (dict(ws=A), bl.ERR_INVALID_ARG),           # workspace overlaps W
])
def test_quantize_weights_rejects(kw, status):
    assert qw(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(W=None), bl.ERR_INVALID_ARG), (dict(N=0), bl.ERR_INVALID_ARG), (dict(ldw=63), bl.ERR_INVALID_ARG),
    (dict(ws_bytes=2047), bl.ERR_WORKSPACE), (dict(T=A + 64), bl.ERR_INVALID_ARG),
])
def test_binarize_weights_rejects(kw, status):
    a = dict(W=A, N=64, K=64, ldw=64, T=B, gamma=C, ws=D, ws_bytes=2048, stream=None)
    a.update(kw)
    assert bl.bitlinear_binarize_weights(**a) == status


def pk(**kw):
    a = dict(T=A, N=64, K=64, ldt=64, layout=bl.LAYOUT_I2, P=B, stream=None)
    a.update(kw)
    return bl.bitlinear_pack(**a)


@pytest.mark.parametrize("kw", [
    dict(T=None), dict(P=None), dict(layout=3), dict(layout=-1), dict(N=0), dict(K=0), dict(K=bl.MAX_K + 1, ldt=bl.MAX_K + 1),
    dict(ldt=10), dict(P=B + 4), dict(P=A + 16), dict(ldt=(1 << 40) + 64),
])
def test_pack_rejects(kw):
    assert pk(**kw) == bl.ERR_INVALID_ARG


def qa(**kw):
    a = dict(X=A, x_dtype=bl.BF16, M=16, K=100, ldx=100, Xq=B, ldq=112, beta=C, stream=None)
    a.update(kw)
    return bl.bitlinear_quantize_act(**a)


@pytest.mark.parametrize("kw", [
    dict(X=None), dict(Xq=None), dict(beta=None), dict(x_dtype=bl.I8), dict(x_dtype=bl.I32), dict(M=0),
    dict(M=bl.MAX_M + 1), dict(K=0), dict(K=bl.MAX_K + 1, ldx=bl.MAX_K + 1, ldq=bl.MAX_K + 16), dict(ldx=99),
    dict(ldq=104), dict(ldq=96), dict(Xq=B + 8), dict(X=A + 1), dict(beta=C + 2), dict(Xq=A + 32),
    dict(ldx=1 << 41), dict(ldq=1 << 42),  # strides beyond 2^40 elements
])
def test_quantize_act_rejects(kw):
    assert qa(**kw) == bl.ERR_INVALID_ARG


def fw(**kw):
    a = dict(P=A, layout=bl.LAYOUT_I2, gamma=B, M=4, N=64, K=64, X=C, x_dtype=bl.BF16, ldx=64, beta_in=None,
             Y=D, y_dtype=bl.F32, ldy=64, ws=E, ws_bytes=1 << 20, algo=bl.ALGO_AUTO, stream=None)
    a.update(kw)
    return bl.bitlinear_forward_algo(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(P=None), bl.ERR_INVALID_ARG), (dict(gamma=None), bl.ERR_INVALID_ARG), (dict(X=None), bl.ERR_INVALID_ARG),
    (dict(Y=None), bl.ERR_INVALID_ARG), (dict(layout=5), bl.ERR_INVALID_ARG), (dict(M=0), bl.ERR_INVALID_ARG),
    (dict(M=bl.MAX_M + 1), bl.ERR_INVALID_ARG), (dict(N=0), bl.ERR_INVALID_ARG), (dict(K=0), bl.ERR_INVALID_ARG),
    (dict(K=bl.MAX_K + 1, ldx=bl.MAX_K + 1), bl.ERR_INVALID_ARG), (dict(x_dtype=bl.I32), bl.ERR_INVALID_ARG),
    (dict(y_dtype=bl.I8), bl.ERR_INVALID_ARG), (dict(ldx=63), bl.ERR_INVALID_ARG), (dict(ldy=63), bl.ERR_INVALID_ARG),
    (dict(algo=9), bl.ERR_INVALID_ARG), (dict(algo=-1), bl.ERR_INVALID_ARG),
    (dict(ldx=1 << 41), bl.ERR_INVALID_ARG), (dict(ldy=1 << 41), bl.ERR_INVALID_ARG),  # stride bound
    (dict(M=40000, ldy=1 << 30), bl.ERR_INVALID_ARG),               # rows x stride beyond 2^44
    (dict(x_dtype=bl.I8), bl.ERR_INVALID_ARG),                      # I8 needs beta_in
    (dict(beta_in=A + 0x100000), bl.ERR_INVALID_ARG),               # bf16 must not pass beta_in
    (dict(x_dtype=bl.I8, beta_in=B + 64, ldx=72), bl.ERR_INVALID_ARG),  # I8 rows must be 16-aligned
    (dict(x_dtype=bl.I8, beta_in=B + 64, X=C + 8), bl.ERR_INVALID_ARG),
    (dict(P=A + 8), bl.ERR_INVALID_ARG), (dict(Y=D + 2), bl.ERR_INVALID_ARG),
    (dict(ws=None), bl.ERR_WORKSPACE), (dict(ws_bytes=64), bl.ERR_WORKSPACE), (dict(ws=E + 8), bl.ERR_INVALID_ARG),
    (dict(Y=C), bl.ERR_INVALID_ARG),                                # Y overlaps X
    (dict(Y=A), bl.ERR_INVALID_ARG),                                # Y overlaps P
    (dict(ws=C), bl.ERR_INVALID_ARG),                               # workspace overlaps X
    (dict(algo=bl.ALGO_GEMV_ADDSUB, M=17), bl.ERR_UNSUPPORTED),
    (dict(algo=bl.ALGO_GEMV_ADDSUB, layout=bl.LAYOUT_B3), bl.ERR_UNSUPPORTED),
])
def test_forward_rejects(kw, status):
    assert fw(**kw) == status


def test_tiled_sizes():
    # I2: 256 weights and 4 operands per k-step; B3: 320 and 5; 1 KiB per operand
    assert bl.bitlinear_act_tiled_bytes(16, 3200, bl.LAYOUT_I2) == 1 * 13 * 4 * 1024
    assert bl.bitlinear_act_tiled_bytes(17, 3200, bl.LAYOUT_I2) == 2 * 13 * 4 * 1024
    assert bl.bitlinear_act_tiled_bytes(1, 8192, bl.LAYOUT_B3) == 1 * 26 * 5 * 1024
    assert bl.bitlinear_act_tiled_bytes(0, 64, bl.LAYOUT_I2) == -1
    assert bl.bitlinear_act_tiled_bytes(4, 64, 3) == -1


def qt(**kw):
    a = dict(X=A, x_dtype=bl.BF16, M=16, K=256, ldx=256, layout=bl.LAYOUT_I2, Xt=B, xt_bytes=4096, beta=C,
             stream=None)
    a.update(kw)
    return bl.bitlinear_quantize_act_tiled(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), bl.ERR_INVALID_ARG), (dict(Xt=None), bl.ERR_INVALID_ARG), (dict(beta=None), bl.ERR_INVALID_ARG),
    (dict(layout=9), bl.ERR_INVALID_ARG), (dict(x_dtype=bl.I8), bl.ERR_INVALID_ARG), (dict(M=0), bl.ERR_INVALID_ARG),
    (dict(ldx=255), bl.ERR_INVALID_ARG), (dict(xt_bytes=4095), bl.ERR_INVALID_ARG), (dict(Xt=B + 4), bl.ERR_INVALID_ARG),
    (dict(Xt=A + 64), bl.ERR_INVALID_ARG),
    (dict(K=70000, ldx=70000, xt_bytes=1 << 30), bl.ERR_UNSUPPORTED),
])
def test_quantize_act_tiled_rejects(kw, status):
    assert qt(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x_dtype=bl.I8_TILED), bl.ERR_INVALID_ARG),                                   # needs beta_in
    (dict(x_dtype=bl.I8_TILED, beta_in=B + 64, X=C + 8), bl.ERR_INVALID_ARG),          # alignment
    (dict(x_dtype=bl.I8_TILED, beta_in=B + 64, algo=bl.ALGO_GEMV_ADDSUB), bl.ERR_UNSUPPORTED),
    (dict(x_dtype=bl.I8_TILED, beta_in=B + 64, algo=bl.ALGO_GEMM_MFMA), bl.ERR_UNSUPPORTED),
    (dict(x_dtype=bl.I8_TILED, beta_in=B + 64, Y=C), bl.ERR_INVALID_ARG),              # Y overlaps X
])
def test_forward_tiled_rejects(kw, status):
    assert fw(**kw) == status


def fx(**kw):
    a = dict(P=A, layout=bl.LAYOUT_I2, gamma=B, M=4, N=64, K=64, X=C, x_dtype=bl.BF16, ldx=64, beta_in=None,
             Y=D, y_dtype=bl.F32, ldy=64, Xq_out=E, ldxq=64, beta_out=E + 0x100000, ws=None, ws_bytes=0,
             algo=bl.ALGO_AUTO, stream=None)
    a.update(kw)
    return bl.bitlinear_forward_ex(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(beta_out=None), bl.ERR_INVALID_ARG),                       # both or neither
    (dict(Xq_out=None), bl.ERR_INVALID_ARG),
    (dict(x_dtype=bl.I8, beta_in=B + 64), bl.ERR_INVALID_ARG),       # int8 input: nothing to return
    (dict(ldxq=48), bl.ERR_INVALID_ARG),                             # ldxq < K
    (dict(ldxq=72), bl.ERR_INVALID_ARG),                             # ldxq % 16
    (dict(Xq_out=E + 8), bl.ERR_INVALID_ARG),                        # alignment
    (dict(beta_out=E + 0x100002), bl.ERR_INVALID_ARG),
    (dict(Xq_out=D), bl.ERR_INVALID_ARG),                            # overlaps Y
    (dict(Xq_out=C), bl.ERR_INVALID_ARG),                            # overlaps X
    (dict(beta_out=E + 16), bl.ERR_INVALID_ARG),                     # overlaps Xq_out
    (dict(beta_out=B), bl.ERR_INVALID_ARG),                          # overlaps gamma
])
def test_forward_ex_rejects(kw, status):
    assert fx(**kw) == status


def test_forward_ex_workspace_is_the_int8_one():
    # with the quantiser's outputs requested the product reads them: a bf16
    # forward needs only the int8 workspace (none for i2 weights)
    assert bl.bitlinear_forward_workspace_bytes(4, 64, 64, bl.LAYOUT_I2, bl.I8) == 0
    assert fx(ws=None, ws_bytes=0, Xq_out=None, beta_out=None) == bl.ERR_WORKSPACE


def test_gemm_rejects_row_offsets_beyond_32_bits():
    # The GEMM addresses the rows of one 256-token tile with 32-bit offsets:
    # caller-quantised rows of stride 2^24 bytes span 255 * 2^24 + K > 2^31
    X = 0x1000000000  # far from every other fake buffer
    kw = dict(x_dtype=bl.I8, X=X, ldx=1 << 24, beta_in=B + 64, M=300, N=4096, K=64, ldy=4096, ws=None, ws_bytes=0)
    assert fw(algo=bl.ALGO_GEMM_MFMA, **kw) == bl.ERR_UNSUPPORTED
    assert fw(algo=bl.ALGO_GEMM_MFMA, **dict(kw, ldx=1 << 20)) != bl.ERR_UNSUPPORTED  # 255 * 2^20 fits
    assert fx(algo=bl.ALGO_GEMM_MFMA, M=300, N=4096, ldy=4096, X=X, ldx=64, ldxq=1 << 24,
              Xq_out=0x3000000000, beta_out=0x2000000000) == bl.ERR_UNSUPPORTED


def test_forward_plain_entry_validates_too():
    assert bl.bitlinear_forward(None, 0, B, 4, 64, 64, C, bl.BF16, 64, None, D, bl.F32, 64, E, 1 << 20, None) \
        == bl.ERR_INVALID_ARG


def test_one_hip_runtime_when_loaded_first():
    """Importing the binding before anything else must still leave a single
    HIP runtime in the process (torch bundles its own libamdhip64)."""
    import subprocess
    import sys
    code = ("from ternary_weight_linear_forward_amd import bitlinear as bl\n"
            "import torch\n"
            "rt = bl._hip_runtimes_loaded()\n"
            "assert len(rt) == 1, rt\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]


def test_auto_algo_dispatch():
    """Host-side dispatch query: the GEMV for few tokens, pre-tiled input and
    b3; the GEMM only when it fills the GPU with workgroup tiles."""
    f = bl.bitlinear_auto_algo
    for M in (1, 4, 16):
        assert f(M, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == bl.ALGO_GEMV_MFMA
    assert f(2048, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == bl.ALGO_GEMM_MFMA
    assert f(2048, 3200, 3200, bl.LAYOUT_B3, bl.BF16) == bl.ALGO_GEMM_MFMA  # decoded inside the GEMM
    assert f(2048, 3200, 3200, bl.LAYOUT_B1, bl.BF16) == bl.ALGO_GEMM_MFMA  # decoded inside the GEMM
    assert f(16, 3200, 3200, bl.LAYOUT_B1, bl.BF16) == bl.ALGO_GEMV_MFMA
    assert f(2048, 3200, 3200, bl.LAYOUT_I2, bl.I8_TILED) == bl.ALGO_GEMV_MFMA
    assert f(176, 1024, 8192, bl.LAYOUT_I2, bl.BF16) == bl.ALGO_GEMV_MFMA  # 16 tiles: GPU mostly idle
    assert f(176, 8192, 8192, bl.LAYOUT_I2, bl.BF16) == bl.ALGO_GEMM_MFMA
    assert f(64, 28672, 8192, bl.LAYOUT_I2, bl.BF16) == bl.ALGO_GEMM_MFMA
    assert f(0, 16, 16, bl.LAYOUT_I2, bl.BF16) == -1
    assert f(16, 16, 16, 7, bl.BF16) == -1
    assert f(16, 16, 16, bl.LAYOUT_I2, 9) == -1


def test_backward_kernel_names():
    """dX takes the small-batch kernel while its 128 x 128 tiles number fewer
    than 256 (the vector-ALU one for one token), dW below 32 tokens; None
    for sizes the calls reject."""
    f = bl.bitlinear_backward_kernel
    assert f(1, 3200, 3200, 0) == "bl::k_bwd_dx_vec<1>"  # one token: vector ALU
    assert f(2, 3200, 3200, 0) == "bl::k_bwd_dx_few"
    assert f(1, 100, 40000, 0) == "bl::k_bwd_dx"  # 313 column tiles
    assert f(2048, 3200, 3200, 0) == "bl::k_bwd_dx"  # 16 x 25 = 400 tiles
    assert f(1280, 3200, 3200, 0) == "bl::k_bwd_dx_few"  # 10 x 25 = 250 tiles
    assert f(1408, 3200, 3200, 0) == "bl::k_bwd_dx"  # 11 x 25 = 275 tiles
    assert f(176, 8192, 8192, 0) == "bl::k_bwd_dx_few"
    assert f(1, 3200, 3200, 1) == "bl::k_bwd_dw_vec"  # one token: an outer product
    assert f(2, 3200, 3200, 1) == "bl::k_bwd_dw_few"
    assert f(31, 3200, 3200, 1) == "bl::k_bwd_dw_few"
    assert f(32, 3200, 3200, 1) == "bl::k_bwd_dw"
    assert f(0, 3200, 3200, 0) is None and f(4, 3200, 3200, 2) is None and f(4, 0, 3200, 1) is None


def test_product_kernel_names():
    """The kernel-name query follows the dispatch: GEMV kernels for few tokens
    (the persistent one for wide layers), GEMM tiles for prefill, the add/sub
    kernel on request; None for requests the library rejects."""
    f = bl.bitlinear_product_kernel
    # 1-4 tokens of float input: the GEMV with the quantiser inside (aligned rows)
    assert f(1, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemv_fq<0, 1, 1>"  # 13 waves of one k-step
    assert f(4, 3200, 8640, bl.LAYOUT_I2, bl.F32) == "bl::k_gemv_fq<0, 0, 4>"
    assert f(1, 3200, 3200, bl.LAYOUT_B3, bl.BF16) == "bl::k_gemv_fq<1, 1, 1>"
    assert f(1, 3200, 8640, bl.LAYOUT_B3, bl.BF16) == "bl::k_gemv_fq<1, 1, 2>"  # 16 waves of two
    assert f(1, 3200, 3200, bl.LAYOUT_I2, bl.I8) == "bl::k_gemv_mfma<0, 1, 1, false>"
    assert f(1, 8640, 3200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemv_persist_fq<0, 1, 1, 8, true>"
    assert f(1, 8640, 3200, bl.LAYOUT_I2, bl.I8).startswith("bl::k_gemv_persist<0, ")
    assert f(1, 28672, 8192, bl.LAYOUT_I2, bl.BF16).startswith("bl::k_gemv_persist<0, ")  # LDS: two launches
    assert f(16, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemv_mfma<0, 1, 1, true>"
    assert f(5, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemv_mfma<0, 1, 1, true>"  # one launch only up to 4 tokens
    assert f(16, 3200, 3200, bl.LAYOUT_I2, bl.I8) == "bl::k_gemv_mfma<0, 1, 1, false>"
    assert f(16, 28672, 8192, bl.LAYOUT_B3, bl.BF16).startswith("bl::k_gemv_persist<1, ")
    assert f(2048, 3200, 3200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemm_mfma_i2<128, 256, 2, 4, 1>"
    assert f(64, 28672, 8192, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemm_mfma_i2<32, 128, 1, 4, 1>"
    assert f(100, 9000, 200, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemm_mfma_i2<32, 128, 1, 4, 1>"
    assert f(64, 8192, 8192, bl.LAYOUT_I2, bl.BF16).startswith("bl::k_gemv_mfma<")  # too few tiles
    assert f(150, 6000, 300, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemm_mfma_i2<32, 128, 1, 4, 1>"
    assert f(3, 64, 64, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMV_ADDSUB) == "bl::k_gemv_addsub<4>"
    assert f(3, 64, 64, bl.LAYOUT_B3, bl.BF16, bl.ALGO_GEMM_MFMA) == "bl::k_gemm_mfma_b3<32, 128, 1, 4, 1>"
    assert f(3, 64, 64, bl.LAYOUT_B1, bl.BF16, bl.ALGO_GEMM_MFMA) == "bl::k_gemm_mfma_b1<32, 128, 1, 4, 1>"
    # b3 and b1 are decoded in the GEMM at every token count (b3: tiles other
    # than 256 x 256)
    assert f(64, 28672, 8192, bl.LAYOUT_B3, bl.BF16) == "bl::k_gemm_mfma_b3<64, 128, 1, 4, 1>"  # b3 only
    assert f(176, 28672, 8192, bl.LAYOUT_B3, bl.BF16) == "bl::k_gemm_mfma_b3<128, 256, 2, 4, 1>"
    assert f(176, 8192, 8192, bl.LAYOUT_B3, bl.BF16).startswith("bl::k_gemm_mfma_b3<")
    assert f(2048, 3200, 3200, bl.LAYOUT_B3, bl.BF16) == "bl::k_gemm_mfma_b3<128, 256, 2, 4, 1>"
    assert f(4000, 4000, 130, bl.LAYOUT_I2, bl.BF16) == "bl::k_gemm_mfma_i2<256, 256, 2, 2, 1>"
    assert f(2048, 3200, 3200, bl.LAYOUT_B1, bl.BF16) == "bl::k_gemm_mfma_b1<128, 256, 2, 4, 1>"
    assert f(1, 3200, 3200, bl.LAYOUT_B1, bl.BF16) == "bl::k_gemv_fq<2, 1, 1>"
    assert f(1, 3200, 3200, bl.LAYOUT_B1, bl.I8) == "bl::k_gemv_mfma<2, 1, 1, false>"
    assert f(3, 64, 64, bl.LAYOUT_B1, bl.BF16, bl.ALGO_GEMV_ADDSUB) is None
    assert f(0, 64, 64, bl.LAYOUT_I2, bl.BF16) is None


def test_backward_rejects():
    """Argument checks of the two backward entry points (no kernel runs)."""
    dx = dict(P=A, layout=bl.LAYOUT_I2, gamma=C, M=4, N=64, K=64, dY=B, lddy=64, dX=D, lddx=64, ws=None, ws_bytes=0,
              stream=None)
    assert bl.bitlinear_backward_dx(**{**dx, "P": None}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "layout": 3}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "lddy": 63}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "lddx": 63}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "lddx": 1 << 41}) == bl.ERR_INVALID_ARG  # stride bound
    assert bl.bitlinear_backward_dx(**{**dx, "lddy": 1 << 42}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "M": 0}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dx(**{**dx, "dX": B + 64}) == bl.ERR_INVALID_ARG  # overlaps dY
    assert bl.bitlinear_backward_dx(**{**dx, "layout": bl.LAYOUT_B3}) == bl.ERR_WORKSPACE
    assert bl.bitlinear_backward_dx_workspace_bytes(4, 64, 64, bl.LAYOUT_I2) == 0
    assert bl.bitlinear_backward_dx_workspace_bytes(4, 64, 64, bl.LAYOUT_B3) == bl.bitlinear_packed_bytes(64, 64, 0)
    assert bl.bitlinear_backward_dx_workspace_bytes(4, 0, 64, bl.LAYOUT_B3) == -1
    assert bl.bitlinear_backward_dx_workspace_bytes(0, 64, 64, bl.LAYOUT_I2) == -1
    # small batches split the weight rows (at least 8 row tiles per split, at
    # most 16 splits, about 512 workgroups) and keep fp32 partials per split
    ws = bl.bitlinear_backward_dx_workspace_bytes
    assert ws(1, 3200, 3200, bl.LAYOUT_I2) == 11 * 1 * 3200 * 4  # 50 workgroups -> 11 splits
    assert ws(16, 8640, 3200, bl.LAYOUT_I2) == 11 * 16 * 3200 * 4
    assert ws(5, 1000, 130, bl.LAYOUT_I2) == 7 * 5 * 130 * 4  # 63 row tiles -> 7 splits
    assert ws(1, 64, 64, bl.LAYOUT_I2) == 0  # 4 row tiles: no split
    assert ws(2048, 3200, 3200, bl.LAYOUT_I2) == 0  # tiled kernel
    assert ws(1, 3200, 3200, bl.LAYOUT_B1) == (bl.bitlinear_packed_bytes(3200, 3200, 0) + 255) // 256 * 256 \
        + 11 * 3200 * 4
    dw = dict(Xq=A, ldq=64, beta=C, M=4, N=64, K=64, dY=B, lddy=64, dW=D, lddw=64, stream=None)
    assert bl.bitlinear_backward_dw(**{**dw, "Xq": None}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dw(**{**dw, "ldq": 63}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dw(**{**dw, "lddw": 10}) == bl.ERR_INVALID_ARG
    assert bl.bitlinear_backward_dw(**{**dw, "dW": B}) == bl.ERR_INVALID_ARG  # overlaps dY
    assert bl.bitlinear_backward_dw(**{**dw, "beta": C + 2}) == bl.ERR_INVALID_ARG


def test_gemm_weight_workspace():
    """No forward rewrites weights: the products decode b3 and b1 themselves,
    so pre-quantised input needs no workspace at any token count and nothing
    in the workspace is sized by N."""
    N, K = 1000, 3000
    ws = bl.bitlinear_forward_workspace_bytes
    for layout in (bl.LAYOUT_I2, bl.LAYOUT_B3, bl.LAYOUT_B1):
        for M in (1, 16, 64, 176, 2048):
            assert ws(M, N, K, layout, bl.I8) == 0
            assert ws(M, N, K, layout, bl.BF16) == ws(M, 1, K, layout, bl.BF16) > 0


def test_transcode_rejects():
    """bitlinear_transcode_i2 argument checks (no launch)."""
    f = bl.bitlinear_transcode_i2
    ok = dict(P=A, layout=bl.LAYOUT_B3, N=64, K=300, P2=B, stream=None)
    assert f(**{**ok, "P": None}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "P2": None}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "layout": bl.LAYOUT_I2}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "layout": 7}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "N": 0}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "K": 0}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "K": bl.MAX_K + 1}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "P2": B + 4}) == bl.ERR_INVALID_ARG  # misaligned
    assert f(**{**ok, "P2": A + 256}) == bl.ERR_INVALID_ARG  # overlaps P
    assert f(**{**ok, "layout": bl.LAYOUT_B1, "P2": A + 16 * 64 * 2}) == bl.ERR_INVALID_ARG


def _jobs(n=3, over=None):
    over = over or {}
    base = []
    for j in range(n):
        d = dict(P=A + 0x1000000 * j, gamma=B + 64 * j, X=C, Y=D + 0x1000000 * j, M=1, N=3200, K=3200, ldx=3200,
                 ldy=3200)
        d.update(over.get(j, {}))
        base.append(d)
    return bl.job_array(base), n


def test_grouped_workspace_bytes():
    # 1-4 tokens of aligned rows: the product launch quantises them itself, no workspace
    arr, n = _jobs(3)
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.BF16) == 0
    # 16 tokens: one tiled input (13 k-steps x 4 operands x 1 KiB) and its beta (256 B) per distinct input
    arr, n = _jobs(3, {0: dict(M=16), 1: dict(M=16), 2: dict(M=16)})
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.BF16) == 13 * 4 * 1024 + 256
    arr, n = _jobs(2, {0: dict(M=16), 1: dict(M=16, X=C + 0x100000)})  # two distinct inputs
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.BF16) == 2 * (13 * 4 * 1024 + 256)
    # unaligned rows (ldx 3201 bf16): quantised by the separate launch
    arr, n = _jobs(1, {0: dict(ldx=3201)})
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.BF16) == 13 * 4 * 1024 + 256
    # a job of 64 tokens runs as its own forward: its workspace is added
    arr, n = _jobs(2, {0: dict(M=16), 1: dict(X=C + 0x100000, M=64)})
    one = bl.bitlinear_forward_workspace_bytes(64, 3200, 3200, bl.LAYOUT_I2, bl.BF16)
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.BF16) == \
        13 * 4 * 1024 + 256 + (one + 255) // 256 * 256
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, n, bl.LAYOUT_I2, bl.I8) == -1
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, 0, bl.LAYOUT_I2, bl.BF16) == -1
    assert bl.bitlinear_forward_grouped_workspace_bytes(arr, bl.MAX_GROUP + 1, bl.LAYOUT_I2, bl.BF16) == -1


def test_grouped_kernel_name():
    arr, n = _jobs(3)  # 1 token, aligned bf16 rows: the quantiser inside, add/sub products
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv_addsub<1>"
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.F32) == "bl::k_group_gemv_addsub<0>"
    arr, n = _jobs(3, {2: dict(K=12288, ldx=12288, X=C + 0x100000)})  # three k-steps per wave
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv_addsub<1>"
    arr, n = _jobs(3, {2: dict(ldx=3201, X=C + 0x100000)})  # unaligned rows: quantiser launch, matrix cores
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv<0, 2>"
    arr, n = _jobs(3, {1: dict(M=2)})  # two tokens: the matrix cores
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv<0, 1>"
    arr, n = _jobs(3)
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_B3, bl.BF16) == "bl::k_group_gemv<1, 1>"
    # one token with a row too long for the grouped launch: left to a plain
    # forward, which does not decide the grouped launch's algorithm
    arr, n = _jobs(3, {1: dict(K=65536, ldx=65536, X=C + 0x100000)})
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv_addsub<1>"
    arr, n = _jobs(2, {1: dict(K=8640, ldx=8640, X=C + 0x100000, M=16)})  # 16 tokens: quantiser launch first
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv<0, 2>"
    arr, n = _jobs(1, {0: dict(M=17)})
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) is None


_M16 = {0: dict(M=16), 1: dict(M=16), 2: dict(M=16)}  # (grouped jobs that need a workspace)


def gfw(arr, n, **kw):
    a = dict(layout=bl.LAYOUT_I2, x_dtype=bl.BF16, y_dtype=bl.F32, ws=E, ws_bytes=1 << 24, stream=None)
    a.update(kw)
    return bl.bitlinear_forward_grouped(arr, n, **a)


@pytest.mark.parametrize("over,kw,status", [
    ({}, dict(layout=7), bl.ERR_INVALID_ARG),
    ({}, dict(x_dtype=bl.I8), bl.ERR_INVALID_ARG),
    ({}, dict(y_dtype=bl.I8), bl.ERR_INVALID_ARG),
    ({1: dict(P=None)}, {}, bl.ERR_INVALID_ARG),
    ({2: dict(M=0)}, {}, bl.ERR_INVALID_ARG),
    ({0: dict(ldx=3199)}, {}, bl.ERR_INVALID_ARG),
    ({0: dict(ldy=3199)}, {}, bl.ERR_INVALID_ARG),
    ({1: dict(P=A + 0x1000008)}, {}, bl.ERR_INVALID_ARG),            # P alignment
    ({1: dict(Y=C)}, {}, bl.ERR_INVALID_ARG),                        # Y overlaps a job's X
    ({1: dict(Y=D)}, {}, bl.ERR_INVALID_ARG),                        # Y overlaps another job's Y
    ({1: dict(Y=A + 0x2000000)}, {}, bl.ERR_INVALID_ARG),            # Y overlaps another job's P
    (_M16, dict(ws=None, ws_bytes=0), bl.ERR_WORKSPACE),
    (_M16, dict(ws_bytes=1000), bl.ERR_WORKSPACE),
    (_M16, dict(ws=E + 8), bl.ERR_INVALID_ARG),
    (_M16, dict(ws=C), bl.ERR_INVALID_ARG),                          # workspace overlaps X
])
def test_grouped_rejects(over, kw, status):
    arr, n = _jobs(3, over)
    assert gfw(arr, n, **kw) == status


def test_grouped_rejects_bad_counts():
    arr, n = _jobs(3)
    assert gfw(arr, 0) == bl.ERR_INVALID_ARG
    assert gfw(arr, bl.MAX_GROUP + 1) == bl.ERR_INVALID_ARG
    assert gfw(None, 1) == bl.ERR_INVALID_ARG


def test_grouped_algo_rejects_and_names():
    """bitlinear_forward_grouped_algo: the vector-ALU products take only i2
    jobs of one token each, all grouped and quantised inside; everything else
    is refused before anything is enqueued (no launch here)."""
    def call(arr, n, algo, **kw):
        a = dict(layout=bl.LAYOUT_I2, x_dtype=bl.BF16, y_dtype=bl.F32, ws=E, ws_bytes=1 << 24, stream=None)
        a.update(kw)
        return bl.bitlinear_forward_grouped_algo(arr, n, a["layout"], a["x_dtype"], a["y_dtype"], algo, a["ws"],
                                                 a["ws_bytes"], a["stream"])
    names = bl.bitlinear_grouped_kernel_algo
    arr, n = _jobs(3)
    assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMV_ADDSUB) == "bl::k_group_gemv_addsub<1>"
    assert names(arr, n, bl.LAYOUT_I2, bl.F32, bl.ALGO_GEMV_ADDSUB) == "bl::k_group_gemv_addsub<0>"
    assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMV_MFMA) == "bl::k_group_gemv<0, 1>"
    assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_AUTO) == bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2,
                                                                                           bl.BF16)
    assert names(arr, n, bl.LAYOUT_B3, bl.BF16, bl.ALGO_GEMV_ADDSUB) is None
    assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMM_MFMA) is None
    assert call(arr, n, bl.ALGO_GEMV_ADDSUB, layout=bl.LAYOUT_B3) == bl.ERR_UNSUPPORTED
    assert call(arr, n, bl.ALGO_GEMV_ADDSUB, layout=bl.LAYOUT_B1) == bl.ERR_UNSUPPORTED
    assert call(arr, n, bl.ALGO_GEMM_MFMA) == bl.ERR_UNSUPPORTED
    assert call(arr, n, 4) == bl.ERR_INVALID_ARG
    assert call(arr, n, -1) == bl.ERR_INVALID_ARG
    assert call(arr, n, bl.ALGO_GEMV_ADDSUB, y_dtype=bl.I8) == bl.ERR_INVALID_ARG  # argument checks first
    for over in ({1: dict(M=2)},                        # two tokens
                 {1: dict(M=20, X=C + 0x100000)},       # a job left to a plain forward
                 {1: dict(ldx=3201, X=C + 0x100000)}):  # rows not 16-byte aligned: quantiser launch
        arr, n = _jobs(3, over)
        assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMV_ADDSUB) is None, over
        assert call(arr, n, bl.ALGO_GEMV_ADDSUB) == bl.ERR_UNSUPPORTED, over
    # one token with a row too long for the grouped launch: that job runs on
    # the single-layer add/sub GEMV, the others in the grouped launch
    arr, n = _jobs(3, {1: dict(K=65536, ldx=65536, X=C + 0x100000)})
    assert names(arr, n, bl.LAYOUT_I2, bl.BF16, bl.ALGO_GEMV_ADDSUB) == "bl::k_group_gemv_addsub<1>"


def test_noalloc_rejects_before_any_device_call():
    # a workspace beyond the allocation-free scratch is refused on the host
    assert bl.bitlinear_forward_workspace_bytes(1024, 16, 131072, bl.LAYOUT_I2, bl.BF16) > bl.NOALLOC_SCRATCH_BYTES
    st = bl.bitlinear_forward_noalloc(A, bl.LAYOUT_I2, B, 1024, 16, 131072, C, bl.BF16, 131072, None, E, bl.F32, 16,
                                      None)
    assert st == bl.ERR_SCRATCH
    assert "scratch" in bl.bitlinear_status_string(bl.ERR_SCRATCH)
    assert bl.bitlinear_forward_noalloc(None, bl.LAYOUT_I2, B, 4, 64, 64, C, bl.BF16, 64, None, D, bl.F32, 64,
                                        None) == bl.ERR_INVALID_ARG


F_ = 0x70000000  # another far-apart fake address


def test_forward_chain_rejects_and_parts():
    """bitlinear_forward_chain argument checks and the parts query (no launch:
    every case fails before anything is enqueued)."""
    f = bl.bitlinear_forward_chain
    M, N, K = 16, 3200, 3200
    nws = bl.bitlinear_forward_workspace_bytes(M, N, K, bl.LAYOUT_I2, bl.F32)
    parts = bl.bitlinear_forward_chain_parts(M, N, K, bl.LAYOUT_I2)
    assert parts == (N + 15) // 16  # the per-tile GEMV: one workgroup per row tile
    assert bl.bitlinear_forward_chain_parts(M, 28672, 8192, bl.LAYOUT_I2) <= 256  # persistent
    assert bl.bitlinear_forward_chain_parts(17, N, K, bl.LAYOUT_I2) == -1
    assert bl.bitlinear_forward_chain_parts(M, N, 70000, bl.LAYOUT_I2) == -1
    ok = dict(P=A, layout=bl.LAYOUT_I2, gamma=B, M=M, N=N, K=K, X=C, x_dtype=bl.F32, ldx=K, pmax_in=F_,
              nparts_in=200, Y=D, y_dtype=bl.F32, ldy=N, pmax_out=F_ + 0x100000, pmax_cols=K, ws=F_ + 0x200000,
              ws_bytes=nws, stream=None)
    assert f(**{**ok, "M": 17}) == bl.ERR_UNSUPPORTED
    assert f(**{**ok, "x_dtype": bl.I8}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "ws_bytes": nws - 1}) == bl.ERR_WORKSPACE
    assert f(**{**ok, "ws": None}) == bl.ERR_WORKSPACE
    assert f(**{**ok, "nparts_in": 0}) == bl.ERR_INVALID_ARG       # pmax_in without parts
    assert f(**{**ok, "pmax_in": None}) == bl.ERR_INVALID_ARG      # parts without pmax_in
    assert f(**{**ok, "pmax_in": F_ + 2}) == bl.ERR_INVALID_ARG     # misaligned
    assert f(**{**ok, "pmax_in": D}) == bl.ERR_INVALID_ARG         # overlaps Y
    assert f(**{**ok, "y_dtype": bl.I32}) == bl.ERR_INVALID_ARG    # maxima of raw accumulators
    assert f(**{**ok, "pmax_cols": 0}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "pmax_cols": N + 1}) == bl.ERR_INVALID_ARG
    assert f(**{**ok, "pmax_out": None}) == bl.ERR_INVALID_ARG     # pmax_cols without pmax_out
    assert f(**{**ok, "pmax_out": D + 64}) == bl.ERR_INVALID_ARG   # overlaps Y
    assert f(**{**ok, "pmax_out": F_ + 16}) == bl.ERR_INVALID_ARG   # overlaps pmax_in
    assert f(**{**ok, "pmax_out": F_ + 0x100002}) == bl.ERR_INVALID_ARG  # misaligned


def test_grouped_leaves_out_jobs_beyond_32_bit_offsets():
    """The grouped launch addresses a job's packed weights with 32-bit byte
    offsets: a job of 2^31 packed bytes or more runs as its own forward (the
    single-layer kernels address whole tiles with 64-bit pointers)."""
    big = dict(N=1 << 27, K=64, ldx=64, ldy=1 << 27)  # 2^27 rows x 16 bytes = 2^31 bytes
    assert bl.bitlinear_packed_bytes(1 << 27, 64, bl.LAYOUT_I2) == 1 << 31
    arr, n = _jobs(1, {0: big})
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) is None
    # rows are packed in whole 16-row tiles: 2^27 - 16 rows are 2^31 - 256 bytes, grouped
    assert bl.bitlinear_packed_bytes((1 << 27) - 1, 64, bl.LAYOUT_I2) == 1 << 31
    arr, n = _jobs(1, {0: dict(big, N=(1 << 27) - 16, ldy=(1 << 27) - 16)})
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_I2, bl.BF16) == "bl::k_group_gemv_addsub<1>"
    # b3: 2^31 / 16 rows of one 80-weight block
    arr, n = _jobs(1, {0: dict(big, K=80, ldx=80)})
    assert bl.bitlinear_grouped_kernel(arr, n, bl.LAYOUT_B3, bl.BF16) is None
