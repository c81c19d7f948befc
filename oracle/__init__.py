"""CPU oracle for the BitLinear forward pass of BitNet b1.58.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite, the
smoke check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may
import this package.  It shares no code with the HIP library and never calls
into it.

The arithmetic lives in ``bitlinear_oracle.c`` (plain loops, IEEE binary32,
no fast-math, int64 accumulation); this module only builds it with gcc and
marshals numpy arrays through ctypes.  Each function names the passage of the
pages it follows:

* "The Era of 1-bit LLMs" abstract: every weight is ternary {-1, 0, +1}.
* LIT-380 record, Key takeaways, bullet 1: BitLinear replaces nn.Linear, an
  absmean function ternarises the weights, activations are 8-bit.
* LIT-380 record, Key takeaways, bullet 4: the product is integer additions.
* HackerPapers digest, threads "GPUs Go Brrr" (2 bits in practice) and "How to
  pack ternary numbers in 8-bit bytes" (several trits per byte); a comment
  there quoting the BitNet paper on the straight-through estimator (backward).

Functions with no independent pin are listed as "parity unpinned" in the
design notes; at present every function here has at least one pin in
``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bitlinear_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

LAYOUT_I2 = 0
LAYOUT_B3 = 1
LAYOUT_B1 = 2

_ERRORS = {
    1: "non-finite input",
    2: "int32 accumulator overflow",
    3: "packed byte holds a code that is never written",
    4: "argument out of range",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE binary32: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        sig = {
            "oracle_absmean": ([P, I, P], ctypes.c_int),
            "oracle_ternarize": ([P, I, ctypes.c_float, P], ctypes.c_int),
            "oracle_binarize": ([P, I, P], ctypes.c_int),
            "oracle_pack_b1": ([P, I, I, P], ctypes.c_int),
            "oracle_unpack_b1": ([P, I, I, P], ctypes.c_int),
            "oracle_packed_bytes": ([I, I, ctypes.c_int], ctypes.c_int64),
            "oracle_pack_i2": ([P, I, I, P], ctypes.c_int),
            "oracle_unpack_i2": ([P, I, I, P], ctypes.c_int),
            "oracle_pack_b3": ([P, I, I, P], ctypes.c_int),
            "oracle_unpack_b3": ([P, I, I, P], ctypes.c_int),
            "oracle_bf16_to_f32": ([P, I, P], None),
            "oracle_quant_act": ([P, I, I, I, P, P], ctypes.c_int),
            "oracle_matmul": ([P, P, I, I, I, P], ctypes.c_int),
            "oracle_rescale": ([P, P, ctypes.c_float, I, I, P], None),
            "oracle_f32_to_bf16": ([P, I, P], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(status: int):
    if status:
        raise OracleError(_ERRORS.get(status, f"status {status}"))


def absmean(w: np.ndarray) -> np.float32:
    """gamma = mean|W| over the whole tensor: the exact mean, rounded once to
    binary32 with ties to even (absmean function, LIT-380 Key takeaways #1)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    g = np.zeros(1, np.float32)
    _check(_load().oracle_absmean(_ptr(w), w.size, _ptr(g)))
    return g[0]


def ternarize(w: np.ndarray, gamma) -> np.ndarray:
    """T = clamp(rint(w / gamma), -1, 1) with IEEE division and ties to even
    (ternary weights: Abstract; absmean mapping: LIT-380 Key takeaways #1)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    t = np.empty(w.shape, np.int8)
    _check(_load().oracle_ternarize(_ptr(w), w.size, ctypes.c_float(float(gamma)), _ptr(t)))
    return t


def quantize_weights(w: np.ndarray):
    """(T, gamma) for a latent fp32 weight matrix W[N x K]."""
    g = absmean(w)
    return ternarize(w, g), g


def binarize(w: np.ndarray) -> np.ndarray:
    """T = +1 where w >= 0 (including -0), -1 where w < 0: the binary weights of
    the predecessor variant (HackerPapers digest: the original BitNet used -1
    or +1; LIT-380 Key takeaways #2: two states against three)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    t = np.empty(w.shape, np.int8)
    _check(_load().oracle_binarize(_ptr(w), w.size, _ptr(t)))
    return t


def quantize_weights_binary(w: np.ndarray):
    """(T, gamma) of the binary variant: sign weights, the same absmean scale."""
    return binarize(w), absmean(w)


_PACK = {LAYOUT_I2: ("oracle_pack_i2", "oracle_unpack_i2"), LAYOUT_B3: ("oracle_pack_b3", "oracle_unpack_b3"),
         LAYOUT_B1: ("oracle_pack_b1", "oracle_unpack_b1")}


def packed_bytes(N: int, K: int, layout: int) -> int:
    return int(_load().oracle_packed_bytes(N, K, layout))


def pack(t: np.ndarray, layout: int) -> np.ndarray:
    """Pack T[N x K] into the i2 (2 bits/weight, "GPUs Go Brrr" thread), b3
    (5 trits per byte, "How to pack ternary numbers in 8-bit bytes" thread) or,
    for binary weights, b1 (1 bit per weight) layout."""
    t = np.ascontiguousarray(t, dtype=np.int8)
    N, K = t.shape
    p = np.zeros(packed_bytes(N, K, layout), np.uint8)
    fn = getattr(_load(), _PACK[layout][0])
    _check(fn(_ptr(t), N, K, _ptr(p)))
    return p


def unpack(p: np.ndarray, N: int, K: int, layout: int) -> np.ndarray:
    p = np.ascontiguousarray(p, dtype=np.uint8)
    if p.size < packed_bytes(N, K, layout):
        raise OracleError("packed buffer too small")
    t = np.empty((N, K), np.int8)
    fn = getattr(_load(), _PACK[layout][1])
    _check(fn(_ptr(p), N, K, _ptr(t)))
    return t


def bf16_to_f32(x_bits: np.ndarray) -> np.ndarray:
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    out = np.empty(x_bits.shape, np.float32)
    _load().oracle_bf16_to_f32(_ptr(x_bits), x_bits.size, _ptr(out))
    return out


def quantize_act(x: np.ndarray):
    """Per-token absmax int8 quantisation (8-bit activations, LIT-380 Key
    takeaways #1).  x: fp32 [M x K], or uint16 bfloat16 bit patterns.
    Returns (q int8 [M x K], beta fp32 [M])."""
    if x.dtype == np.uint16:
        x = bf16_to_f32(x)
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    beta = np.empty(M, np.float32)
    _check(_load().oracle_quant_act(_ptr(x), M, K, K, _ptr(q), _ptr(beta)))
    return q, beta


def matmul(q: np.ndarray, t: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * T[n, k], exact (LIT-380 Key takeaways #4)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    t = np.ascontiguousarray(t, dtype=np.int8)
    M, K = q.shape
    N, K2 = t.shape
    if K != K2:
        raise OracleError("inner dimensions differ")
    acc = np.empty((M, N), np.int32)
    _check(_load().oracle_matmul(_ptr(q), _ptr(t), M, N, K, _ptr(acc)))
    return acc


def rescale(acc: np.ndarray, beta: np.ndarray, gamma) -> np.ndarray:
    """y = float(acc) * ((gamma * beta_m) / 127) in binary32."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _load().oracle_rescale(_ptr(acc), _ptr(beta), ctypes.c_float(float(gamma)), M, N, _ptr(y))
    return y


def f32_to_bf16(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_f32_to_bf16(_ptr(y), y.size, _ptr(out))
    return out


def forward(t: np.ndarray, gamma, x: np.ndarray):
    """The whole BitLinear forward on already-ternarised weights.
    Returns dict(q, beta, acc, y)."""
    q, beta = quantize_act(x)
    acc = matmul(q, t)
    y = rescale(acc, beta, gamma)
    return {"q": q, "beta": beta, "acc": acc, "y": y}


# ---------------------------------------------------------------------------
# Backward pass with the straight-through estimator.  The pages quote the
# BitNet paper: training uses the straight-through estimator, which bypasses
# the non-differentiable functions (Sign and Clip there; here also the
# rounding of the absmean and absmax quantisers) when gradients are
# propagated (HackerPapers digest, comment quoting the BitNet paper on the
# straight-through estimator).  Reading: each quantiser's derivative is taken
# as 1 and its scale (gamma, beta_m) as a constant, so the forward acts like
# the linear map y = Xhat @ What^T of the dequantised operands
#     What[n, k] = gamma * T[n, k],    Xhat[m, k] = q[m, k] * r_m,
# r_m = fl32(beta_m / 127), Xhat rounded to binary32 (the same rounding
# order as the forward's rescale is not needed: Xhat only feeds a gradient).
# Its gradients are the plain matrix products below, summed in binary64.
# ---------------------------------------------------------------------------
def dequantize_act(q: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """Xhat[m, k] = fl32(q[m, k] * fl32(beta_m / 127))."""
    r = (np.asarray(beta, np.float32) / np.float32(127.0)).astype(np.float32)
    return (np.asarray(q, np.float32) * r[:, None]).astype(np.float32)


def backward_dx(t: np.ndarray, gamma, dy: np.ndarray) -> np.ndarray:
    """Gradient with respect to the layer input: dX = dY @ What = gamma *
    (dY @ T), float64 [M x K].  t: int8 [N x K]; dy: fp32 [M x N]."""
    dy = np.asarray(dy, np.float64)
    return float(np.float32(gamma)) * (dy @ np.asarray(t, np.float64))


def backward_dw(q: np.ndarray, beta: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """Gradient with respect to the latent weights W (through the ternariser
    by the straight-through estimator): dW = dY^T @ Xhat, float64 [N x K]."""
    xhat = dequantize_act(q, beta).astype(np.float64)
    return np.asarray(dy, np.float64).T @ xhat


def threads_used() -> int:
    """OpenMP threads the matmul runs on (OMP_NUM_THREADS, else all visible cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))
