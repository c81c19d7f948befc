"""ctypes binding of libbitlinear (include/bitlinear.h).

Argument marshalling only: every step of the BitLinear forward runs in the HIP
kernels of libbitlinear.so.  The ``bitlinear_*`` functions mirror the C entry
points one to one (device pointers as Python ints, the HIP stream as an int);
the lower-case helpers below them take torch tensors, allocate outputs with
torch (device memory and streams are all torch is used for) and call those.

Importing this module raises if the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m ternary_weight_linear_forward_amd.build`")

# torch wheels bundle their own HIP runtime.  Load it first so that the
# library's libamdhip64.so.7 dependency binds to that same runtime: two HIP
# runtimes in one process would not share devices, streams or allocations.
try:
    import torch  # noqa: F401
except ImportError:
    pass

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes_loaded() -> list:
    try:
        with open(f"/proc/{os.getpid()}/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in paths})


if len(_hip_runtimes_loaded()) > 1:
    raise ImportError("two HIP runtimes are loaded in this process "
                      f"({', '.join(_hip_runtimes_loaded())}); import torch before loading libbitlinear")

# --- enums (bitlinear.h) ---------------------------------------------------
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH, ERR_DEVICE, ERR_SCRATCH = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20
F32, BF16, I8, I32, I8_TILED = range(5)
LAYOUT_I2, LAYOUT_B3, LAYOUT_B1 = 0, 1, 2
ALGO_AUTO, ALGO_GEMV_ADDSUB, ALGO_GEMV_MFMA, ALGO_GEMM_MFMA = range(4)
MAX_K = 131072
MAX_M = 65536

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int

class Job(ctypes.Structure):
    """bitlinear_job_t: one BitLinear of a grouped forward (device pointers)."""
    _fields_ = [("P", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("X", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("ldy", ctypes.c_int64)]


MAX_GROUP = 32
_JOBS = ctypes.POINTER(Job)

_SIGNATURES = {
    "bitlinear_status_string": ([_INT], ctypes.c_char_p),
    "bitlinear_version": ([], _INT),
    "bitlinear_packed_bytes": ([_I64, _I64, _INT], _I64),
    "bitlinear_quantize_weights_workspace_bytes": ([_I64, _I64], _I64),
    "bitlinear_forward_workspace_bytes": ([_I64, _I64, _I64, _INT, _INT], _I64),
    "bitlinear_act_tiled_bytes": ([_I64, _I64, _INT], _I64),
    "bitlinear_auto_algo": ([_I64, _I64, _I64, _INT, _INT], _INT),
    "bitlinear_product_kernel": ([_I64, _I64, _I64, _INT, _INT, _INT], ctypes.c_char_p),
    "bitlinear_quantize_act_tiled": ([_P, _INT, _I64, _I64, _I64, _INT, _P, _I64, _P, _P], _INT),
    "bitlinear_quantize_weights": ([_P, _I64, _I64, _I64, _P, _P, _P, _I64, _P], _INT),
    "bitlinear_binarize_weights": ([_P, _I64, _I64, _I64, _P, _P, _P, _I64, _P], _INT),
    "bitlinear_pack": ([_P, _I64, _I64, _I64, _INT, _P, _P], _INT),
    "bitlinear_forward_chain": ([_P, _INT, _P, _I64, _I64, _I64, _P, _INT, _I64, _P, _I64, _P, _INT, _I64, _P, _I64,
                                 _P, _I64, _P], _INT),
    "bitlinear_forward_chain_parts": ([_I64, _I64, _I64, _INT], _I64),
    "bitlinear_transcode_i2": ([_P, _INT, _I64, _I64, _P, _P], _INT),
    "bitlinear_quantize_act": ([_P, _INT, _I64, _I64, _I64, _P, _I64, _P, _P], _INT),
    "bitlinear_forward": ([_P, _INT, _P, _I64, _I64, _I64, _P, _INT, _I64, _P, _P, _INT, _I64, _P, _I64, _P], _INT),
    "bitlinear_backward_dx_workspace_bytes": ([_I64, _I64, _I64, _INT], _I64),
    "bitlinear_backward_kernel": ([_I64, _I64, _I64, _INT], ctypes.c_char_p),
    "bitlinear_backward_dx": ([_P, _INT, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _I64, _P], _INT),
    "bitlinear_backward_dw": ([_P, _I64, _P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P], _INT),
    "bitlinear_forward_algo": (
        [_P, _INT, _P, _I64, _I64, _I64, _P, _INT, _I64, _P, _P, _INT, _I64, _P, _I64, _INT, _P], _INT),
    "bitlinear_forward_noalloc": ([_P, _INT, _P, _I64, _I64, _I64, _P, _INT, _I64, _P, _P, _INT, _I64, _P], _INT),
    "bitlinear_forward_grouped_workspace_bytes": ([_JOBS, _INT, _INT, _INT], _I64),
    "bitlinear_forward_grouped": ([_JOBS, _INT, _INT, _INT, _INT, _P, _I64, _P], _INT),
    "bitlinear_grouped_kernel": ([_JOBS, _INT, _INT, _INT], ctypes.c_char_p),
    "bitlinear_forward_grouped_algo": ([_JOBS, _INT, _INT, _INT, _INT, _INT, _P, _I64, _P], _INT),
    "bitlinear_grouped_kernel_algo": ([_JOBS, _INT, _INT, _INT, _INT], ctypes.c_char_p),
    "bitlinear_forward_ex": (
        [_P, _INT, _P, _I64, _I64, _I64, _P, _INT, _I64, _P, _P, _INT, _I64, _P, _I64, _P, _P, _I64, _INT, _P],
        _INT),
}
EXPORTED = tuple(_SIGNATURES)

for _name, (_args, _res) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class BitlinearError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bitlinear_status_string(status)} (status {status})")


def _check(status: int, where: str) -> None:
    if status != OK:
        raise BitlinearError(status, where)


# --- raw C entry points (same names) ----------------------------------------
def bitlinear_status_string(status: int) -> str:
    return _lib.bitlinear_status_string(status).decode()


def bitlinear_version() -> int:
    return _lib.bitlinear_version()


def bitlinear_packed_bytes(N: int, K: int, layout: int) -> int:
    return _lib.bitlinear_packed_bytes(N, K, layout)


def bitlinear_quantize_weights_workspace_bytes(N: int, K: int) -> int:
    return _lib.bitlinear_quantize_weights_workspace_bytes(N, K)


def bitlinear_forward_workspace_bytes(M: int, N: int, K: int, layout: int, x_dtype: int) -> int:
    return _lib.bitlinear_forward_workspace_bytes(M, N, K, layout, x_dtype)


def bitlinear_act_tiled_bytes(M: int, K: int, layout: int) -> int:
    return _lib.bitlinear_act_tiled_bytes(M, K, layout)


def bitlinear_auto_algo(M: int, N: int, K: int, layout: int, x_dtype: int) -> int:
    return _lib.bitlinear_auto_algo(M, N, K, layout, x_dtype)


def bitlinear_product_kernel(M: int, N: int, K: int, layout: int, x_dtype: int, algo: int = 0):
    r = _lib.bitlinear_product_kernel(M, N, K, layout, x_dtype, algo)
    return None if r is None else r.decode()


def bitlinear_backward_kernel(M: int, N: int, K: int, which: int):
    r = _lib.bitlinear_backward_kernel(M, N, K, which)
    return None if r is None else r.decode()


def bitlinear_quantize_act_tiled(X, x_dtype, M, K, ldx, layout, Xt, xt_bytes, beta, stream) -> int:
    return _lib.bitlinear_quantize_act_tiled(X, x_dtype, M, K, ldx, layout, Xt, xt_bytes, beta, stream)


def bitlinear_quantize_weights(W, N, K, ldw, T, gamma, ws, ws_bytes, stream) -> int:
    return _lib.bitlinear_quantize_weights(W, N, K, ldw, T, gamma, ws, ws_bytes, stream)


def bitlinear_binarize_weights(W, N, K, ldw, T, gamma, ws, ws_bytes, stream) -> int:
    return _lib.bitlinear_binarize_weights(W, N, K, ldw, T, gamma, ws, ws_bytes, stream)


def bitlinear_backward_dx_workspace_bytes(M: int, N: int, K: int, layout: int) -> int:
    return _lib.bitlinear_backward_dx_workspace_bytes(M, N, K, layout)


def bitlinear_backward_dx(P, layout, gamma, M, N, K, dY, lddy, dX, lddx, ws, ws_bytes, stream) -> int:
    return _lib.bitlinear_backward_dx(P, layout, gamma, M, N, K, dY, lddy, dX, lddx, ws, ws_bytes, stream)


def bitlinear_backward_dw(Xq, ldq, beta, M, N, K, dY, lddy, dW, lddw, stream) -> int:
    return _lib.bitlinear_backward_dw(Xq, ldq, beta, M, N, K, dY, lddy, dW, lddw, stream)


def bitlinear_pack(T, N, K, ldt, layout, P, stream) -> int:
    return _lib.bitlinear_pack(T, N, K, ldt, layout, P, stream)


def bitlinear_forward_chain(P, layout, gamma, M, N, K, X, x_dtype, ldx, pmax_in, nparts_in, Y, y_dtype, ldy, pmax_out,
                            pmax_cols, ws, ws_bytes, stream) -> int:
    return _lib.bitlinear_forward_chain(P, layout, gamma, M, N, K, X, x_dtype, ldx, pmax_in, nparts_in, Y, y_dtype,
                                        ldy, pmax_out, pmax_cols, ws, ws_bytes, stream)


def bitlinear_forward_chain_parts(M, N, K, layout) -> int:
    return _lib.bitlinear_forward_chain_parts(M, N, K, layout)


def bitlinear_transcode_i2(P, layout, N, K, P2, stream) -> int:
    return _lib.bitlinear_transcode_i2(P, layout, N, K, P2, stream)


def bitlinear_quantize_act(X, x_dtype, M, K, ldx, Xq, ldq, beta, stream) -> int:
    return _lib.bitlinear_quantize_act(X, x_dtype, M, K, ldx, Xq, ldq, beta, stream)


def bitlinear_forward(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws, ws_bytes,
                      stream) -> int:
    return _lib.bitlinear_forward(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws,
                                  ws_bytes, stream)


def bitlinear_forward_algo(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws, ws_bytes,
                           algo, stream) -> int:
    return _lib.bitlinear_forward_algo(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, ws,
                                       ws_bytes, algo, stream)


def bitlinear_forward_ex(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, Xq_out, ldxq,
                         beta_out, ws, ws_bytes, algo, stream) -> int:
    return _lib.bitlinear_forward_ex(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, Xq_out,
                                     ldxq, beta_out, ws, ws_bytes, algo, stream)


def job_array(jobs) -> ctypes.Array:
    """A ctypes array of Job from a sequence of Job (or of field dicts)."""
    arr = (Job * max(len(jobs), 1))()
    for i, j in enumerate(jobs):
        arr[i] = j if isinstance(j, Job) else Job(**j)
    return arr


def bitlinear_forward_noalloc(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy, stream) -> int:
    return _lib.bitlinear_forward_noalloc(P, layout, gamma, M, N, K, X, x_dtype, ldx, beta_in, Y, y_dtype, ldy,
                                          stream)


def bitlinear_forward_grouped_workspace_bytes(jobs, njobs: int, layout: int, x_dtype: int) -> int:
    return _lib.bitlinear_forward_grouped_workspace_bytes(jobs, njobs, layout, x_dtype)


def bitlinear_forward_grouped(jobs, njobs: int, layout: int, x_dtype: int, y_dtype: int, ws, ws_bytes: int,
                              stream) -> int:
    return _lib.bitlinear_forward_grouped(jobs, njobs, layout, x_dtype, y_dtype, ws, ws_bytes, stream)


def bitlinear_grouped_kernel(jobs, njobs: int, layout: int, x_dtype: int):
    r = _lib.bitlinear_grouped_kernel(jobs, njobs, layout, x_dtype)
    return None if r is None else r.decode()


def bitlinear_forward_grouped_algo(jobs, njobs: int, layout: int, x_dtype: int, y_dtype: int, algo: int, ws,
                                   ws_bytes: int, stream) -> int:
    return _lib.bitlinear_forward_grouped_algo(jobs, njobs, layout, x_dtype, y_dtype, algo, ws, ws_bytes, stream)


def bitlinear_grouped_kernel_algo(jobs, njobs: int, layout: int, x_dtype: int, algo: int):
    r = _lib.bitlinear_grouped_kernel_algo(jobs, njobs, layout, x_dtype, algo)
    return None if r is None else r.decode()


# --- torch-tensor helpers (allocation + marshalling) ------------------------
def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    return {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8, torch.int32: I32}[t.dtype]


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _weight_quant(entry, W, stream):
    torch = _torch()
    N, K = W.shape
    T = torch.empty((N, K), dtype=torch.int8, device=W.device)
    gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    nws = bitlinear_quantize_weights_workspace_bytes(N, K)
    if nws < 0:
        raise BitlinearError(ERR_INVALID_ARG, entry.__name__)
    ws = torch.empty(nws, dtype=torch.uint8, device=W.device)
    _check(entry(_ptr(W), N, K, W.stride(0), _ptr(T), _ptr(gamma), _ptr(ws), nws, _stream(stream)), entry.__name__)
    return T, gamma


def quantize_weights(W, stream=None):
    """Latent fp32 W [N x K] (cuda) -> ternary (T int8 [N x K], gamma fp32 [1])."""
    return _weight_quant(bitlinear_quantize_weights, W, stream)


def binarize_weights(W, stream=None):
    """Latent fp32 W [N x K] (cuda) -> binary (T int8 [N x K] in {-1, +1}, gamma fp32 [1])."""
    return _weight_quant(bitlinear_binarize_weights, W, stream)


def pack(T, layout: int = LAYOUT_I2, stream=None):
    """Ternary int8 T [N x K] (cuda) -> packed uint8 P."""
    torch = _torch()
    N, K = T.shape
    nbytes = bitlinear_packed_bytes(N, K, layout)
    if nbytes < 0:
        raise BitlinearError(ERR_INVALID_ARG, "pack")
    P = torch.empty(nbytes, dtype=torch.uint8, device=T.device)
    _check(bitlinear_pack(_ptr(T), N, K, T.stride(0), layout, _ptr(P), _stream(stream)), "bitlinear_pack")
    return P


def forward_chain(P, layout: int, gamma, X, N: int, K: int | None = None, pmax_in=None, pmax_cols: int = 0,
                  y_dtype=None, out=None, stream=None):
    """One link of a chain (bitlinear_forward_chain): X [M <= 16 x >=K] fp32/bf16; pmax_in the previous link's
    partial maxima (or None); with pmax_cols > 0 also returns this link's partial maxima over Y[:, :pmax_cols].
    Returns (Y, pmax_out or None)."""
    torch = _torch()
    M = X.shape[0]
    K = X.shape[1] if K is None else K
    if out is None:
        out = torch.empty((M, N), dtype=y_dtype or torch.float32, device=X.device)
    xdt = _dtype_code(X)
    nws = bitlinear_forward_workspace_bytes(M, N, K, layout, xdt)
    parts = bitlinear_forward_chain_parts(M, N, K, layout)
    if nws < 0 or parts < 0:
        raise BitlinearError(ERR_INVALID_ARG, "forward_chain")
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=X.device)
    pmax_out = torch.empty(parts * 16, dtype=torch.float32, device=X.device) if pmax_cols > 0 else None
    nparts_in = pmax_in.numel() // 16 if pmax_in is not None else 0
    _check(bitlinear_forward_chain(_ptr(P), layout, _ptr(gamma), M, N, K, _ptr(X), xdt, X.stride(0), _ptr(pmax_in),
                                   nparts_in, _ptr(out), _dtype_code(out), out.stride(0), _ptr(pmax_out), pmax_cols,
                                   _ptr(ws), nws, _stream(stream)), "bitlinear_forward_chain")
    return out, pmax_out


def transcode_i2(P, layout: int, N: int, K: int, stream=None):
    """Packed b3 / b1 weights P (cuda) -> the same weights packed as i2 (a load-time step)."""
    torch = _torch()
    nbytes = bitlinear_packed_bytes(N, K, LAYOUT_I2)
    if nbytes < 0:
        raise BitlinearError(ERR_INVALID_ARG, "transcode_i2")
    P2 = torch.empty(nbytes, dtype=torch.uint8, device=P.device)
    _check(bitlinear_transcode_i2(_ptr(P), layout, N, K, _ptr(P2), _stream(stream)), "bitlinear_transcode_i2")
    return P2


def quantize_act(X, stream=None):
    """Activations X [M x K] fp32/bf16 (cuda) -> (Xq int8 [M x ldq], beta fp32 [M]); ldq = K rounded up to 16."""
    torch = _torch()
    M, K = X.shape
    ldq = (K + 15) // 16 * 16
    Xq = torch.empty((M, ldq), dtype=torch.int8, device=X.device)
    beta = torch.empty(M, dtype=torch.float32, device=X.device)
    _check(bitlinear_quantize_act(_ptr(X), _dtype_code(X), M, K, X.stride(0), _ptr(Xq), ldq, _ptr(beta),
                                  _stream(stream)), "bitlinear_quantize_act")
    return Xq, beta


def quantize_act_tiled(X, layout: int = LAYOUT_I2, stream=None):
    """Activations X [M x K] fp32/bf16 (cuda) -> (Xt int8 in the tiled activation layout, beta fp32 [M])."""
    torch = _torch()
    M, K = X.shape
    nbytes = bitlinear_act_tiled_bytes(M, K, layout)
    if nbytes < 0:
        raise BitlinearError(ERR_INVALID_ARG, "quantize_act_tiled")
    Xt = torch.empty(nbytes, dtype=torch.int8, device=X.device)
    beta = torch.empty(M, dtype=torch.float32, device=X.device)
    _check(bitlinear_quantize_act_tiled(_ptr(X), _dtype_code(X), M, K, X.stride(0), layout, _ptr(Xt), nbytes,
                                        _ptr(beta), _stream(stream)), "bitlinear_quantize_act_tiled")
    return Xt, beta


def forward(P, layout: int, gamma, X, N: int, K: int | None = None, beta=None, y_dtype=None, algo: int = ALGO_AUTO,
            ws=None, out=None, stream=None):
    """BitLinear forward.  X [M x >=K] fp32/bf16 (quantised inside the call) or
    int8 (then 'beta' is required).  Returns Y [M x N] (fp32 by default; bf16,
    or int32 raw accumulators with y_dtype=torch.int32)."""
    torch = _torch()
    tiled = X.dim() == 1 and X.dtype == torch.int8
    if tiled:
        if K is None or beta is None:
            raise ValueError("tiled activations need K and beta")
        M = beta.numel()
        xdt = I8_TILED
        ldx = 0
    else:
        M = X.shape[0]
        K = X.shape[1] if K is None else K
        xdt = _dtype_code(X)
        ldx = X.stride(0)
    if out is None:
        out = torch.empty((M, N), dtype=y_dtype or torch.float32, device=X.device)
    nws = bitlinear_forward_workspace_bytes(M, N, K, layout, xdt)
    if nws < 0:
        raise BitlinearError(ERR_INVALID_ARG, "forward")
    if nws > 0 and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=X.device)
    _check(bitlinear_forward_algo(_ptr(P), layout, _ptr(gamma), M, N, K, _ptr(X), xdt, ldx, _ptr(beta),
                                  _ptr(out), _dtype_code(out), out.stride(0), _ptr(ws) if nws > 0 else None,
                                  nws, algo, _stream(stream)), "bitlinear_forward")
    return out


def forward_with_quant(P, layout: int, gamma, X, N: int, K: int | None = None, y_dtype=None,
                       algo: int = ALGO_AUTO, stream=None):
    """BitLinear forward on fp32/bf16 X [M x >=K] that also returns the
    quantiser's outputs: (Y [M x N], Xq int8 [M x ldq], beta fp32 [M]) with
    ldq = K rounded up to 16 (bitlinear_forward_ex)."""
    torch = _torch()
    M = X.shape[0]
    K = X.shape[1] if K is None else K
    ldq = (K + 15) // 16 * 16
    out = torch.empty((M, N), dtype=y_dtype or torch.float32, device=X.device)
    Xq = torch.empty((M, ldq), dtype=torch.int8, device=X.device)
    beta = torch.empty(M, dtype=torch.float32, device=X.device)
    nws = bitlinear_forward_workspace_bytes(M, N, K, layout, I8)
    if nws < 0:
        raise BitlinearError(ERR_INVALID_ARG, "forward_with_quant")
    ws = torch.empty(nws, dtype=torch.uint8, device=X.device) if nws > 0 else None
    _check(bitlinear_forward_ex(_ptr(P), layout, _ptr(gamma), M, N, K, _ptr(X), _dtype_code(X), X.stride(0), None,
                                _ptr(out), _dtype_code(out), out.stride(0), _ptr(Xq), ldq, _ptr(beta), _ptr(ws), nws,
                                algo, _stream(stream)), "bitlinear_forward_ex")
    return out, Xq, beta


def grouped_jobs(specs, y_dtype=None, outs=None):
    """Job array and outputs for forward_grouped.  specs: sequence of (P, gamma,
    X, N) or (P, gamma, X, N, K) with X [M x >=K] fp32/bf16 (cuda)."""
    torch = _torch()
    jobs, ys = [], []
    for idx, sp in enumerate(specs):
        P, gamma, X, N = sp[:4]
        K = sp[4] if len(sp) > 4 else X.shape[1]
        M = X.shape[0]
        Y = outs[idx] if outs is not None else torch.empty((M, N), dtype=y_dtype or torch.float32, device=X.device)
        ys.append(Y)
        jobs.append(Job(P=_ptr(P), gamma=_ptr(gamma), X=_ptr(X), Y=_ptr(Y), M=M, N=N, K=K, ldx=X.stride(0),
                        ldy=Y.stride(0)))
    return job_array(jobs), ys


def forward_grouped(specs, layout: int = LAYOUT_I2, y_dtype=None, ws=None, outs=None, stream=None,
                    algo: int = ALGO_AUTO):
    """Several BitLinear forwards in one grouped call
    (bitlinear_forward_grouped_algo).  specs as grouped_jobs; every X must have
    the same dtype.  Returns the list of outputs Y [M x N]."""
    torch = _torch()
    if not specs:
        return []
    xdt = _dtype_code(specs[0][2])
    arr, ys = grouped_jobs(specs, y_dtype, outs)
    n = len(specs)
    nws = bitlinear_forward_grouped_workspace_bytes(arr, n, layout, xdt)
    if nws < 0:
        raise BitlinearError(ERR_INVALID_ARG, "forward_grouped")
    if nws > 0 and (ws is None or ws.numel() < nws):
        ws = torch.empty(nws, dtype=torch.uint8, device=specs[0][2].device)
    _check(bitlinear_forward_grouped_algo(arr, n, layout, xdt, _dtype_code(ys[0]), algo,
                                          _ptr(ws) if nws > 0 else None, nws, _stream(stream)),
           "bitlinear_forward_grouped_algo")
    return ys


def backward_dx(P, layout: int, gamma, dY, K: int, out=None, stream=None):
    """Straight-through-estimator input gradient dX = gamma * dY @ T.
    dY fp32 [M x N] (cuda); returns dX fp32 [M x K]."""
    torch = _torch()
    M, N = dY.shape
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=dY.device)
    nws = bitlinear_backward_dx_workspace_bytes(M, N, K, layout)
    if nws < 0:
        raise BitlinearError(ERR_INVALID_ARG, "backward_dx")
    ws = torch.empty(nws, dtype=torch.uint8, device=dY.device) if nws > 0 else None
    _check(bitlinear_backward_dx(_ptr(P), layout, _ptr(gamma), M, N, K, _ptr(dY), dY.stride(0), _ptr(out),
                                 out.stride(0), _ptr(ws), nws, _stream(stream)), "bitlinear_backward_dx")
    return out


def backward_dw(Xq, beta, dY, K: int, out=None, stream=None):
    """Straight-through-estimator latent-weight gradient dW = dY^T @ Xhat,
    from the forward's int8 activations Xq [M x >=K] and beta [M].
    Returns dW fp32 [N x K]."""
    torch = _torch()
    M, N = dY.shape
    if out is None:
        out = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    _check(bitlinear_backward_dw(_ptr(Xq), Xq.stride(0), _ptr(beta), M, N, K, _ptr(dY), dY.stride(0), _ptr(out),
                                 out.stride(0), _stream(stream)), "bitlinear_backward_dw")
    return out
