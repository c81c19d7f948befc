"""The kernels' evaluation of the per-token quantiser, emulated on the host in
numpy binary32, against the oracle (no GPU).

The kernels compute pre = 2^64 if beta < 2^-96 else 1, s = RN32(127 /
(beta * pre)) and q = rint(RN32(RN32(x * pre) * s)); the GEMVs that quantise
1 to 4 tokens round by adding 1.5 * 2^23 and keeping the low byte of the sum.
The oracle takes the row to the scale where beta lies in [1, 2) instead.  The
two must agree on every row, from subnormal rows to rows near the largest
binary32 (8-bit absmax activations: LIT-380 record, Key takeaways, bullet 1)."""
import numpy as np

import oracle
from ternary_weight_linear_forward_amd import synth

F = np.float32


def kernel_quant(x):
    x = np.asarray(x, F)
    beta = np.abs(x).max(axis=1)
    pre = np.where(beta < F(2.0 ** -96), F(2.0 ** 64), F(1.0)).astype(F)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(beta > 0, F(127) / (beta * pre), F(0)).astype(F)
    v = ((x * pre[:, None]).astype(F) * s[:, None]).astype(F)
    q_rint = np.clip(np.rint(v), -127, 127).astype(np.int8)
    # magic-add rounding: the low byte of fl32(v + 1.5 * 2^23)
    m = (v + F(12582912.0)).astype(F).view(np.uint32)
    q_magic = (m & 0xFF).astype(np.uint8).view(np.int8)
    assert np.all(np.abs(v) < 127.5)
    return q_rint, q_magic, beta


def test_kernel_formula_matches_oracle_over_the_exponent_range():
    r = synth.rng(90)
    base = r.standard_normal((6, 200)).astype(np.float64)
    base[0, 3] = 0.0
    base[1] = np.round(base[1] * 8) / 8  # many ties after scaling
    for k in list(range(-149, 120, 3)) + [-127, -126, -97, -96, -95]:
        x = np.ldexp(base, k).astype(F)
        x = x[np.abs(x).max(axis=1) < np.finfo(F).max / 2]
        q_ref, b_ref = oracle.quantize_act(x)
        q_rint, q_magic, beta = kernel_quant(x)
        assert np.array_equal(beta, b_ref), k
        assert np.array_equal(q_rint, q_ref), k
        assert np.array_equal(q_magic, q_ref), k


def test_unscaled_step_would_overflow_below_the_threshold():
    # the former evaluation s = RN32(127 / beta) gives +inf at tiny beta and
    # would round every nonzero to +-127: the pre-scale is what avoids it
    x = np.array([[1e-38, 3e-39, -5e-39, 0.0]], F)
    with np.errstate(over="ignore", divide="ignore"):
        assert np.isinf(F(127) / np.abs(x).max())
    q_rint, q_magic, _ = kernel_quant(x)
    assert q_rint[0].tolist() == [127, 38, -64, 0] == q_magic[0].tolist()
    assert np.array_equal(q_rint, oracle.quantize_act(x)[0])
