"""Helpers for the GPU tests: numpy <-> torch transfers and the oracle-side
expected values.  Inputs come from ternary_weight_linear_forward_amd.synth and
go unchanged to both sides."""
import numpy as np
import torch

DEV = torch.device("cuda")


def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:  # bfloat16 bit patterns
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f32_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_f32_parity(got: np.ndarray, want: np.ndarray, rtol: float = 1e-5):
    """The fp32 tolerance of the rescaled output (1e-5 relative), and, because
    both sides apply the same binary32 operations in the same order, bit
    equality."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = rtol * np.abs(want.astype(np.float64)) + 1e-30
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} elements beyond rtol {rtol}; first at {np.argwhere(bad)[0]}"
    assert np.array_equal(f32_bits(got), f32_bits(want)), "within tolerance but not bit-identical"


def assert_bf16_parity(got_bits: np.ndarray, want_f32: np.ndarray, want_bits: np.ndarray, rtol: float = 2e-2):
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = want_f32.astype(np.float64)
    assert np.all(np.abs(got - want) <= rtol * np.abs(want) + 1e-30)
    assert np.array_equal(got_bits, want_bits)
