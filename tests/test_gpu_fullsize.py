"""GPU parity at the full layer sizes of the pages' 3B and 70B models, with the
kernels the benchmark times (automatic dispatch).  Everything is compared in
full: gamma, T and the packed bytes of every layer, and the int32
accumulators and fp32 outputs of every forward, element by element, against
the oracle's (its integer product runs on every host core)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth, workloads  # noqa: E402

from gpu_helpers import assert_f32_parity, f32_bits, to_dev, to_host  # noqa: F401  # noqa: E402

pytestmark = pytest.mark.gpu
LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3}
_cache = {}


def log(*a):
    print(*a, flush=True)


def prepared(wl, li):
    """Quantise and pack one layer on the GPU and check it in full against the oracle."""
    key = (wl.name, li)
    if key in _cache:
        return _cache[key]
    _cache.clear()
    layer = wl.layers[li]
    log("prepare", wl.name, layer)
    w = synth.latent_weights(layer.N, layer.K, seed=workloads.seed_for(wl, li, 0))
    wd = to_dev(w)
    T, gamma = bl.quantize_weights(wd)
    t_ref, g_ref = oracle.quantize_weights(w)
    assert to_host(gamma).view(np.uint32)[0] == np.array(g_ref, np.float32).view(np.uint32)
    assert np.array_equal(to_host(T), t_ref)
    packed = {}
    for name in wl.layouts:
        P = bl.pack(T, LAYOUTS[name])
        assert np.array_equal(to_host(P), oracle.pack(t_ref, LAYOUTS[name])), name
        packed[name] = P
    del wd, T
    _cache[key] = (t_ref, g_ref, gamma, packed)
    return _cache[key]


def check_forward(wl, li, M, layout, act="normal"):
    layer = wl.layers[li]
    t_ref, g_ref, gamma, packed = prepared(wl, li)
    log("forward", wl.name, layer.name, "M", M, layout)
    seed = workloads.seed_for(wl, li, 1) + M
    if act == "student_t":
        x = synth.activations_student_t_bf16(M, layer.K, seed=seed)
    else:
        x = synth.activations_bf16(M, layer.K, seed=seed)
    xd = to_dev(x)
    P = packed[layout]
    acc = to_host(bl.forward(P, LAYOUTS[layout], gamma, xd, layer.N, layer.K, y_dtype=torch.int32))
    y = to_host(bl.forward(P, LAYOUTS[layout], gamma, xd, layer.N, layer.K, y_dtype=torch.float32))
    ref = _reference(wl, li, M, x, t_ref, g_ref)
    assert np.array_equal(acc, ref["acc"]), f"acc differs at {np.argwhere(acc != ref['acc'])[:5]}"
    assert_f32_parity(y, ref["y"])
    assert np.abs(acc.astype(np.int64)).max() <= 127 * layer.K


_ref_cache = {}


def _reference(wl, li, M, x, t_ref, g_ref):
    """The oracle's forward of one (layer, M), kept while the same layer is
    checked in another layout."""
    key = (wl.name, li, M)
    if key not in _ref_cache:
        _ref_cache.clear()
        _ref_cache[key] = oracle.forward(t_ref, g_ref, x)
    return _ref_cache[key]


def test_tiny_config_full_pipeline():
    """The tiny workload through every entry point, compared in full."""
    wl = workloads.TINY
    layer = wl.layers[0]
    w = synth.latent_weights(layer.N, layer.K, seed=workloads.seed_for(wl, 0, 0))
    x = synth.activations_f32(wl.batches[0], layer.K, seed=workloads.seed_for(wl, 0, 1))
    T, gamma = bl.quantize_weights(to_dev(w))
    t_ref, g_ref = oracle.quantize_weights(w)
    ref = oracle.forward(t_ref, g_ref, x)
    assert np.array_equal(to_host(T), t_ref)
    for name, lay in LAYOUTS.items():
        P = bl.pack(T, lay)
        assert np.array_equal(to_host(P), oracle.pack(t_ref, lay))
        for algo in ((bl.ALGO_AUTO, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA) if name == "b3" else
                     (bl.ALGO_AUTO, bl.ALGO_GEMV_ADDSUB, bl.ALGO_GEMV_MFMA, bl.ALGO_GEMM_MFMA)):
            acc = to_host(bl.forward(P, lay, gamma, to_dev(x), layer.N, layer.K, y_dtype=torch.int32, algo=algo))
            assert np.array_equal(acc, ref["acc"])
            y = to_host(bl.forward(P, lay, gamma, to_dev(x), layer.N, layer.K, algo=algo))
            assert_f32_parity(y, ref["y"])
    Xq, beta = bl.quantize_act(to_dev(x))
    assert np.array_equal(to_host(Xq)[:, :layer.K], ref["q"])
    assert np.array_equal(f32_bits(to_host(beta)), f32_bits(ref["beta"]))


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("li", range(7), ids=[l.name for l in workloads.DECODE_3B.layers])
def test_decode_3b(li, M):
    check_forward(workloads.DECODE_3B, li, M, "i2")


@pytest.mark.parametrize("li", [0, 1, 2], ids=["3200x3200", "8640x3200", "3200x8640"])
def test_prefill_3b(li):
    check_forward(workloads.PREFILL_3B, li, 2048, "i2", act="student_t")


@pytest.mark.parametrize("M", [1, 16, 64, 176])
@pytest.mark.parametrize("li", range(7), ids=[l.name for l in workloads.LAYERS_70B.layers])
def test_llama70b(li, M):
    for layout in ("i2", "b3"):
        check_forward(workloads.LAYERS_70B, li, M, layout)
