"""The 3B decoder stack's BitLinear chain at batch 16 (qkv -> o -> gate_up ->
down per layer), against the oracle.

Each link quantises the first K columns of the previous link's fp32 output
inside its own forward call (a strided view, no copy).  Parity is checked per
link with teacher forcing: the oracle gets the same fp32 input the GPU link
got, so one rounding-boundary flip cannot cascade down the chain.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import assert_f32_parity, f32_bits, to_dev, to_host
from ternary_weight_linear_forward_amd import bitlinear as bl
from ternary_weight_linear_forward_amd import synth, workloads

pytestmark = pytest.mark.gpu

M = 16


def _stack_weights(chain):
    """Per link: GPU-packed weights and gamma, and the oracle's (T, gamma)
    from the same latent fp32 matrix."""
    out = []
    for link in chain:
        layer = link.layer
        w = synth.latent_weights(layer.N, layer.K, seed=workloads.seed_for(workloads.STACK_3B, link.index, 0))
        T, gamma = bl.quantize_weights(to_dev(w))
        P = bl.pack(T, bl.LAYOUT_I2)
        del T
        out.append((P, gamma, oracle.quantize_weights(w)))
    return out


@pytest.fixture(scope="module")
def stack2():
    chain = workloads.stack_chain(2)
    x0 = synth.activations_bf16(M, chain[0].layer.K, seed=workloads.seed_for(workloads.STACK_3B, 0, 1))
    return chain, _stack_weights(chain), x0


def _run_chain(chain, weights, x0_dev, outs=None):
    """Eager forward through the chain; returns every link's input view and output."""
    ins, ys = [], []
    x = x0_dev
    for i, (link, (P, gamma, _)) in enumerate(zip(chain, weights)):
        K = link.layer.K
        xin = x if i == 0 else x[:, :K]
        y = bl.forward(P, bl.LAYOUT_I2, gamma, xin, link.layer.N, K, out=None if outs is None else outs[i])
        ins.append(xin)
        ys.append(y)
        x = y
    return ins, ys


def test_stack_links_teacher_forced(stack2):
    chain, weights, x0 = stack2
    ins, ys = _run_chain(chain, weights, to_dev(x0))
    torch.cuda.synchronize()
    for link, (P, gamma, (t_ref, g_ref)), xin, y in zip(chain, weights, ins, ys):
        assert np.array_equal(f32_bits(to_host(gamma).reshape(1)), f32_bits(np.float32(g_ref).reshape(1))), link
        x_host = to_host(xin)
        if link.index > 0:
            assert x_host.dtype == np.float32 and x_host.shape == (M, link.layer.K)
            assert np.isfinite(x_host).all()
        ref = oracle.forward(t_ref, g_ref, x_host)
        assert_f32_parity(to_host(y), ref["y"])


def test_stack_graph_replay_matches_eager(stack2):
    """The chain captured once as a HIP graph and replayed, with eager work
    and host synchronisation between replays: every replay's final output is
    bit-identical to the eager chain's."""
    chain, weights, x0 = stack2
    x0_dev = to_dev(x0)
    _, ys_eager = _run_chain(chain, weights, x0_dev)
    want = to_host(ys_eager[-1])
    outs = [torch.empty_like(y) for y in ys_eager]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        _run_chain(chain, weights, x0_dev, outs)  # warm-up on the capture stream
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            _run_chain(chain, weights, x0_dev, outs)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _run_chain(chain[:1], weights[:1], x0_dev)  # unrelated eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f32_bits(to_host(outs[-1])), f32_bits(want)), f"replay {r}"


def _run_chain_f1(chain, weights, x0_dev, outs=None):
    """The chain through bitlinear_forward_chain: each link's product also
    writes its per-workgroup maxima of |Y| over the next link's K columns, and
    the next link's quantiser takes beta from them."""
    ins, ys, pms = [], [], []
    x, pm = x0_dev, None
    for i, (link, (P, gamma, _)) in enumerate(zip(chain, weights)):
        K = link.layer.K
        xin = x if i == 0 else x[:, :K]
        cols = chain[i + 1].layer.K if i + 1 < len(chain) else 0
        y, pm_out = bl.forward_chain(P, bl.LAYOUT_I2, gamma, xin, link.layer.N, K, pmax_in=pm, pmax_cols=cols,
                                     out=None if outs is None else outs[i])
        ins.append(xin)
        ys.append(y)
        pms.append(pm_out)
        x, pm = y, pm_out
    return ins, ys, pms


def test_stack_f1_chain_matches_plain_chain_and_oracle(stack2):
    """Producer-side per-token maxima (f1): every link's output is
    bit-identical to the plain chain's, each link's partial maxima reduce to
    exactly max |y[:, :K_next]| per token, and each link equals the oracle on
    its own fp32 input (teacher forcing)."""
    chain, weights, x0 = stack2
    x0_dev = to_dev(x0)
    _, ys_plain = _run_chain(chain, weights, x0_dev)
    ins, ys, pms = _run_chain_f1(chain, weights, x0_dev)
    torch.cuda.synchronize()
    for i, (link, (P, gamma, (t_ref, g_ref)), xin, y, yp, pm) in enumerate(
            zip(chain, weights, ins, ys, ys_plain, pms)):
        y_host = to_host(y)
        assert np.array_equal(f32_bits(y_host), f32_bits(to_host(yp))), link
        assert_f32_parity(y_host, oracle.forward(t_ref, g_ref, to_host(xin))["y"])
        if i + 1 < len(chain):
            cols = chain[i + 1].layer.K
            parts = bl.bitlinear_forward_chain_parts(M, link.layer.N, link.layer.K, bl.LAYOUT_I2)
            pm_host = to_host(pm).reshape(parts, 16)
            want = np.abs(y_host[:, :cols]).max(axis=1)
            assert np.array_equal(f32_bits(pm_host.max(axis=0)), f32_bits(want)), link
            assert (pm_host >= 0).all()
        else:
            assert pm is None


@pytest.mark.parametrize("M_,N,K,cols", [(16, 3200, 3200, 3200), (5, 9600, 3200, 3200), (16, 17280, 3200, 8640),
                                          (1, 300, 200, 123)])
def test_chain_link_bf16_output_and_consumer(M_, N, K, cols):
    """One producer with bf16 output (the maxima are taken on the bf16 values
    as stored) and a consumer reading those bf16 columns with the producer's
    maxima: both bit-identical to bitlinear_forward, the maxima exact."""
    print("chain bf16", M_, N, K, cols, flush=True)
    t1 = synth.ternary_weights(N, K, seed=N + K)
    t2 = synth.ternary_weights(64, cols, seed=N + cols + 1)
    P1, P2 = to_dev(oracle.pack(t1, bl.LAYOUT_I2)), to_dev(oracle.pack(t2, bl.LAYOUT_I2))
    g = to_dev(np.array([0.021], np.float32))
    x = to_dev(synth.activations_bf16(M_, K, seed=K + M_))
    y, pm = bl.forward_chain(P1, bl.LAYOUT_I2, g, x, N, K, pmax_cols=cols, y_dtype=torch.bfloat16)
    y_plain = bl.forward(P1, bl.LAYOUT_I2, g, x, N, K, y_dtype=torch.bfloat16)
    assert np.array_equal(to_host(y.view(torch.int16)), to_host(y_plain.view(torch.int16)))
    parts = bl.bitlinear_forward_chain_parts(M_, N, K, bl.LAYOUT_I2)
    pm_host = to_host(pm).reshape(parts, 16)
    want = np.abs(to_host(y.float())[:, :cols]).max(axis=1)
    assert np.array_equal(f32_bits(pm_host.max(axis=0)[:M_]), f32_bits(want))
    assert (pm_host[:, M_:] == 0).all()
    z, _ = bl.forward_chain(P2, bl.LAYOUT_I2, g, y[:, :cols], 64, cols, pmax_in=pm)
    z_plain = bl.forward(P2, bl.LAYOUT_I2, g, y[:, :cols], 64, cols)
    assert np.array_equal(f32_bits(to_host(z)), f32_bits(to_host(z_plain)))


def test_stack_f1_graph_replay_matches_eager(stack2):
    """The f1 chain captured as a HIP graph (the maxima buffers included) and
    replayed with eager work between replays: bit-identical to eager."""
    chain, weights, x0 = stack2
    x0_dev = to_dev(x0)
    _, ys_eager, _ = _run_chain_f1(chain, weights, x0_dev)
    want = to_host(ys_eager[-1])
    outs = [torch.empty_like(y) for y in ys_eager]
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        _run_chain_f1(chain, weights, x0_dev, outs)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            _run_chain_f1(chain, weights, x0_dev, outs)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        _run_chain(chain[:1], weights[:1], x0_dev)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(f32_bits(to_host(outs[-1])), f32_bits(want)), f"replay {r}"


_carry = {}


@pytest.mark.parametrize("depth", range(workloads.STACK_DEPTH))
def test_stack_all_layers_teacher_forced(depth):
    """All 26 decoder layers (104 links) of the stack, in order: each layer
    starts from the GPU output of the layer before, and each of its four links
    is compared in full with the oracle on the same fp32 input."""
    chain = workloads.stack_chain()
    links = chain[4 * depth: 4 * depth + 4]
    if depth == 0:
        x = to_dev(synth.activations_bf16(M, links[0].layer.K, seed=workloads.seed_for(workloads.STACK_3B, 0, 1)))
    elif _carry.get("depth") == depth - 1:
        x = _carry["x"]
    else:
        pytest.skip("starts from the previous layer's output: run the layers in order")
    print("stack layer", depth, flush=True)
    weights = _stack_weights(links)
    ins, ys = _run_chain(links, weights, x)
    torch.cuda.synchronize()
    for link, (P, gamma, (t_ref, g_ref)), xin, y in zip(links, weights, ins, ys):
        assert to_host(gamma).view(np.uint32)[0] == np.float32(g_ref).view(np.uint32), link
        x_host = to_host(xin)
        ref = oracle.forward(t_ref, g_ref, synth.bf16_bits_to_f32(x_host) if x_host.dtype == np.uint16 else x_host)
        assert_f32_parity(to_host(y), ref["y"])
    _carry.update(depth=depth, x=ys[-1])
