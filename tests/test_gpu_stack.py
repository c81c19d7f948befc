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
