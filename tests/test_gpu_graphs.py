"""HIP-graph capture of the multi-launch paths: the prefill forward (quantiser
into the workspace, then the GEMM; b3 weights rewritten as i2 first where the
GEMM does not decode them), and the backward (dX with its weight rows split
over workgroups plus the in-order sum, dW).  Each graph is replayed several
times with other eager work between the replays, and every replay must give
the eager result bit for bit: the library records no memset and keeps no state
between calls."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth  # noqa: E402

from gpu_helpers import assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu
LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3}


def log(*a):
    print(*a, flush=True)


def replay_matches(run, out, noise):
    """Capture run() (which writes out) in a graph on a side stream, then
    replay it 3 times, each after clearing out and running noise() eagerly."""
    want = to_host(out).copy()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        run()
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan"))
        noise()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32)), f"replay {r}"


@pytest.mark.parametrize("layout,M,N,K", [("i2", 300, 4000, 640), ("b3", 300, 4000, 640), ("b3", 64, 20000, 256)],
                         ids=["i2_gemm", "b3_gemm_300_tokens", "b3_gemm_64_tokens"])
def test_prefill_forward_graph_replay(layout, M, N, K):
    log("graph prefill", layout, M, N, K)
    t = synth.ternary_weights(N, K, seed=M + N)
    x_np = synth.activations_bf16(M, K, seed=K)
    x = to_dev(x_np)
    P = to_dev(oracle.pack(t, LAYOUTS[layout]))
    gamma = to_dev(np.array([0.02], np.float32))
    assert bl.bitlinear_product_kernel(M, N, K, LAYOUTS[layout], bl.BF16).startswith("bl::k_gemm_mfma_")
    out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    bl.forward(P, LAYOUTS[layout], gamma, x, N, K, out=out)
    torch.cuda.synchronize()
    assert_f32_parity(to_host(out), oracle.forward(t, np.float32(0.02), x_np)["y"])
    x2 = to_dev(synth.activations_bf16(M // 2, K, seed=K + 1))
    replay_matches(lambda: bl.forward(P, LAYOUTS[layout], gamma, x, N, K, out=out), out,
                   lambda: bl.forward(P, LAYOUTS[layout], gamma, x2, N, K))


def test_backward_graph_replay():
    M, N, K = 1, 3200, 3200
    log("graph backward", M, N, K)
    assert bl.bitlinear_backward_dx_workspace_bytes(M, N, K, bl.LAYOUT_I2) > 0  # the split path
    t = synth.ternary_weights(N, K, seed=71)
    P = to_dev(oracle.pack(t, bl.LAYOUT_I2))
    gamma = to_dev(np.array([0.03], np.float32))
    dy = to_dev(synth.activations_f32(M, N, seed=72))
    dx = torch.empty((M, K), dtype=torch.float32, device=dy.device)
    bl.backward_dx(P, bl.LAYOUT_I2, gamma, dy, K, out=dx)
    dy2 = to_dev(synth.activations_f32(5, N, seed=73))
    replay_matches(lambda: bl.backward_dx(P, bl.LAYOUT_I2, gamma, dy, K, out=dx), dx,
                   lambda: bl.backward_dx(P, bl.LAYOUT_I2, gamma, dy2, K))
    x = to_dev(synth.activations_bf16(M, K, seed=74))
    Xq, beta = bl.quantize_act(x)
    dw = torch.empty((N, K), dtype=torch.float32, device=dy.device)
    bl.backward_dw(Xq, beta, dy, K, out=dw)
    replay_matches(lambda: bl.backward_dw(Xq, beta, dy, K, out=dw), dw,
                   lambda: bl.backward_dx(P, bl.LAYOUT_I2, gamma, dy2, K))
