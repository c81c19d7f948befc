"""GPU parity of the grouped forward (bitlinear_forward_grouped): several
BitLinears of at most 16 tokens in one quantiser launch and one product
launch, every output compared in full with the oracle (int32 accumulators
exact, fp32 / bf16 outputs bit-identical).  Covers the decode layer set of the
3B model at 1, 4 and 16 tokens, inputs shared between jobs (q / k / v), mixed
token counts, ragged shapes, every layout and input dtype, jobs the grouped
launch leaves to a plain forward (more than 16 tokens, very long rows), tiny
activation rows, replay from a HIP graph, and the vector-ALU (add/subtract)
products of bitlinear_forward_grouped_algo for one-token i2 jobs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from ternary_weight_linear_forward_amd import bitlinear as bl  # noqa: E402
from ternary_weight_linear_forward_amd import synth, workloads  # noqa: E402

from gpu_helpers import assert_bf16_parity, assert_f32_parity, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu
LAYOUTS = {"i2": bl.LAYOUT_I2, "b3": bl.LAYOUT_B3, "b1": bl.LAYOUT_B1}


def log(*a):
    print(*a, flush=True)


class Case:
    """Jobs (M, N, K, input id) with seeded weights and inputs; jobs with the
    same input id share one X."""

    def __init__(self, layout, shapes, xk="bf16", seed=0, tiny=False, pad=False, algo=bl.ALGO_AUTO):
        self.layout, self.xk, self.algo = layout, xk, algo
        self.t, self.g, self.P, self.gd = [], [], [], []
        self.x_host, self.x_dev = {}, {}
        self.shapes = shapes
        for idx, (M, N, K, xid) in enumerate(shapes):
            s = seed + 101 * idx
            t = synth.binary_weights(N, K, s) if layout == "b1" else synth.ternary_weights(N, K, s)
            self.t.append(t)
            g = np.float32(0.01 + 0.001 * idx)
            self.g.append(g)
            self.P.append(to_dev(oracle.pack(t, LAYOUTS[layout])))
            self.gd.append(to_dev(np.array([g], np.float32)))
            if xid not in self.x_host:
                x = (synth.activations_bf16 if xk == "bf16" else synth.activations_f32)(M, K, seed + 7 * xid + 1)
                if tiny:
                    xf = (synth.bf16_bits_to_f32(x) if xk == "bf16" else x).astype(np.float64)
                    xf[::2] *= 2.0 ** -130
                    x = synth.to_bf16_bits(xf.astype(np.float32)) if xk == "bf16" else xf.astype(np.float32)
                self.x_host[xid] = x
                if pad:  # rows padded to 16 bytes, passed as a strided view
                    ld = -(-K * x.itemsize // 16) * 16 // x.itemsize
                    xw = np.zeros((M, ld), x.dtype)
                    xw[:, :K] = x
                    self.x_dev[xid] = to_dev(xw)[:, :K]
                else:
                    self.x_dev[xid] = to_dev(x)

    def kernel(self):
        xdt = bl.BF16 if self.xk == "bf16" else bl.F32
        return bl.bitlinear_grouped_kernel_algo(bl.grouped_jobs(self.specs())[0], len(self.shapes),
                                                LAYOUTS[self.layout], xdt, self.algo)

    def specs(self):
        return [(self.P[j], self.gd[j], self.x_dev[xid], N, K) for j, (M, N, K, xid) in enumerate(self.shapes)]

    def check(self, y_kinds=("i32", "f32", "bf16")):
        refs = []
        for j, (M, N, K, xid) in enumerate(self.shapes):
            x = self.x_host[xid]
            refs.append(oracle.forward(self.t[j], self.g[j], synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x))
        for yk in y_kinds:
            ydt = {"i32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16}[yk]
            ys = bl.forward_grouped(self.specs(), LAYOUTS[self.layout], y_dtype=ydt, algo=self.algo)
            for j, (y, ref) in enumerate(zip(ys, refs)):
                y = to_host(y)
                if yk == "i32":
                    assert np.array_equal(y, ref["acc"]), f"job {j}: acc differs at {np.argwhere(y != ref['acc'])[:5]}"
                elif yk == "f32":
                    assert_f32_parity(y, ref["y"])
                else:
                    assert_bf16_parity(y, ref["y"], oracle.f32_to_bf16(ref["y"]))


def decode_layers(M):
    return [(M, l.N, l.K, idx) for idx, l in enumerate(workloads.DECODE_3B.layers)]


@pytest.mark.parametrize("M", [1, 4, 16])
def test_grouped_decode_3b_layer_set(M):
    c = Case("i2", decode_layers(M), seed=M)
    kname = bl.bitlinear_grouped_kernel(bl.grouped_jobs(c.specs())[0], 7, bl.LAYOUT_I2, bl.BF16)
    log("grouped decode 3b", M, kname)
    assert kname == ("bl::k_group_gemv_addsub<1>" if M == 1 else "bl::k_group_gemv<0, 1>" if M == 4
                     else "bl::k_group_gemv<0, 2>"), kname
    c.check()


def test_grouped_decode_3b_all_token_counts_in_one_call():
    shapes = decode_layers(1) + [(4, N, K, 10 + i) for (_, N, K, i) in decode_layers(4)] + \
        [(16, N, K, 20 + i) for (_, N, K, i) in decode_layers(16)]
    log("grouped decode 3b, 21 jobs")
    Case("i2", shapes, seed=5).check(("i32", "f32"))


def test_grouped_shared_inputs():
    # q, k, v share one input; gate and up another; o and down their own
    shapes = [(4, 3200, 3200, 0), (4, 3200, 3200, 0), (4, 3200, 3200, 0), (4, 3200, 3200, 1),
              (4, 8640, 3200, 2), (4, 8640, 3200, 2), (4, 3200, 8640, 3)]
    Case("i2", shapes, seed=9).check()


@pytest.mark.parametrize("xk", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["i2", "b3", "b1"])
def test_grouped_ragged(layout, xk):
    shapes = [(1, 17, 64, 0), (3, 700, 1001, 1), (16, 1000, 77, 2), (5, 333, 3203, 3), (2, 8640, 3200, 4),
              (16, 48, 12288 if layout != "b1" else 8192, 5), (9, 1, 1, 6)]
    log("grouped ragged", layout, xk)
    Case(layout, shapes, xk=xk, seed=13).check()


def test_grouped_with_jobs_left_to_plain_forwards():
    # 20 tokens, and a row of 28672 (112 k-steps): outside the grouped launch
    shapes = [(1, 3200, 3200, 0), (20, 640, 3200, 1), (1, 1024, 28672, 2), (16, 8640, 3200, 3)]
    Case("i2", shapes, seed=17).check(("i32", "f32"))


@pytest.mark.parametrize("layout", ["i2", "b3"])
def test_grouped_llama70b_shapes(layout):
    shapes = [(16, 8192, 8192, 0), (16, 1024, 8192, 0), (16, 1024, 8192, 0), (1, 28672, 8192, 1)]
    Case(layout, shapes, seed=21).check(("i32", "f32"))


def test_grouped_tiny_rows():
    shapes = [(4, 3200, 3200, 0), (16, 8640, 3200, 1), (1, 3200, 8640, 2)]
    Case("i2", shapes, seed=23, tiny=True).check(("i32", "f32"))
    Case("b3", shapes, xk="f32", seed=24, tiny=True).check(("i32", "f32"))


def test_grouped_graph_replay():
    """The grouped forward captured in a HIP graph and replayed with eager work
    between replays gives the eager result every time."""
    c = Case("i2", decode_layers(4), seed=31)
    specs = c.specs()
    want = [to_host(y) for y in bl.forward_grouped(specs)]
    outs = [torch.empty_like(torch.from_numpy(w)).to("cuda") for w in want]
    ws = torch.empty(max(bl.bitlinear_forward_grouped_workspace_bytes(bl.grouped_jobs(specs)[0], len(specs),
                                                                        bl.LAYOUT_I2, bl.BF16), 1),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        bl.forward_grouped(specs, outs=outs, ws=ws)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            bl.forward_grouped(specs, outs=outs, ws=ws)
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        bl.forward_grouped(specs[:2])  # unrelated eager work
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(to_host(o).view(np.uint32), w.view(np.uint32)), r


def test_grouped_split_over_several_launches():
    # 4096 row tiles per job: more workgroups than one grouped launch maps, so
    # the jobs are spread over several product launches
    shapes = [(2, 65536, 64, 0), (1, 65536, 130, 1), (4, 65536, 64, 0)]
    Case("i2", shapes, seed=37).check(("i32", "f32"))


@pytest.mark.parametrize("xk", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["i2", "b3", "b1"])
def test_grouped_quantiser_inside(layout, xk):
    """1 to 4 tokens in every job, 16-byte aligned rows: the product launch
    quantises the activations itself (no quantiser launch); ragged K and N,
    zero, tie and tiny rows."""
    shapes = [(1, 17, 64, 0), (3, 700, 1001, 1), (4, 1000, 77, 2), (2, 333, 3203, 3), (4, 8640, 3200, 4),
              (1, 48, 8192, 5), (4, 3200, 3200, 6)]
    c = Case(layout, shapes, xk=xk, seed=41, pad=True)
    x = c.x_host[6]
    xf = synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x
    xf = xf.copy()
    xf[0] = 0.0                                         # zero token
    xf[1, :7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0]
    xf[1, 7:] = 0.0                                     # ties
    xf[2] = (xf[2].astype(np.float64) * 2.0 ** -130).astype(np.float32)  # subnormal token
    c.x_host[6] = synth.to_bf16_bits(xf) if x.dtype == np.uint16 else xf
    c.x_dev[6] = to_dev(c.x_host[6])
    kname = c.kernel()
    log("grouped, quantiser inside", layout, xk, kname)
    assert kname == f"bl::k_group_gemv<{LAYOUTS[layout]}, {bl.BF16 if xk == 'bf16' else bl.F32}>", kname
    c.check()


@pytest.mark.parametrize("xk", ["bf16", "f32"])
def test_grouped_addsub_decode_3b(xk):
    """The 3B decode layer set at one token with the products on the vector
    ALU: the same results as the oracle (and so as the matrix-core products)."""
    c = Case("i2", decode_layers(1), xk=xk, seed=43, algo=bl.ALGO_GEMV_ADDSUB)
    kname = c.kernel()
    log("grouped add/sub decode 3b", xk, kname)
    assert kname == f"bl::k_group_gemv_addsub<{bl.BF16 if xk == 'bf16' else bl.F32}>", kname
    c.check()


@pytest.mark.parametrize("xk", ["bf16", "f32"])
def test_grouped_addsub_ragged_and_special_rows(xk):
    """Ragged K and N, one to three k-steps per wave (K up to 12288), and a
    zero, a tie and a tiny row, each job one token."""
    shapes = [(1, 17, 64, 0), (1, 700, 1001, 1), (1, 1000, 77, 2), (1, 333, 3203, 3), (1, 8640, 3200, 4),
              (1, 48, 8192, 5), (1, 130, 12288, 6), (1, 64, 256, 7), (1, 40, 640, 8), (1, 2000, 3200, 9)]
    c = Case("i2", shapes, xk=xk, seed=47, pad=True, algo=bl.ALGO_GEMV_ADDSUB)
    for xid, fill in ((7, "zero"), (8, "ties"), (9, "tiny")):
        x = c.x_host[xid]
        xf = (synth.bf16_bits_to_f32(x) if x.dtype == np.uint16 else x).copy()
        if fill == "zero":
            xf[:] = 0.0
        elif fill == "ties":
            xf[0, :] = 0.0
            xf[0, :7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -127.0]
        else:
            xf = (xf.astype(np.float64) * 2.0 ** -130).astype(np.float32)
        c.x_host[xid] = synth.to_bf16_bits(xf) if x.dtype == np.uint16 else xf
        c.x_dev[xid] = to_dev(c.x_host[xid])
    log("grouped add/sub ragged", xk, c.kernel())
    c.check()


def test_grouped_addsub_matches_matrix_cores_bitwise():
    """Both product algorithms of the grouped forward give the same bits."""
    c = Case("i2", decode_layers(1), seed=53)
    specs = c.specs()
    for ydt in (torch.int32, torch.float32, torch.bfloat16):
        a = bl.forward_grouped(specs, y_dtype=ydt, algo=bl.ALGO_GEMV_ADDSUB)
        m = bl.forward_grouped(specs, y_dtype=ydt, algo=bl.ALGO_GEMV_MFMA)
        for ya, ym in zip(a, m):
            assert torch.equal(ya.view(torch.int16 if ydt == torch.bfloat16 else torch.int32),
                               ym.view(torch.int16 if ydt == torch.bfloat16 else torch.int32))


def test_grouped_addsub_with_a_long_row_left_to_the_plain_gemv():
    """A one-token job whose row is too long for the grouped launch (112
    k-steps) runs on the single-layer add/sub GEMV beside the grouped ones."""
    shapes = [(1, 3200, 3200, 0), (1, 1024, 28672, 1), (1, 8640, 3200, 0)]
    c = Case("i2", shapes, seed=59, algo=bl.ALGO_GEMV_ADDSUB)
    log("grouped add/sub with a plain job", c.kernel())
    c.check(("i32", "f32"))
