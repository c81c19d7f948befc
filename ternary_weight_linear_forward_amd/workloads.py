"""Named workloads: the layer shapes of the pages' 3B and 70B LLaMA-style models.

The pages report the 3B model's decode latency and memory and the 70B model's
batch and throughput (LIT-380 record, Key takeaways, bullets 4 and 5); the
shapes below are those models' linear layers (3B: hidden 3200, FFN 8640,
26 layers; 70B: hidden 8192, FFN 28672, grouped k/v of width 1024).  W is
[N x K] like nn.Linear.weight, X is [M x K], Y is [M x N].
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .synth import BASE_SEED


@dataclass(frozen=True)
class Layer:
    name: str
    N: int
    K: int


@dataclass(frozen=True)
class Workload:
    name: str
    layers: tuple
    batches: tuple
    layouts: tuple = ("i2",)
    act_dist: str = "normal"          # "normal" | "student_t"
    x_dtype: str = "bf16"             # "f32" | "bf16"
    seed: int = BASE_SEED
    notes: str = field(default="", compare=False)


TINY = Workload(
    name="tiny_512x256",
    layers=(Layer("w", 512, 256),),
    batches=(16,),
    x_dtype="f32",
    seed=BASE_SEED + 0,
    notes="W fp32 [512 x 256] ~ N(0, 0.02^2); X fp32 [16 x 256] ~ N(0, 1)",
)

_3B = (
    Layer("q", 3200, 3200), Layer("k", 3200, 3200), Layer("v", 3200, 3200), Layer("o", 3200, 3200),
    Layer("gate", 8640, 3200), Layer("up", 8640, 3200), Layer("down", 3200, 8640),
)

DECODE_3B = Workload(
    name="decode_3b",
    layers=_3B,
    batches=(1, 4, 16),
    seed=BASE_SEED + 100,
    notes="3B decode GEMV: q/k/v/o 3200x3200, gate/up 8640x3200, down 3200x8640; M in {1,4,16}; i2",
)

PREFILL_3B = Workload(
    name="prefill_3b",
    layers=(Layer("qkvo", 3200, 3200), Layer("gate_up", 8640, 3200), Layer("down", 3200, 8640)),
    batches=(2048,),
    act_dist="student_t",
    seed=BASE_SEED + 200,
    notes="3B prefill GEMM: M = 2048, Student-t(4) activations; i2",
)

LAYERS_70B = Workload(
    name="llama70b_layers",
    layers=(Layer("q", 8192, 8192), Layer("k", 1024, 8192), Layer("v", 1024, 8192), Layer("o", 8192, 8192),
            Layer("gate", 28672, 8192), Layer("up", 28672, 8192), Layer("down", 8192, 28672)),
    batches=(1, 16, 64, 176),
    layouts=("i2", "b3"),
    seed=BASE_SEED + 300,
    notes="70B layers on one GPU, K = 8192 (down: K = 28672), M in {1,16,64,176}; i2 and b3",
)

STACK_3B = Workload(
    name="stack_3b_26",
    layers=(Layer("qkv", 9600, 3200), Layer("o", 3200, 3200), Layer("gate_up", 17280, 3200), Layer("down", 3200, 8640)),
    batches=(16,),
    seed=BASE_SEED + 400,
    notes="26-layer 3B BitLinear stack, batch 16 decode; per layer qkv -> o -> gate_up -> down",
)
STACK_DEPTH = 26

ALL = {w.name: w for w in (TINY, DECODE_3B, PREFILL_3B, LAYERS_70B, STACK_3B)}


def seed_for(workload: Workload, layer_index: int, tensor: int, copy: int = 0) -> int:
    """Seed of one tensor: the workload base + layer, tensor kind and copy index."""
    return workload.seed + 1000 * copy + 10 * layer_index + tensor


@dataclass(frozen=True)
class StackLink:
    """One BitLinear of the stack in execution order.  Its input is the first
    K columns of the previous link's output (width 'ld_in'), or the stack
    input X0 for the first link."""
    index: int        # 0 .. 4*depth-1, execution order
    depth: int        # decoder layer 0 .. depth-1
    layer: Layer
    ld_in: int        # row stride of the input (the producer's N; K for X0)


def stack_chain(depth: int = STACK_DEPTH) -> list:
    """The stack's BitLinears: per decoder layer qkv (3200 -> 9600), o reading
    columns 0..3199 of qkv's output, gate_up (3200 -> 17280), down reading
    columns 0..8639 of gate_up's output.  down's output feeds the next
    layer's qkv.  Each link re-quantises its fp32 input per token."""
    links = []
    prev_n = STACK_3B.layers[0].K
    for d in range(depth):
        for layer in STACK_3B.layers:
            links.append(StackLink(len(links), d, layer, prev_n))
            prev_n = layer.N
    return links
