"""The five workload shapes the decode path is built and measured for.

Shapes follow the models the pages discuss: an OPT-125m-sized layer, an OPT-6.7B-sized
stack, a ReLU-fied Llama-7B-sized gated stack (novita.ai activation-sparsity article,
sections 第一階段 and 第二階段), a batch sweep on it, and an OPT-175B-sized slice (the
model PowerInfer runs on one consumer GPU, section 降低推理門檻 of the same article).
Activity levels follow PowerInfer-2's ~10% active neurons in decode (PowerInfer-2 article,
section 4.1.2 CPU-Centric Decoding).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np


@dataclass(frozen=True)
class Config:
    cid: int               # stable id used in seeds
    name: str
    d: int                 # model dimension
    n: int                 # FFN width d_ffn (number of neurons)
    rank: int              # predictor rank r
    gated: bool            # h = relu(gate) * up  instead of  h = relu(up)
    w_dtype: str           # "f16" or "f32" for the layer weights
    p_dtype: str           # predictor weights dtype
    layers: int
    activity: Tuple[float, ...]  # per-layer target fraction of active neurons
    zipf_s: float          # Zipf exponent of per-neuron activation frequency
    hot_frac: float        # fraction of neurons packed first as "hot"
    x_kind: str            # "normal": x ~ N(0,1); "relu_rmsnorm": x = relu(rmsnorm(z))
    batches: Tuple[int, ...] = (1,)
    rotate_copies: int = 1  # packed copies cycled by the benchmark so a small layer is not cache-resident
    description: str = ""

    def layer_activity(self, layer: int) -> float:
        return float(self.activity[layer])

    @property
    def w_bytes(self) -> int:
        return 2 if self.w_dtype == "f16" else 4

    @property
    def p_bytes(self) -> int:
        return 2 if self.p_dtype == "f16" else 4

    @property
    def m(self) -> int:
        """Weight rows touched per active neuron: up(+gate) and down."""
        return 3 if self.gated else 2


def _const(v, L):
    return tuple([float(v)] * L)


C1 = Config(1, "opt125m_layer", 768, 3072, 64, False, "f32", "f32", 1, _const(0.10, 1), 1.1, 0.20,
            "normal", (1,), rotate_copies=32,
            description="OPT-125m-shaped ReLU FFN layer, fp32, r=64, 10% active, Zipf(1.1)")
C2 = Config(2, "opt6.7b_stack", 4096, 16384, 256, False, "f16", "f16", 32,
            tuple(float(v) for v in np.linspace(0.05, 0.10, 32)), 1.1, 0.20, "normal", (1,),
            description="OPT-6.7B-shaped ReLU FFN stack, 32 layers, fp16, r=256, 5-10% active, Zipf(1.1)")
C3 = Config(3, "llama7b_gated_stack", 4096, 11008, 256, True, "f16", "f16", 32, _const(0.10, 32), 1.0,
            0.20, "relu_rmsnorm", (1,),
            description="Llama-7B-shaped ReLU-fied gated FFN, 32 layers, fp16, r=256, 10% active, Zipf(1.0)")
C4 = Config(4, "llama7b_gated_batch", 4096, 11008, 256, True, "f16", "f16", 32, _const(0.10, 32), 1.0,
            0.20, "relu_rmsnorm", (1, 4, 16, 32),
            description="C3 shape, batch 1/4/16/32 with independent per-token masks")
C5 = Config(5, "opt175b_slice", 12288, 49152, 1024, False, "f16", "f16", 24, _const(0.05, 24), 1.2,
            0.10, "normal", (1,),
            description="OPT-175B-shaped FFN slice, 24 layers, fp16, r=1024, 5% active, Zipf(1.2)")

# The OPT-6.7B-shaped stack with every layer at 10% target activity: the metric's own
# condition (~10% of neurons active in decode, PowerInfer-2 article, section 4.1.2). Same
# config id, so the same seeded weights, tokens and predictor subspaces as C2; only the
# per-neuron biases (which set the activity) differ.
C2_10 = Config(2, "opt6.7b_stack_10pct", 4096, 16384, 256, False, "f16", "f16", 32,
               _const(0.10, 32), 1.1, 0.20, "normal", (1,),
               description="OPT-6.7B-shaped ReLU FFN stack, 32 layers, fp16, r=256, every layer "
                           "10% active, Zipf(1.1)")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C2_10)}
CONFIGS.update({f"C{c.cid}": c for c in (C1, C2, C3, C4, C5)})
CONFIGS["C2_10"] = C2_10


def get_config(name: str) -> Config:
    return CONFIGS[name]
