"""The five layer shapes the benchmark and the parity tests run.

Shapes follow the models the PowerInfer pages name (project page, section
"Supported models"; paper summary, "Key Results"): a toy layer, a
LLaMA-7B-ReLU-shaped gated FFN, an OPT-30B-shaped non-gated FFN, a
Falcon-40B-shaped non-gated FFN with int4 weights, and a Llama2-70B-ReLU-shaped
gated FFN decoded at batch 1, 4 and 16.  Densities follow the sparsity levels
the pages quote (about 90 % sparse; 26 % of neurons carrying 80 % of the
activations for OPT-30B).
"""

from dataclasses import dataclass
from typing import Optional, Tuple


@dataclass(frozen=True)
class LayerConfig:
    name: str            # short name used on the command line
    cfg_id: int          # first element of every seed spawn key
    workload: str        # human-readable description
    d_model: int         # d
    d_ffn: int           # n
    rank: int            # r (predictor rank)
    gated: bool
    w_dtype: str         # "f32" | "f16" | "q4g32"
    p_dtype: str         # "f32" | "f16"
    act_dtype: str       # "f32" | "f16"
    n_layers: int        # L distinct layers walked per token
    tokens: int          # seeded tokens per layer
    density: float       # target mean firing probability (1 - sparsity)
    zipf_s: Optional[float]               # power-law exponent; None => solve from top_share
    top_share: Optional[Tuple[float, float]] = None  # (fraction of neurons, share of firing mass)
    batches: Tuple[int, ...] = (1,)
    modes: Tuple[str, ...] = ("predicted",)
    tau: float = 0.5

    @property
    def max_batch(self) -> int:
        return max(self.batches)


CONFIGS = (
    LayerConfig(
        name="toy", cfg_id=0,
        workload="toy non-gated ReLU FFN fp32 d=512 n=2048 r=64, 1 layer",
        d_model=512, d_ffn=2048, rank=64, gated=False,
        w_dtype="f32", p_dtype="f32", act_dtype="f32",
        n_layers=1, tokens=1000, density=0.10, zipf_s=1.1,
        modes=("predicted", "exact", "dense"),
    ),
    LayerConfig(
        name="llama7b", cfg_id=1,
        workload="LLaMA-7B-ReLU-shaped gated FFN fp16 d=4096 n=11008 r=1024, 32 layers, batch 1",
        d_model=4096, d_ffn=11008, rank=1024, gated=True,
        w_dtype="f16", p_dtype="f16", act_dtype="f16",
        n_layers=32, tokens=256, density=0.10, zipf_s=1.1,
        modes=("predicted", "exact", "dense"),
    ),
    LayerConfig(
        name="opt30b", cfg_id=2,
        workload="OPT-30B-shaped non-gated ReLU FFN fp16 d=7168 n=28672 r=1024, 48 layers, batch 1",
        d_model=7168, d_ffn=28672, rank=1024, gated=False,
        w_dtype="f16", p_dtype="f16", act_dtype="f16",
        n_layers=48, tokens=256, density=0.05, zipf_s=None, top_share=(0.26, 0.80),
    ),
    LayerConfig(
        name="falcon40b", cfg_id=3,
        workload="Falcon-40B-shaped non-gated ReLU FFN int4-g32 d=8192 n=32768 r=1024, 60 layers, batch 1",
        d_model=8192, d_ffn=32768, rank=1024, gated=False,
        w_dtype="q4g32", p_dtype="f16", act_dtype="f16",
        n_layers=60, tokens=256, density=0.08, zipf_s=1.1,
    ),
    LayerConfig(
        name="llama70b", cfg_id=4,
        workload="Llama2-70B-ReLU-shaped gated FFN fp16 d=8192 n=28672 r=1024, 80 layers, batch 1/4/16",
        d_model=8192, d_ffn=28672, rank=1024, gated=True,
        w_dtype="f16", p_dtype="f16", act_dtype="f16",
        n_layers=80, tokens=128 * 16, density=0.10, zipf_s=1.1,
        batches=(1, 4, 16),
    ),
)


def config_by_name(name: str) -> LayerConfig:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown config {name!r}; known: {[c.name for c in CONFIGS]}")
