"""The five synthetic workloads (shapes, storage dtype, TwELL tile/capacity, density).

Scale and density follow the pages' setting: billion-parameter language models
whose ReLU FFN activations are more than 99% zero, and whose first tokens of a
sequence are denser than the rest (q2bstudio.com post on TwELL, third
paragraph; gist.science "Sparser, Faster, Lighter Transformer Language
Models", Resumen Técnico §3 and §4).  No dataset or trained weights are used:
Gaussian inputs with a per-token gate bias stand in for them.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .synth import FfnInputs, ffn_inputs, gate_bias_for_density

SEQ = 2048  # tokens per sequence in the batched workloads


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    F: int
    tile: int
    cap: int
    dtype: str
    density: float                    # density of ordinary tokens
    hot_density: Optional[float] = None   # density of the first ``hot_tokens`` of each sequence
    hot_tokens: int = 0
    literal_bias: Optional[float] = None  # use this bias instead of the density formula
    description: str = ""

    @property
    def n_tiles(self) -> int:
        return self.F // self.tile

    def bias_vector(self, T: Optional[int] = None) -> np.ndarray:
        T = self.T if T is None else T
        if self.literal_bias is not None:
            b = np.full(T, self.literal_bias)
        else:
            b = np.full(T, gate_bias_for_density(self.density))
        if self.hot_density is not None and self.hot_tokens > 0:
            t = np.arange(T)
            b = np.where((t % SEQ) < self.hot_tokens, gate_bias_for_density(self.hot_density), b)
        return b.astype(np.float32)

    def inputs(self, seed: int = 0, T: Optional[int] = None) -> FfnInputs:
        T = self.T if T is None else T
        return ffn_inputs(T, self.d, self.F, self.dtype, seed, self.bias_vector(T))

    def with_density(self, rho: float) -> "Workload":
        return Workload(f"{self.name}@{rho:g}", self.T, self.d, self.F, self.tile, self.cap,
                        self.dtype, rho, description=self.description)

    def summary(self) -> Dict[str, object]:
        out = {"workload": self.name, "T": self.T, "d_model": self.d, "d_ff": self.F,
               "tile": self.tile, "cap": self.cap, "dtype": self.dtype,
               "density": self.density}
        if self.hot_density is not None:
            out.update(hot_density=self.hot_density, hot_tokens_per_seq=self.hot_tokens)
        return out


CONFIGS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 64, 256, 1024, 128, 8, "f32", 0.01, literal_bias=-2.326,
                         description="tiny fp32 layer, about 1% active"),
    "layer_1p5b_bf16": Workload("layer_1p5b_bf16", 4 * SEQ, 2048, 8192, 256, 16, "bf16", 0.01,
                                description="1.5B-class bf16 layer, about 1% uniform activation"),
    "skewed_bf16": Workload("skewed_bf16", 4 * SEQ, 2048, 8192, 256, 16, "bf16", 0.01,
                            hot_density=0.20, hot_tokens=64,
                            description="1.5B-class shapes; first 64 tokens of each sequence 20% active"),
    "large_bf16": Workload("large_bf16", 8 * SEQ, 4096, 14336, 256, 16, "bf16", 0.005,
                           description="larger bf16 layer, about 0.5% activation"),
}

SWEEP_DENSITIES: Tuple[float, ...] = (0.001, 0.005, 0.01, 0.02, 0.05, 0.10)


def workload(name: str) -> Workload:
    if name in CONFIGS:
        return CONFIGS[name]
    if name.startswith("sweep@"):
        return CONFIGS["layer_1p5b_bf16"].with_density(float(name.split("@", 1)[1]))
    raise KeyError(name)
