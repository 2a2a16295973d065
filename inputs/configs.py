"""The denoiser workloads: model geometry, layouts, seeds and distributions.

A layout is a list of runs of the joint sequence, ``("text", n)`` or
``("image", h, w)``; the last run is the target image block, the rest is the
prompt prefix.  Distributions (all drawn by ``inputs.synth``):

* projection matrices N(0, 0.02) -- float32 for the tiny model, rounded to
  bfloat16 for the full-size model;
* per-head q/k norm weights 1 + N(0, 0.02) (trained norms sit near one;
  N(0, 0.02) norms would flatten every softmax row);
* prefix rows and latent tokens N(0, 1);
* the step modulation [s1|g1|s2|g2], the t = 0 prefix modulation (a model
  constant, shared by every prefix of that model) and final_scale N(0, 0.1).

Tensor ids: block ``l`` uses 100 + 16*l + j for j = 0..8 in the order
(to_q, to_k, to_v, to_out, gate, up, down, norm_q, norm_k); img_in 1,
proj_out 2, mods0 3 under the model seed; prefix rows 10 under the prefix
seed; tokens 11, mods 12, final_scale 13 under the workload seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

BLOCK_NAMES = ("to_q", "to_k", "to_v", "to_out", "gate", "up", "down", "norm_q", "norm_k")
TID_IMG_IN, TID_PROJ_OUT, TID_MODS0 = 1, 2, 3
TID_PREFIX_X, TID_TOK, TID_MODS, TID_FINAL_SCALE = 10, 11, 12, 13
# time path (temb MLP, shared modulation, final-norm scale) and the txt_in front
TID_T_LIN1, TID_T_LIN2, TID_MODULATION, TID_NORM_OUT = 20, 21, 22, 23
TID_TXT_NORM, TID_TXT_IN1, TID_TXT_IN2, TID_TXT_FEATS = 24, 25, 26, 27
TEMB_IN = 256  # the sinusoidal timestep embedding's width (128 cos + 128 sin)
W_SIGMA, NORM_SIGMA, ROW_SIGMA, MOD_SIGMA = 0.02, 0.02, 1.0, 0.1


def block_tid(layer: int, j: int) -> int:
    return 100 + 16 * layer + j


@dataclass(frozen=True)
class ModelSpec:
    name: str
    seed: int
    layers: int
    heads: int
    head_dim: int = 128
    mlp_ratio: int = 3
    in_ch: int = 64
    axes: Tuple[int, int, int] = (16, 56, 56)
    theta: float = 10000.0
    eps: float = 1e-6
    bf16: bool = True

    @property
    def dim(self) -> int:
        return self.heads * self.head_dim

    @property
    def inter(self) -> int:
        return self.dim * self.mlp_ratio

    def block_shapes(self):
        h, i, d = self.dim, self.inter, self.head_dim
        return ((h, h), (h, h), (h, h), (h, h), (i, h), (i, h), (h, i), (d,), (d,))


TINY_MODEL = ModelSpec("tiny", seed=21, layers=2, heads=2, bf16=False)
FULL_MODEL = ModelSpec("qi21-32x4096", seed=7, layers=32, heads=32, bf16=True)


def model_spec(name: str) -> ModelSpec:
    return {m.name: m for m in (TINY_MODEL, FULL_MODEL)}[name]


@dataclass(frozen=True)
class Workload:
    name: str
    model: ModelSpec
    seed: int
    target: Tuple[int, int]
    prefixes: Tuple[Tuple[Tuple, ...], ...]
    prefix_seeds: Tuple[int, ...] = field(default=())
    note: str = ""

    def layout(self, p: int = 0) -> List[tuple]:
        return list(self.prefixes[p]) + [("image",) + tuple(self.target)]

    @property
    def n(self) -> int:
        return self.target[0] * self.target[1]

    def prefix_len(self, p: int = 0) -> int:
        return sum(s[1] if s[0] == "text" else s[1] * s[2] for s in self.prefixes[p])

    def prefix_seed(self, p: int = 0) -> int:
        return self.prefix_seeds[p] if self.prefix_seeds else self.seed


CONFIGS = {
    "tiny": Workload("tiny", TINY_MODEL, 21, (16, 16), ((("text", 18),),),
                     note="2 blocks, dim 256 (2 heads x 128), mlp 768, Text(18) + Image(16,16)"),
    "512": Workload("512", FULL_MODEL, 7, (32, 32), ((("text", 18),),),
                    note="512^2 step: 1024 target rows, prefix Text(18)"),
    "1024": Workload("1024", FULL_MODEL, 1024, (64, 64), ((("text", 18),),),
                     note="1024^2 step: 4096 target rows, prefix Text(18)"),
    "cond": Workload("cond", FULL_MODEL, 4118, (64, 64), ((("text", 22), ("image", 64, 64)),),
                     note="prefill Text(22)+Image(64,64) = 4118 rows block-causal, then a 1024^2 step"),
    "2048": Workload("2048", FULL_MODEL, 2048, (128, 128), ((("text", 18),),),
                     note="2048^2 step: 16384 target rows, prefix Text(18)"),
    "cfg512": Workload("cfg512", FULL_MODEL, 7, (32, 32), ((("text", 18),), (("text", 18),)),
                       prefix_seeds=(7, 8),
                       note="CFG pair at 512^2: two Text(18) prefixes (seeds 7, 8), shared tokens and modulation"),
    "ragged": Workload("ragged", FULL_MODEL, 4087, (61, 67), ((("text", 37),),),
                       note="parity case: 4087 target rows (ragged last tile of every GEMM and attention key "
                            "tile) behind a Text(37) prefix"),
}
