"""The five synthetic weight stacks (shapes, distributions, codec and budget).

These stand in for the six unnamed 1.4B-14B models that the AQLoRA abstract
evaluates on (arXiv listing of the AQLoRA paper, English abstract); that
evaluation's fine-tuning dataset is not used because the codec and the
ranking consume weights only.  Matrices are listed block-major, in the order
given per block; layer index = block * matrices_per_block + position.
"""
from __future__ import annotations

from dataclasses import dataclass, field

GIB = 1 << 30

NORMAL, STUDENT_T4 = 0, 1
BF16, FP16 = 0, 1


@dataclass(frozen=True)
class StackConfig:
    cid: int                       # config id: seeds the per-layer generators
    name: str
    blocks: int
    per_block: tuple               # ((matrix name, rows, cols), ...)
    dtype: int = BF16
    dq: bool = True
    dist: int = NORMAL
    sigma_lo: float = 0.02
    sigma_hi: float = 0.0          # > sigma_lo: per-matrix sigma ~ U[lo, hi)
    outlier_frac: float = 0.0
    outlier_scale: float = 10.0
    budgets_gib: tuple = ()        # fp16 promotion budgets in GiB (() = none)
    kcap: int = -1                 # cap on K (-1 = none)
    dequant_repeats: int = 0       # standalone dequant passes after selection
    layers: list = field(init=False, repr=False, compare=False)

    def __post_init__(self):
        ls = []
        for b in range(self.blocks):
            for (nm, r, c) in self.per_block:
                ls.append((f"block{b}.{nm}", r, c))
        object.__setattr__(self, "layers", ls)

    @property
    def n_layers(self) -> int:
        return len(self.layers)

    def n(self, i: int) -> int:
        _, r, c = self.layers[i]
        return r * c

    @property
    def sizes(self) -> list:
        return [r * c for (_, r, c) in self.layers]

    @property
    def total(self) -> int:
        return sum(self.sizes)

    def budgets_bytes(self) -> list:
        return [int(g * GIB) for g in self.budgets_gib]


TOY = StackConfig(
    cid=1, name="toy 2-block decoder, fp16 N(0,0.02), no double quant, top-K=2",
    blocks=2,
    per_block=(("q", 256, 256), ("k", 256, 256), ("v", 256, 256), ("o", 256, 256),
               ("gate", 688, 256), ("up", 688, 256), ("down", 256, 688)),
    dtype=FP16, dq=False, kcap=2)

SINGLE = StackConfig(
    cid=2, name="single 4096x4096 bf16 N(0,0.02), 0.1% x10 outliers, double quant",
    blocks=1, per_block=(("w", 4096, 4096),),
    outlier_frac=0.001)

S1P4B = StackConfig(
    cid=3, name="1.4B-shaped: 24 blocks d=2048, bf16 N(0,s) s~U[0.01,0.04], double quant, 0.2 GiB",
    blocks=24,
    per_block=(("qkv", 6144, 2048), ("out", 2048, 2048), ("up", 8192, 2048), ("down", 2048, 8192)),
    sigma_lo=0.01, sigma_hi=0.04, budgets_gib=(0.2,))

S7B = StackConfig(
    cid=4, name="7B Llama-shaped: 32 blocks d=4096 ffn=11008, bf16 Student-t(4) std 0.02, double quant",
    blocks=32,
    per_block=(("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
               ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)),
    dist=STUDENT_T4, budgets_gib=(0.2, 0.5, 1.0))

# The 14B stack names no budget: 0.2 GiB (the quality setting's extra memory in
# the AQLoRA abstract) is the one its step dequantises against; 0.5 and 1.0
# GiB are also ranked, as for the 7B stack.
S14B = StackConfig(
    cid=5, name="14B-shaped: 40 blocks d=5120 ffn=13824, bf16 N(0,0.02), 0.05% x10 outliers, "
                "double quant, 0.2 GiB (also 0.5 and 1.0 ranked), dequant of unpromoted x2",
    blocks=40,
    per_block=(("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120), ("o", 5120, 5120),
               ("gate", 13824, 5120), ("up", 13824, 5120), ("down", 5120, 13824)),
    outlier_frac=0.0005, budgets_gib=(0.2, 0.5, 1.0), dequant_repeats=2)

CONFIGS = [TOY, SINGLE, S1P4B, S7B, S14B]
BY_NAME = {"toy": TOY, "single": SINGLE, "1.4b": S1P4B, "7b": S7B, "14b": S14B}
