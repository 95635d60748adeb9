"""Layer shapes of the MoE workloads.

Pure data: no arithmetic of the method lives here.  ``WORKLOADS`` holds the
five named layer configurations; ``small_case`` builds reduced shapes that keep
a workload's structure (expert count, k, biases, capacity) for fast tests.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    cid: int            # stream id used by the seeded generator
    T: int              # tokens
    d: int              # model width
    E: int              # routed experts
    k: int              # experts per token
    h: int              # routed expert hidden width
    dtype: str          # "f32" or "bf16": storage type of x and every weight
    n_shared: int = 0   # always-on shared experts
    h_shared: int = 0   # hidden width of each shared expert
    cf: float = 0.0     # capacity factor; <= 0 means no capacity limit
    logit_bias: str = "none"    # "none" | "zipf": offsets added to the logits
    select_bias: str = "none"   # "none" | "normal": selection-only bias
    zipf_s: float = 1.1
    select_var: float = 0.5     # variance of the selection bias
    alpha: float = 0.01

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def sigma_in(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def sigma_down(self) -> float:
        return 1.0 / math.sqrt(self.h)

    @property
    def sigma_down_shared(self) -> float:
        return 1.0 / math.sqrt(self.h_shared) if self.h_shared else 0.0


WORKLOADS = {
    "tiny_f32": MoEConfig("tiny_f32", 1, T=64, d=128, E=8, k=2, h=256, dtype="f32"),
    "mixtral_bf16": MoEConfig("mixtral_bf16", 2, T=4096, d=4096, E=8, k=2, h=14336, dtype="bf16"),
    "finegrained_shared_bf16": MoEConfig(
        "finegrained_shared_bf16", 3, T=8192, d=2048, E=128, k=8, h=1024, dtype="bf16",
        n_shared=4, h_shared=1024, logit_bias="zipf"),
    "capacity_balance_bf16": MoEConfig(
        "capacity_balance_bf16", 4, T=16384, d=3072, E=64, k=2, h=4096, dtype="bf16",
        cf=1.25, select_bias="normal"),
    "decode_bf16": MoEConfig(
        "decode_bf16", 5, T=64, d=6144, E=128, k=8, h=2048, dtype="bf16",
        n_shared=1, h_shared=8192),
}

ORDER = ["tiny_f32", "mixtral_bf16", "finegrained_shared_bf16", "capacity_balance_bf16",
         "decode_bf16"]


def small_case(name: str, T: int, d: int, h: int, h_shared: int | None = None,
               cid_offset: int = 100) -> MoEConfig:
    """A reduced copy of a workload: same E, k, dtype, biases and capacity factor."""
    base = WORKLOADS[name]
    return replace(base, name=f"{name}_small", cid=base.cid + cid_offset, T=T, d=d, h=h,
                   h_shared=(h_shared if h_shared is not None else (h if base.n_shared else 0)))
