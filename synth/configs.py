"""The five seeded workloads of the verify hot path, and small variants of them.

Each entry states the batch B, the drafted block length gamma, the drafter hidden
size d, the vocabulary V, how the confidence inputs, the cut and the target
logits are drawn, and how many seeded steps the workload has.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    index: int                 # seed-stream id of the workload (1..5)
    B: int
    gamma: int
    d: int
    V: int
    bias: float                # scalar bias of the confidence head
    temp_slope: float          # STS temperatures T_i = 1 + temp_slope * i, i = 0..gamma-1
    mode: str                  # "threshold", "budget", "static" or "combined"
    cutoff: Optional[float] = None              # fixed per-request cutoff c
    cutoff_range: Optional[Tuple[float, float]] = None  # c_b ~ U[lo, hi] per request and step
    budget_per_request: Optional[float] = None  # T = floor(budget_per_request * B)
    logit_var: float = 1.0     # target logits ~ N(0, logit_var)
    shift: str = "none"        # per-request confidence-logit shift: none | normal | bimodal
    latent: bool = False       # per-position latent logit zeta ~ N(0,1) added to the shift
    match: str = "const"       # const | decay | sigmoid | bimodal
    match_p: float = 0.7
    steps: int = 10

    @property
    def budget(self) -> int:
        if self.mode not in ("budget", "combined"):
            return 0
        return int(self.budget_per_request * self.B)

    @property
    def rows_dense(self) -> int:
        return self.B * (self.gamma + 1)

    def scaled(self, **kw) -> "Config":
        """A smaller (or otherwise altered) copy with the same drawing recipe."""
        return replace(self, **kw)


CONFIGS = {
    # Tiny reference case; "seed 0" is step 0 of this stream.
    "tiny": Config(name="tiny", index=1, B=4, gamma=8, d=256, V=1024, bias=0.5,
                   temp_slope=0.05, mode="threshold", cutoff=0.3, logit_var=1.0,
                   match="const", match_p=0.7, steps=10),
    # Batch-1 latency case.
    "batch1": Config(name="batch1", index=2, B=1, gamma=16, d=4096, V=151936, bias=0.0,
                     temp_slope=0.03, mode="threshold", cutoff=0.2, logit_var=2.0,
                     match="decay", match_p=0.9, steps=10),
    # Mid batch with per-request cutoffs and per-request logit shifts.
    "mid": Config(name="mid", index=3, B=64, gamma=16, d=4096, V=151936, bias=0.0,
                  temp_slope=0.03, mode="threshold", cutoff_range=(0.1, 0.5),
                  logit_var=2.0, shift="normal", latent=True, match="sigmoid", steps=10),
    # Large batch under a batch-wide budget T = 3B.
    "budget": Config(name="budget", index=4, B=256, gamma=16, d=7168, V=129280, bias=0.0,
                     temp_slope=0.03, mode="budget", budget_per_request=3.0,
                     logit_var=2.0, latent=True, match="sigmoid", steps=10),
    # Mixed traffic, per-request cutoff arm.
    "mixed_threshold": Config(name="mixed_threshold", index=5, B=256, gamma=16, d=4096,
                              V=151936, bias=0.0, temp_slope=0.03, mode="threshold",
                              cutoff=0.25, logit_var=2.0, shift="bimodal",
                              match="bimodal", steps=100),
    # Mixed traffic, batch-budget arm (same seeded inputs as the threshold arm).
    "mixed_budget": Config(name="mixed_budget", index=5, B=256, gamma=16, d=4096,
                           V=151936, bias=0.0, temp_slope=0.03, mode="budget",
                           budget_per_request=2.9, logit_var=2.0, shift="bimodal",
                           match="bimodal", steps=100),
    # The same mixed traffic under the cutoff and the budget together (the same
    # seed stream as the two arms above, so the same batches).
    "mixed_combined": Config(name="mixed_combined", index=5, B=256, gamma=16, d=4096,
                             V=151936, bias=0.0, temp_slope=0.03, mode="combined",
                             cutoff=0.25, budget_per_request=2.9, logit_var=2.0,
                             shift="bimodal", match="bimodal", steps=100),
}


def config_by_name(name: str) -> Config:
    return CONFIGS[name]
