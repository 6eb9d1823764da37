"""The verification workloads: five dense ones and one with shared rows.

Shapes follow the pages' settings: Qwen2.5-scale vocabularies and bf16 verifier
logits (SpecDiff-2 appendix B.1), windows of gamma = 16 and 32 tokens (appendix
A.3), K = 8 drafts (section 7.3), temperatures 1.0 and below (section 7.3,
appendix A.1).  The vocabulary size 152064 and the noise levels are synthetic
choices of this workload suite; no dataset is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int            # prefixes
    K: int            # drafts per prefix
    gamma: int        # drafted positions per draft
    V: int            # vocabulary
    dtype: str        # "f32" or "bf16"
    sigma0: float     # drafter noise at position 0
    sigma_step: float  # drafter noise added per position (sigma_j = sigma0 + sigma_step * j)
    temp: float       # temperature applied to both p and q
    boost: float      # logit added to the row's mode token
    boost_prob: float  # share of rows that receive the boost
    trials: int = 0   # distribution-check trials (tiny workload only)
    layout: str = "dense"  # "dense" rows per (prefix, draft), or "pooled" shared rows
    tau: float = 0.0  # pooled: verifier-row spread between draft prefixes at one position
    notes: str = field(default="", compare=False)

    @property
    def data_seed(self) -> int:
        return 20261202 + self.cid

    @property
    def seed(self) -> int:
        return 1 + self.cid

    @property
    def row_pairs(self) -> int:
        return self.B * self.K * self.gamma

    def scored_bytes(self) -> int:
        """Logit bytes of the scored row pairs (p row j and q row j, j < gamma)."""
        es = 4 if self.dtype == "f32" else 2
        return self.row_pairs * 2 * self.V * es


CONFIGS = {
    1: Config(1, "tiny", B=1, K=1, gamma=4, V=32, dtype="f32", sigma0=1.0, sigma_step=0.0,
              temp=1.0, boost=6.0, boost_prob=1.0, trials=1_000_000,
              notes="distribution check; fp32 logits"),
    2: Config(2, "single_stream", B=1, K=1, gamma=8, V=152064, dtype="bf16", sigma0=1.0,
              sigma_step=0.0, temp=1.0, boost=8.0, boost_prob=1.0),
    3: Config(3, "self_selection", B=16, K=8, gamma=16, V=152064, dtype="bf16", sigma0=1.5,
              sigma_step=0.0, temp=1.0, boost=8.0, boost_prob=1.0),
    4: Config(4, "batched_serving", B=256, K=1, gamma=8, V=152064, dtype="bf16", sigma0=0.75,
              sigma_step=0.0, temp=0.7, boost=8.0, boost_prob=1.0),
    5: Config(5, "long_window", B=64, K=16, gamma=32, V=152064, dtype="bf16", sigma0=0.5,
              sigma_step=0.05, temp=0.7, boost=8.0, boost_prob=0.7),
    6: Config(6, "shared_marginal", B=16, K=8, gamma=16, V=152064, dtype="bf16", sigma0=1.5,
              sigma_step=0.0, temp=1.0, boost=8.0, boost_prob=1.0, layout="pooled", tau=0.5,
              notes="the K drafts sampled from one set of drafter marginals (shared q rows); "
                    "one verifier row per distinct draft prefix"),
}


def get_config(c) -> Config:
    if isinstance(c, Config):
        return c
    if isinstance(c, str):
        for cfg in CONFIGS.values():
            if cfg.name == c or str(cfg.cid) == c:
                return cfg
        raise KeyError(c)
    return CONFIGS[int(c)]
