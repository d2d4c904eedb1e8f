"""The five synthetic workloads the tests and the benchmark run (shapes only; no arithmetic).

Shapes follow the Windowed-MTP setting (abstract: million-token context, a draft head that takes
k steps, GQA target models, verification of the k+1 draft tokens). The pages fix no values of S,
W, head counts or head_dim for Windowed-MTP; these workloads choose them and the inputs are seeded
synthetic draws (see synth.py) standing in for real prompts, whose effect on the method the pages
call input-invariant.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    context: int           # prefix length L before drafting (per sequence unless ragged)
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str             # "f32" or "bf16"
    sink: int
    window: int
    draft_depth: int       # k
    verify_m: int = 0      # candidates verified (k+1); 0 = no verify leg in this workload
    k_scale: Optional[float] = None  # keys drawn as N(0,1) * k_scale before rounding
    ragged_lo: int = 0     # if > 0: per-sequence L drawn uniformly from [ragged_lo, context]
    decode_steps: int = 1  # decode iterations (each = draft_depth ring appends + draft steps)
    seed: int = 1000


TINY = Workload("tiny-draft-L4096-fp32", batch=1, context=4096, n_q_heads=8, n_kv_heads=2,
                head_dim=64, dtype="f32", sink=4, window=256, draft_depth=1, seed=1001)
MID = Workload("mid-context-L131072-bf16", batch=1, context=131072, n_q_heads=32, n_kv_heads=4,
               head_dim=128, dtype="bf16", sink=4, window=2048, draft_depth=3,
               k_scale=128 ** -0.5, seed=1002)
MILLION = Workload("million-token-draft-L1048576-bf16", batch=1, context=1048576, n_q_heads=32,
                   n_kv_heads=2, head_dim=256, dtype="bf16", sink=4, window=4096, draft_depth=5,
                   seed=1003)
VERIFY = Workload("verify-m4-L1048576-bf16", batch=1, context=1048576, n_q_heads=32,
                  n_kv_heads=2, head_dim=128, dtype="bf16", sink=0, window=0, draft_depth=3,
                  verify_m=4, seed=1004)
BATCHED = Workload("batched-ring-B8-ragged-bf16", batch=8, context=1048576, n_q_heads=16,
                   n_kv_heads=2, head_dim=128, dtype="bf16", sink=4, window=2048, draft_depth=4,
                   ragged_lo=65536, decode_steps=10000, seed=1005)

ALL = (TINY, MID, MILLION, VERIFY, BATCHED)
