"""Seeded synthetic inputs for paged MQA logits (shared by tests and bench).

This package produces input bytes only: context lengths, block tables, paged
K caches, queries and head weights.  It contains none of the scoring
arithmetic, so the oracle and the HIP path can both consume it without
sharing any of the method's code.
"""
from .synth import (CONFIGS, WorkloadConfig, draw_context_lens, make_fp4,
                    make_fp8, make_workload)

__all__ = ["CONFIGS", "WorkloadConfig", "draw_context_lens", "make_fp8",
           "make_fp4", "make_workload"]
