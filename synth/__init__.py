"""Seeded synthetic inputs shared by the oracle-side tests and the HIP-side tests and bench.

This package holds workload shapes and random-number plumbing only.  It computes none of the
method's results (no mixing, norm, projection, attention, sampling, verification or selection):
the oracle and the HIP library each do that on their own.  Planted verify logits use a row's
largest and smallest value only to construct an input with a known accepted-prefix length.
"""
from .configs import DrafterShape, Workload, WORKLOADS, workload
from .inputs import (
    make_weights, make_block_tokens, make_lengths, make_hidden, make_cache_kv,
    make_drafts, make_planted_verify_logits, make_planted_streak_logits, leading_successes,
    tensor_seed, capacity_for,
)

__all__ = [
    "DrafterShape", "Workload", "WORKLOADS", "workload",
    "make_weights", "make_block_tokens", "make_lengths", "make_hidden", "make_cache_kv",
    "make_drafts", "make_planted_verify_logits", "make_planted_streak_logits",
    "leading_successes", "tensor_seed", "capacity_for",
]
