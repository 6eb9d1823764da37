"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This package only generates inputs (logits and drafted tokens).  It holds none of
the verification arithmetic: neither the oracle nor the HIP library imports it,
and it imports neither of them.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .synth import generate, generate_pooled, tiny_trial_drafts, to_host  # noqa: F401
