"""Seeded synthetic workloads for tree verification.

This package builds inputs only: bf16 query/key/value tensors, draft trees given as
``parent[]`` arrays, vocabulary logits and draft tokens. It holds none of the
verification arithmetic (no attention, no argmax, no acceptance walk). Both the CPU
oracle tests and the HIP path consume the same arrays from here.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    SEED_ROOT,
    Workload,
    accept_trial,
    bf16_bits_from_f32,
    chain_parent,
    kary_bfs_parent,
    make,
    random_tree_parent,
    rng_for,
    tie_rows,
)
