"""Seeded synthetic inputs for tree verification.

This package only draws random numbers and lays them out in the buffers the
verification pass reads (queries, paged K/V, block tables, draft trees,
target logits, draft probabilities, uniforms).  It performs none of the
verification arithmetic itself: no attention, no acceptance decisions, no
commit, no block selection.  Both the CPU oracle tests and the GPU path read
the same bytes from here.
"""
from .configs import CONFIGS, Config, small_variant  # noqa: F401
from .inputs import make_inputs, Inputs  # noqa: F401
