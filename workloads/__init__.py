"""Seeded synthetic inputs for one round of tree-structured verification.

This package only draws random numbers and lays them out in the shapes the
round consumes.  It performs none of the method's own arithmetic (no top-k,
no tree selection, no attention, no argmax walk, no commit), so that both the
GPU path and the CPU oracle can take their inputs from it.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    EXPAND_CONFIGS,
    Config,
    Cost,
    ExpandConfig,
    attention_inputs,
    pitched,
    config,
    drafter_logits,
    expand_config,
    marginals,
    node_distributions,
    prefix_lengths,
    target_logits,
)
