"""Seeded synthetic inputs for the hot path (no method arithmetic lives here).

Both the CPU reference and the GPU library are fed from these generators; they
only draw random tensors of the shapes and distributions the workloads call
for.  See ``synth`` for the recipes.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    sps_table,
    verify_inputs,
    verify_config,
    markov_config,
    markov_inputs,
    markov_targets,
    rnn_config,
    rnn_inputs,
)
