"""MI355X-native hot path of confidence-scheduled speculative decoding.

The compute lives in libsdv.so (HIP for gfx950, C ABI in include/sdv.h);
this package is its thin Python binding.
"""

from ._lib import (  # noqa: F401
    EXPORTS,
    SdvError,
    lib,
    sd_abi_version,
    sd_status_string,
    sd_schedule,
    sd_schedule_workspace_size,
    sd_verify,
    sd_verify_workspace_size,
    sd_verify_noalloc,
    sd_markov_draft,
    sd_markov_draft_workspace_size,
    sd_rnn_draft,
    sd_rnn_draft_workspace_size,
    sd_uniforms,
    sd_lightspec_update,
    sd_lightspec_plan,
    SD_SCHED_EARLY_STOP,
    SD_SCHED_GLOBAL_ARGMAX,
    SD_SCHED_CAPPED_TOPK,
    SD_SCHED_THRESHOLD,
    SD_VERIFY_STOP_AT_REJECTION,
    SD_ST_BAD_TOKEN,
    SD_ST_NONFINITE,
    SD_ST_ZERO_Z,
    SD_ST_ZERO_RESIDUAL,
    SD_ST_ZERO_Q,
)
