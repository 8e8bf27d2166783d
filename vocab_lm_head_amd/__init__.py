"""MI355X-native vocab-parallel LM head + cross entropy.

The work happens in ``libvplmhead.so`` (hand-written HIP for gfx950, C ABI in
``include/vp_lmhead.h``); this package only builds it (``build``) and binds it
(``_lib``).  Importing the package needs the built library -- there is no CPU
fallback.
"""
from ._lib import (  # noqa: F401
    DEFAULT_IGNORE_INDEX, VPError, alloc_workspace, lib, status_string, vp_ce_combine,
    vp_embed_bwd, vp_embed_bwd_workspace, vp_embed_fwd, vp_lmhead_ce_bwd,
    vp_lmhead_ce_bwd_workspace, vp_lmhead_ce_fwd, vp_lmhead_ce_fwd_workspace, vp_padded_vocab,
    vp_shard_range,
)
# the forward for callers that cannot allocate (fixed per-GPU scratch, no workspace)
from ._lib import NOALLOC_SCRATCH_BYTES, VP_ERR_SCRATCH, vp_lmhead_ce_fwd_noalloc  # noqa: F401
# materialised-logits comparator (beside the fused path, to measure what it saves)
from ._lib import (  # noqa: F401
    logits_ld, vp_ce_max, vp_lmhead_logits, vp_logits_ce_bwd, vp_logits_ce_stats,
)
