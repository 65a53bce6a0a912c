"""CPU oracle (test infrastructure; see kvd_oracle's header)."""
from .kvd_oracle import (  # noqa: F401
    ConcatCache, accept, apply_suppression, argmax_rows, attend, attend_cross, attend_self,
    attend_self_ragged, beam_select,
    decode_step, full_causal_attention, log_softmax_rows, narrow, reorder, rope, rope_theta, verify_accept,
    verify_accept_masked, widen,
)
