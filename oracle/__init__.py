"""fp64 CPU oracle for KDA (test infrastructure only; never imported by the product path)."""
from .kda_ref import (c_backward, c_decode_step, c_forward, c_prologue_forward, c_short_conv,  # noqa: F401
                      c_short_conv_step, decode_step, load_c, prologue, prologue_backward, recurrence, recurrence_backward, rel_l2, short_conv, short_conv_backward,
                      token_step)
