"""fp64 CPU oracle for KDA (test infrastructure only; never imported by the product path)."""
from .kda_ref import (c_decode_step, c_forward, c_prologue_forward, decode_step, load_c,  # noqa: F401
                      prologue, recurrence, rel_l2, token_step)
