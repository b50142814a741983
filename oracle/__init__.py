"""fp64 CPU oracle for KDA (test infrastructure only; never imported by the product path)."""
from .kda_ref import (c_decode_step, c_forward, decode_step, load_c, recurrence,  # noqa: F401
                      rel_l2, token_step)
