"""Float64 CPU oracle for the SAF hybrid attention layer -- TEST INFRASTRUCTURE.

This package is a plain, slow, dense implementation of what the layer
computes, written from "When Can Attention Heads Be Statically Defined?"
(Section 3, Section 3.2 Equation 3, Appendix A.1 Equations 5-7, Appendix D.2,
and the trainable-pattern gradients of Appendix C.3.2), and of fitting a
compact pattern to a calibration mean (``saf_fit_oracle``: Algorithm 1,
Section 3.2 "Fitting" Equation 4, Appendix A.2, Appendix D.1 Equation 20),
and of the calibration statistics (``saf_calib_oracle``: Section 3.1,
Equations 1 and 2).
It exists only to check the HIP library.  Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the library and its Python binding never do, and nothing here
imports them.

Every function is pinned by a CPU test to something other than itself
(closed forms, a hand-worked example, library routines, finite differences).
"""

from . import saf_calib_oracle, saf_fit_oracle
from .saf_oracle import (
    frozen_head_bwd,
    frozen_head_fwd,
    frozen_head_pattern_grad,
    frozen_logits,
    frozen_lognorm,
    frozen_pattern,
    frozen_rows_fwd,
    frozen_rows_pattern_grad,
    hybrid_bwd,
    hybrid_fwd,
    hybrid_pattern_grad,
    ordinary_head_bwd,
    ordinary_head_fwd,
    ordinary_rows_fwd,
    default_scale,
)

__all__ = [
    "saf_calib_oracle",
    "saf_fit_oracle",
    "frozen_head_bwd",
    "frozen_head_fwd",
    "frozen_head_pattern_grad",
    "frozen_logits",
    "frozen_lognorm",
    "frozen_pattern",
    "frozen_rows_fwd",
    "frozen_rows_pattern_grad",
    "hybrid_bwd",
    "hybrid_fwd",
    "hybrid_pattern_grad",
    "ordinary_head_bwd",
    "ordinary_head_fwd",
    "ordinary_rows_fwd",
    "default_scale",
]
