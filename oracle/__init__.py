"""CPU oracle for the AutoFP block-scaled low-bit linear layer.

TEST INFRASTRUCTURE. This package is the slow, plain reference that the HIP
library is checked against. Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. The HIP library does
not import, link or call it, and the two share no code, tables or constants.

Source of every rule: "AutoEMatic: Runtime-Adaptive Mixed-Precision LLM
Inference via Automatic Exponent-Mantissa Refinement" (arXiv 2611.10165v1).
Each function cites the section, equation, table or figure it follows.
"""

from .autofp_ref import *  # noqa: F401,F403
from .kv_ref import *  # noqa: F401,F403
from . import formats_ref  # noqa: F401  (AutoFP8, exponent-scaled offsets, FP6g)
from . import gptq_ref  # noqa: F401  (refinement-aware GPTQ calibration, App. E)
