"""Float64 CPU oracle for the LinearARD attention-relation KL (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import this package.  It shares no code with the HIP library.
"""

from .relkl import (backward, backward_unit, default_scale, forward, forward_unit,  # noqa: F401
                    keep_mask, logits, row_lse)
from . import closed_form  # noqa: F401
from . import cross, rope  # noqa: F401
