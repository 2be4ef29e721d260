"""LinearARD attention-relation KL on MI355X (gfx950): HIP kernels behind a C-ABI.

The HIP library (liblard.so) is loaded lazily on first use; nothing here computes on the
CPU.  See include/lard.h for the C ABI.
"""

from .relkl import (LardError, load_library, library_path, relation_kl, relkl_bwd,  # noqa: F401
                    relkl_fwd, workspace_size)
