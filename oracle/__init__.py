"""fp64 CPU oracle for fused QK-RMSNorm + 3D M-RoPE joint text+image attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this
package: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP library and imports nothing from it.

Two independent implementations of the same definition live here:

* ``reference``  -- vectorised NumPy in float64 (the oracle proper);
* ``brute``      -- plain Python loops over scalars (tiny inputs only).

Every function cites the passage of the source pages it follows. The pages
are: the Ideogram 4.0 announcement thread (digg.com repost), the Korean
"Ideogram 4 deep dive" article, the unsloth commit log for the Ideogram 4
diffusion backend, and the SimpleTuner Ideogram 4 quickstart.
"""

from .reference import (  # noqa: F401
    axis_of_pair,
    inv_freq,
    rms_norm,
    mrope,
    valid_tokens,
    attention,
    oracle_fwd,
)
from . import brute  # noqa: F401
