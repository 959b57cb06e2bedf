"""fp64 CPU oracle for the KLA operator.

TEST INFRASTRUCTURE ONLY: imported by the test-suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP kernels or their binding.
"""

from .kla_oracle import (gdn_decode_step, gdn_forward, gdn_recurrence, kla_decode_step, kla_forward,
                         kla_recurrence)
from .kla_chunk_oracle import kla_chunkwise
from .kla_backward_oracle import gdn_backward, kla_backward
from .pgdn_oracle import (GAIN_GIVEN, GAIN_KACZMARZ, pgdn_chunkwise, pgdn_decode_step, pgdn_forward,
                          pgdn_preconditioner, pgdn_recurrence)

__all__ = ["kla_recurrence", "kla_forward", "kla_decode_step", "kla_chunkwise", "gdn_recurrence",
           "gdn_forward", "gdn_decode_step", "kla_backward", "gdn_backward", "GAIN_GIVEN", "GAIN_KACZMARZ",
           "pgdn_recurrence", "pgdn_forward", "pgdn_decode_step", "pgdn_chunkwise", "pgdn_preconditioner"]
