"""float64 CPU oracle of the KDA recurrence -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library and its Python binding never do.
"""

from .kda_oracle import Oracle, default, gate_log_decay, kda_decode_step, kda_fwd, output_gate  # noqa: F401
