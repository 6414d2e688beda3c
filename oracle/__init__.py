"""CPU oracle of the two-level sparse decode operator (test infrastructure only).

Imported only by the test suite, the smoke check and the benchmark's
CPU-baseline leg; the HIP library never uses it."""
from .hsab_oracle import *  # noqa: F401,F403
