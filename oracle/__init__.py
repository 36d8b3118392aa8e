"""CPU oracle for paged chunk attention. TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may
import or run anything in this package. The HIP library never calls it, and it
shares no code, table or helper with the HIP library.
"""
from .oomb_oracle import *  # noqa: F401,F403
