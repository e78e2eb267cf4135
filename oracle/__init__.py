"""CPU oracle for KV-cache transform coding (test infrastructure only).

Only the tests, the package's smoke entry and the benchmark's CPU-baseline leg
may import this package.  The product library never calls it.

See kvtc_oracle for the method and the readings taken where the pages are
silent.
"""
from .kvtc_oracle import *  # noqa: F401,F403
