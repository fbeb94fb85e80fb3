"""CPU oracle for the SALA hybrid attention hot path (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package; the product path never does. See ``sala_oracle`` for the definitions.
"""

from .sala_oracle import *  # noqa: F401,F403
from .sala_oracle import __all__  # noqa: F401
