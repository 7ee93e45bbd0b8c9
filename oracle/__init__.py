"""CPU oracle of the packed DiT block (test infrastructure).

Plain fp64 numpy written from the pages' definitions.  It is test
infrastructure only: the tests, the package's ``smoke()`` check and the
benchmark's CPU-baseline leg may call it; the HIP library never does and
shares no code with it.
"""

from .dit_oracle import *  # noqa: F401,F403
