"""CPU oracle of the FlashMap drafting step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.
"""
from .flashmap_ref import *  # noqa: F401,F403
from . import sampling_ref as sampling  # noqa: F401,E402
