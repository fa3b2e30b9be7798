"""Float64 CPU oracle of the dual-stream MMDiT block core (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use this package; the
HIP product path never imports or calls it and shares no code with it.
"""
from .mmdit_oracle import *  # noqa: F401,F403
from .mmdit_oracle import MOD_ORDER  # noqa: F401
