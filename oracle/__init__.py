"""Plain CPU oracle of the RNS-CKKS hot path (test infrastructure only)."""
from .oracle import *  # noqa: F401,F403
from .oracle import Ctx, build, lib  # noqa: F401
