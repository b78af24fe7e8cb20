"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .oracle import *  # noqa: F401,F403
from .oracle import build, lib  # noqa: F401
