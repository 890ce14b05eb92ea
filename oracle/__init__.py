"""fp64 CPU oracle (test infrastructure; never imported by the product path)."""
from .oracle import *  # noqa: F401,F403
from .oracle import __all__  # noqa: F401
