"""fp64 CPU oracle (test infrastructure only; see oracle/palu.py)."""
from .palu import *  # noqa: F401,F403
from .palu import __all__  # noqa: F401
