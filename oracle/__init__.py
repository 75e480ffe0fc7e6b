"""fp64 CPU oracle (test infrastructure only; never on the library's path)."""
from . import prism_oracle  # noqa: F401
from .prism_oracle import *  # noqa: F401,F403
