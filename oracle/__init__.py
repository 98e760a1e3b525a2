"""fp64 CPU oracle for GSA (test infrastructure only; see gsa_oracle.py)."""
from .gsa_oracle import *  # noqa: F401,F403
from .gsa_oracle import __all__  # noqa: F401
