"""CPU float64 oracle (test infrastructure only; see ``oracle.ref``)."""
from .ref import *  # noqa: F401,F403
