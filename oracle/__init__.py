"""CPU oracle (test infrastructure only): plain float64 numpy implementation of the method."""
from . import nabla_ref  # noqa: F401
