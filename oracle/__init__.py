"""CPU float64 oracle for the SSD forward and the SSDi8 INT8 path (test infrastructure)."""
from . import ssd_oracle  # noqa: F401
