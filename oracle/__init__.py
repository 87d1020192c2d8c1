"""fp64 CPU oracle of the SFI decode path.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU
baseline leg, never by the device path.
"""
from . import sfi_oracle  # noqa: F401
