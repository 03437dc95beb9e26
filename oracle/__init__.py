"""fp64 CPU oracle of the WHALE attention-fusion module.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP package."""
from . import whale_oracle  # noqa: F401
