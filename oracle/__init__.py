"""Test-only fp64 CPU oracle (see aaac_ref). Imported by tests, the smoke check and the bench's
CPU-baseline leg; never by the HIP package."""
from . import aaac_ref  # noqa: F401
