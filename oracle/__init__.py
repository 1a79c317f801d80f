"""CPU oracle of the MoE expert layer (test infrastructure only).

Imported by the tests, by the build entry's smoke check and by the bench's
CPU-baseline leg; never by the product path.
"""
from . import moe_oracle  # noqa: F401
