"""CPU oracle of the MoE expert-layer path. Test infrastructure only: imported by the
tests, the smoke check and the benchmark's CPU-baseline leg, never by the product."""
from . import moe_oracle  # noqa: F401
