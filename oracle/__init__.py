"""CPU oracle for the FSDP data-parallel hot path (test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the library)."""
from .fsdp_oracle import *  # noqa: F401,F403
from .fsdp_oracle import Plan, plan_layout  # noqa: F401
