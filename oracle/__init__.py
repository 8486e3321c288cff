"""CPU oracle for the local MoE FFN forward (test infrastructure only; see
moe_oracle's header). Importable only by tests, the smoke check and the
benchmark's CPU-baseline leg."""
from . import moe_oracle  # noqa: F401
