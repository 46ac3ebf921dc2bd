"""fp64 CPU oracle of the fine-grained MoE layer -- test infrastructure only.

Imported by the tests, the entry script's smoke check and the benchmark's CPU
baseline leg; never by the product path.
"""
from . import moe_oracle  # noqa: F401
