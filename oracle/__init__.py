"""CPU oracle for the dots.llm1 fine-grained MoE FFN layer.

TEST INFRASTRUCTURE: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import it.  The HIP library never calls it.
"""
from . import moe_oracle  # noqa: F401
