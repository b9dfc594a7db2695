"""CPU oracle of the MoE FFN layer (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  It shares no code with the GPU path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import Mat, Result, block_forward, moe_forward, residual_add, rmsnorm  # noqa: F401
