"""CPU oracle (test infrastructure only; see fp8_oracle's header)."""
from .fp8_oracle import *  # noqa: F401,F403
from .fp8_oracle import (E4M3_MAX, TILE, OP_N, OP_T, BSCALE_BLOCK128, BSCALE_ROW128)  # noqa: F401
