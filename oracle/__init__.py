"""CPU oracle of the batched verify step of lossless speculative decoding.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow reference the GPU library is
checked against. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import, call or execute anything in it; the product path (the HIP library and its Python
binding) never does, and shares no code, headers, tables or helpers with it.

Every function follows the pages' statement of the method (mlx-dspark release notes and
changelog) or the plain mathematical definition; each module header cites its passages.
Pins: tests/test_oracle_*.py check these functions against closed forms, hand cases,
library routines (torch CPU attention, rocRAND's Philox) and chi-square losslessness.
"""
from . import attention, philox, sampling  # noqa: F401
from .attention import verify_attention  # noqa: F401
from .sampling import RowParams, verify_sample_accept, sample_proposals  # noqa: F401
