"""Seeded synthetic workloads for the grouped-query attention library.

This package is the only code shared between the CPU oracle side (tests,
CPU baseline) and the GPU side (parity tests, benchmark): it draws seeded
random numbers, casts them to storage dtypes and builds quantized caches.
It holds none of the attention arithmetic.
"""

from .configs import CONFIGS, Workload, by_name  # noqa: F401
from .gen import (  # noqa: F401
    normal,
    q4_encode,
    q4_pack_codes,
    request_lengths,
    seed_sequence,
)
