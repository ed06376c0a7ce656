"""CPU oracle of the MAC-Attention decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it, and it
imports nothing from the GPU package.
"""
from .oracle import (  # noqa: F401
    EMPTY_LSE,
    full_decode,
    load,
    merge,
    run_stream,
    run_streams,
    summary,
    threshold2,
    unmerge,
)
