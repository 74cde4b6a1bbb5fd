"""MI355X (gfx950) batched speculative-sampling verify step.

The computation lives in libspecverify.so (hand-written HIP kernels behind a
C ABI declared in include/specverify.h); this package is its thin Python
binding plus the seeded synthetic workloads used by the tests and benchmark.
"""

from .binding import (  # noqa: F401
    SpecVerifyError,
    load,
    profile_enable,
    profile_read,
    release,
    verify,
)
