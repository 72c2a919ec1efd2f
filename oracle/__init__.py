"""Float64 CPU oracle for paged flash-decode attention over an E4M3 (or
NVFP4 or MXFP8) KV cache, and for the writers that fill those caches from bf16 keys
and values.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this package; only the tests, the smoke check and the CPU-baseline leg
of the benchmark do.  It shares no code with the HIP library: it decodes
E4M3 bit by bit, gathers pages with plain indexing and evaluates the softmax
from its definition, in float64, with no blocking, fusion or online
rescaling.

Every function is pinned by the `-m "not gpu"` tests in tests/test_oracle.py
(library routines, closed forms, invariants and a brute-force twin).  No
function here is "parity unpinned".
"""

from .fp8pa_ref import (  # noqa: F401
    E4M3_TABLE,
    e4m3_decode_code,
    bf16_bits_to_f64,
    attended_range,
    k_scale_of_head,
    decode,
    merge,
)
from .fp8pa_write_ref import (  # noqa: F401
    E4M3_MAX,
    e4m3_encode,
    cache_write,
)
from .nvfp4_ref import (  # noqa: F401
    E2M1_TABLE,
    e2m1_decode_code,
    e2m1_encode,
    nvfp4_side_bytes,
    nvfp4_gather,
    nvfp4_cache_write,
)
from .mxfp8_ref import (  # noqa: F401
    e8m0_decode,
    mxfp8_side_bytes,
    mxfp8_gather,
    mxfp8_cache_write,
)
