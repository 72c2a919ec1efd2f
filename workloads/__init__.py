"""Seeded synthetic inputs for paged FP8 decode attention.

Shared by the tests, the smoke check and the benchmark.  This package holds
no attention arithmetic: it only draws random numbers, encodes them into the
input formats (bf16 queries, E4M3 cache codes) and lays out pages.
"""

from .gen import Workload, make_workload, make_config, make_nvfp4_workload, make_mxfp8_workload, CONFIGS, POISON_CODE  # noqa: F401
