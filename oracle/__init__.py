"""fp64 CPU attention oracle — TEST INFRASTRUCTURE ONLY.

Importable only from the tests, the smoke check and the benchmark's CPU
baseline.  The GPU library must never depend on it.
"""
from .oracle import (attention, attention_gqa, attention_rows, build, gqa_kv_index, load,  # noqa: F401
                     num_threads)
from .bwd_oracle import attention_bwd  # noqa: F401
from .kvcache_oracle import attention_kvcache  # noqa: F401
from . import quant_oracle  # noqa: F401
