"""fp64 CPU oracle of the RAT+ operator -- test infrastructure only.

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path never does.
"""
from .rat_oracle import (  # noqa: F401
    DecodeCache, attend, default_scale, gates, key_set, pairs, prefill, scan,
)
from . import topk_oracle  # noqa: F401,E402
from . import local_oracle  # noqa: F401,E402
