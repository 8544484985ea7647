"""MI355X (gfx950) paged KV cache: host block manager, HIP append / copy /
decode kernels behind a C ABI (include/pa.h), and a thin Python binding."""
from ._lib import PAError, lib, LIB_PATH  # noqa: F401
from .block_manager import BlockManager  # noqa: F401
from .cache import PagedKVCache, StepPlan  # noqa: F401
from . import ops  # noqa: F401

__all__ = ["PAError", "BlockManager", "PagedKVCache", "StepPlan", "ops", "lib", "LIB_PATH"]
