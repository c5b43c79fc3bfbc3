"""R-KV decode-time KV-cache compression step for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in librkv.so behind the C ABI of
include/rkv.h; `binding` mirrors that ABI function by function and `RKVStep`
runs the three calls on torch device tensors.
"""
from . import binding  # noqa: F401
from .binding import (RkvError, make_cache, make_config, rkv_compact, rkv_is_triggered,  # noqa: F401
                      rkv_last_error, rkv_score, rkv_select, rkv_status_string, rkv_step,
                      rkv_workspace_size)
from .step import RKVStep  # noqa: F401
