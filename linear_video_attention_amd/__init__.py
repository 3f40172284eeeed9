"""MI355X (gfx950) forward pass of the Video DeltaNet hybrid video-video attention layer.

The layer runs in hand-written HIP kernels behind the C ABI of ``include/vdn.h``; this package
holds those sources (``csrc/``), their in-tree build (``build.py``) and a thin ctypes binding
(``vdn.py``) with the ABI's names.
"""

from .vdn import (Plan, VdnError, lib, vdn_forward, vdn_key_ranges, vdn_plan_create,  # noqa: F401
                  vdn_plan_destroy, vdn_scan_frames)
