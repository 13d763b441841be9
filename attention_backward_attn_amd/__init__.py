"""MI355X (gfx950) fused attention backward: HIP kernels behind a C ABI.

The compiled library ``libattnbwd.so`` is loaded lazily by
``attention_backward_attn_amd.binding`` on first use; importing the package
itself loads nothing.
"""

__all__ = ["inputs", "binding", "mask", "build"]
