"""VideoNSA attention layer forward for MI355X (gfx950): hand-written HIP
kernels behind a C-ABI library (``libnsa.so``), with a thin ctypes binding.

The binding is loaded lazily so that ``inputs`` (the seeded generator) can be
imported without the GPU library."""

__all__ = ["inputs", "binding"]
