"""MI355X-native MoE expert-parallel dispatch and combine.

``combine_epx_get_amd.epx`` is the thin ctypes binding over the HIP library
(``libepx.so``, C ABI declared in ``include/epx.h``); importing it fails when
the library has not been built. ``combine_epx_get_amd.workloads`` draws the
seeded synthetic inputs.
"""
