"""MI355X-native streaming-MoE decode path (int4 expert streaming).

The computation lives in libedge0.so (HIP kernels for gfx950, C ABI in
include/edge0.h); ``edge0`` is its thin binding and ``weights`` uploads
expert arrays into a slot pool through the library's pack call.
"""
