"""MI355X-native MoE layer hot path: router top-k, row-wise dispatch, grouped
SwiGLU expert GEMMs (BF16 and MXFP8), weighted combine; forward and backward.

The compute lives in libmoe.so (hand-written HIP for gfx950, C ABI in
include/moe.h).  ``binding`` wraps the C calls, ``layer`` composes one layer
step from them, ``workloads`` makes the seeded synthetic inputs.
"""
