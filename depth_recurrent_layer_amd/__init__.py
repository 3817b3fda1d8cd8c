"""MI355X-native forward pass of one Dreamer depth-recurrent attention-mixture layer.

The work happens in libdreamer.so (HIP kernels for gfx950, C ABI in include/dreamer.h);
``depth_recurrent_layer_amd.dreamer`` is its ctypes binding.  Build the library with
``python -m depth_recurrent_layer_amd.build``.
"""
__all__ = ["dreamer"]
