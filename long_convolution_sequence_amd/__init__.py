"""MI355X-native exact autoregressive long convolution (Flash Inference hot path).

The compute path is the HIP library ``libfi.so`` behind the C-ABI declared in
``include/fi.h``; ``long_convolution_sequence_amd.fi`` is its thin ctypes
binding.  ``workloads`` holds the seeded synthetic inputs.
"""
