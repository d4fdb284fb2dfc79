"""MI355X-native lossless KV-cache entropy coder (speculative KV coding).

``entropy_coding_amd.kvc`` is the thin ctypes binding over ``libkvc.so``
(HIP for gfx950, C ABI declared in ``include/kvc.h``); importing it loads the
library and fails loudly if it has not been built.  ``workloads`` holds the
seeded synthetic inputs.
"""

__all__ = ["kvc", "workloads"]
