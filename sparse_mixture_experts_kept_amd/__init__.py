"""MI355X-native (gfx950) Mixtral sparse mixture-of-experts feed-forward layer.

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/moe.h``); ``sparse_mixture_experts_kept_amd.moe`` is the
thin ctypes binding.  Importing this package does not load the library; the
binding loads it on first use and raises if it has not been built.
"""
