"""MI355X-native Looped Latent Attention (LLA) latent-cache hot path.

The compute lives in a C-ABI HIP library (``liblla.so``, declared in
``include/lla.h``); ``looped_transformer_latent_amd.lla`` is the thin ctypes
binding.  ``gen`` is the seeded input generator shared by tests and bench.
"""
__all__ = ["gen", "lla", "workloads"]
