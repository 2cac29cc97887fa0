"""MI355X-native compressed sparse attention (CSA) forward path.

The compute lives in ``libcsa.so`` (hand-written HIP kernels for gfx950 behind a C ABI,
declared in ``include/csa.h``); ``deepseek_v4_csa_amd.ops`` is the thin ctypes binding
with the same entry-point names, and ``deepseek_v4_csa_amd.inputs`` the seeded
synthetic workloads.  Importing the package loads nothing; ``ops`` loads the library
on first use and raises if it is missing.
"""
__all__ = ["ops", "inputs"]
