"""MI355X-native MAC-Attention (Match-Amend-Complete) decode step.

The compute path is the HIP library ``libmac_attention.so`` built from
``csrc/``; ``mac`` is its ctypes binding.  Importing this package loads
nothing; ``attention_reuse_amd.mac`` loads the library on first use and
raises if it is missing.
"""
__all__ = ["mac", "workload"]
