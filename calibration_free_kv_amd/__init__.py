"""libkvq: calibration-free rotate-then-quantize KV-cache compression for MI355X.

The compute path lives in the HIP library ``libkvq.so`` (C ABI declared in
``include/kvq.h``); ``calibration_free_kv_amd.kvq`` is its thin Python binding.
"""
