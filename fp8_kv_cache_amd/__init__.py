"""MI355X-native fused q/kv RMSNorm + RoPE + FP8 (E4M3, UE8M0) quantize +
paged KV-cache insert.

The operator lives in the HIP library ``libqkv_prep.so`` (C ABI declared in
``include/qkv_prep.h``); ``fp8_kv_cache_amd.qkv_prep`` is its Python binding
and ``fp8_kv_cache_amd.workloads`` draws seeded synthetic inputs.  Build the
library with ``python -m fp8_kv_cache_amd.build``."""
