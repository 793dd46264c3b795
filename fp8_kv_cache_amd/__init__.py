"""MI355X-native fused q/kv RMSNorm + RoPE + FP8 (E4M3, UE8M0) quantize +
paged KV-cache insert, with its cache reader and an MXFP8 norm-quant operator
on the same codec.

The operators live in the HIP library ``libqkv_prep.so`` (C ABI declared in
``include/qkv_prep.h`` and ``include/qkv_prep_mxfp8.h``);
``fp8_kv_cache_amd.qkv_prep`` is its Python binding.  Bandwidth-ceiling and
number-format probes live apart in ``libqkv_prep_probe.so``
(``include/qkv_prep_probe.h``, binding ``fp8_kv_cache_amd.probe``).
``fp8_kv_cache_amd.workloads`` draws seeded synthetic inputs.  Build both
libraries with ``python -m fp8_kv_cache_amd.build``."""
