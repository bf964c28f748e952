"""kvq: mixed-precision quantized KV cache and decode attention for MI355X (gfx950).

The library proper is ``libkvq.so`` (HIP, C ABI in ``include/kvq.h``); ``kvq`` is its thin Python binding.
Import ``quantized_decode_attention_append_amd.kvq`` to use it (it raises if the library is not built).
"""
