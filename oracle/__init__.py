"""CPU oracle for the quantized KV cache and its decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The product path
(the HIP library and its Python binding) never calls it, and the two share no
code: no kernels, headers, helpers, tables or constant generators.

What it computes, and where the pages fix it (pages cited by title and passage):

* ``quant``     - the symmetric qN_0 block quantizer (32 values, one fp16 scale,
                  no offset; "BeeLlama.cpp v0.4.1" page, list of standard KV cache
                  types q2_0..q8_0) and the KVarN per-channel variance
                  normalization ("KV cache quant benchmarks: KVarN ..." page, TL;DR;
                  BeeLlama.cpp v0.4.1 page, KVarN paragraph).
* ``layout``    - the byte layout of the cache arena and its exact size per bit
                  width and tail length (BeeLlama.cpp v0.4.1 page, KV MiB table;
                  KVarN benchmark page, cache-size column; offload page, byte
                  arithmetic of a QSA layer).
* ``cache``     - the cache state machine: qN_0 body, bf16 precision tail or
                  8-bit recent-token ring, requantization of tokens leaving the
                  window ("Hard numbers on Qwen3.8-27B's KV cache" page, KV
                  low-bit section and the comment on two KV paths per layer).
* ``attention`` - exact softmax attention over the dequantized values in fp64,
                  dense over all positions and sparse over an indexer budget of
                  positions (offload page, QSA paragraph).
* ``indexer``   - the QSA indexer: pooled index keys, their scores against an
                  index query and the choice of a budget of positions (offload
                  page, QSA paragraph).
* ``sizes``     - algorithmic bytes of a decode call (rows read, query read, output written).

Where the pages are silent the functions state the reading they take. The quantizer emulates fp32 arithmetic exactly (numpy
float32 operations are IEEE round-to-nearest-even, with no contraction), and
attention is evaluated in fp64.
"""
from .quant import (quantize_blocks, dequantize_blocks, kvarn_sigma, f16_rne, QMAX)  # noqa: F401
from .layout import (planes, cache_bytes, slab_layout, pack_k_rows, pack_v_tiles,  # noqa: F401
                     pack_bf16_v_tiles, unpack_k_rows, unpack_v_tiles, pack_k_tiles, unpack_k_tiles,
                     pack_bf16_k_tiles, unpack_bf16_k_tiles)
from .cache import OracleCache  # noqa: F401
from . import indexer  # noqa: F401
from .attention import attend, decode_reference, sparse_reference, multi_query_reference, prefill_reference  # noqa: F401
from .sizes import (decode_bytes, decode_kv_bytes, query_out_bytes, sparse_bytes, sparse_kv_bytes,  # noqa: F401
                    row_bytes, kv_token_bytes, ring_token_bytes)
