"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 NumPy statement of what the paged KV cache and its decode
attention compute.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it.  It shares no code with the HIP
library (``paged_kv_cache_212_amd``) and never imports it.

Sources (the four PagedAttention web pages; sections named by their headings):

* page 1, jisaku.com glossary "PagedAttention（ページドアテンション）",
  sections 「PagedAttentionの解決策」 (fixed-size blocks, block table, the
  100-token example) and 「コピーオンライト（Copy-on-Write）共有」;
* page 2, hubblespacetelescope blog on vLLM/PagedAttention, section
  「OSの知恵をGPUへ：「PagedAttention」の革新的ブレークスルー」 (one block per 16
  filled tokens, slack only in the last block, sharing by reference count);
* page 3, abeam.tech review of "Efficient Memory Management for Large Language
  Model Serving with PagedAttention", sections 「用語解説」,
  「モデル構造ではなくサービング基盤の変更」, 「KV キャッシュマネージャ」,
  「並列サンプリングやビームサーチでの共有」 and 「よくある質問」;
* page 4, pro-knowledge-base glossary, FAQ (results are unchanged by paging).

The attention formula softmax(q·Kᵀ/√d)·V is standard decode self-attention
over the cached keys and values; the pages state that paging leaves the result
of attention unchanged, so the oracle is that plain definition evaluated over
the K/V reassembled through the block table.

``prefill_ref`` (oracle/prefill.py) extends the decode step to a chunk of
query tokens per sequence attending causally over the paged cache (prefill,
chunked prefill); with one token per sequence it is the decode step.

``quantize_ref`` (oracle/quant.py) encodes K/V rows into the 8-bit codes of a
quantized cache (INT8, as page 1 pairs with paging in section
「他のKVキャッシュ最適化との組み合わせ」, and FP8 E4M3); ``decode_ref`` then
attends over code * scale.

Pinning: every function here is pinned by ``tests/test_oracle*.py`` against
values not produced by the oracle itself (brute force over the unpaged token
rows, torch's scaled_dot_product_attention in fp64, closed forms, a worked
example from page 1, hand-enumerated layout offsets, invariances).  No function
is "parity unpinned".
"""
from .numerics import bits_of, to_f64  # noqa: F401
from .allocator import AllocatorModel, AllocError  # noqa: F401
from .cache import (new_pools, append_ref, copy_ref, gather_ref, k_offset,  # noqa: F401
                    v_offset)
from .attention import decode_ref, dense_ref, partitioned_ref, merge_partials  # noqa: F401
from .prefill import prefill_ref  # noqa: F401
from .quant import quantize_ref, dequantize_ref  # noqa: F401
from .run import run_case, oracle_sequence_out  # noqa: F401
