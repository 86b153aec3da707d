"""Plain, slow CPU oracle for paged-attention decode.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its Python binding) never imports, links or calls it, and this
package imports nothing from the product path.

What it computes, in float64 with NumPy, written from the pages' statement of
the method:

* ``paged_attention_decode``: every running sequence has one query token per
  head; it attends over its K/V, which sit in fixed-size physical blocks reached
  through a per-sequence block table.  Sources: "vLLM-v0.17.1技术解析：
  PagedAttention内存管理与显存优化技巧" §2.2 (blocks, block table, physical
  block pool); "在A10G上榨干LLaMA-7B：vLLM与PagedAttention实战" §2.1 (logical
  to physical blocks, mapping invisible to the model).
* ``reshape_and_cache``: the new tokens' K/V go to the cache slots named by an
  int32 slot mapping.  Source: the l189.com article on KV cache and
  PagedAttention (www.l189.com/news/180929) §2.2.
* ``copy_blocks``: copy-on-write of shared blocks.  Source: "在A10G上榨干
  LLaMA-7B" §2.2.
* ``gather_kv``: the block gather on its own, the first step of the decode.
* ``swap_blocks``: whole blocks moved between the GPU pools and a swap
  space in host memory.  Sources: "vLLM-v0.17.1技术解析" §4.1 (the
  swap-space flag) and "在A10G上榨干LLaMA-7B" §5.2.
* ``paged_attention_prefill``: several new tokens per sequence (a prompt, or
  the part of a prompt past a cached shared prefix) attend causally over the
  paged cache.  Sources: "在A10G上榨干LLaMA-7B" §2.1 step 1 and §2.2 (a
  prompt's K/V are stored block by block, then used; shared prompt blocks),
  "vLLM-v0.17.1技术解析" §3.2 (attention computed by a fused kernel).

* ``checks.step_input_violations``: which well-formedness conditions a
  step's block tables, context lengths, slot mapping and copy pairs break,
  as a bit mask.  Sources: "vLLM-v0.17.1技术解析" §2.2, "在A10G上榨干
  LLaMA-7B" §2.1 and §2.2, the l189.com article §2.2.

Numeric formats (fp16, bf16, OCP fp8 E4M3FN, INT8) are decoded and encoded in
``oracle.codecs`` from their published bit-level definitions.  The 8-bit
formats carry fp32 scales, one per pool or one per head (``head_scales``).

Parity status: every function here is pinned by CPU tests against brute force,
closed forms, library special cases and the pages' worked examples; none is
"parity unpinned".
"""

from . import checks
from .codecs import (
    DTYPES,
    SCALED,
    bits_dtype,
    decode,
    e4m3_decode,
    e4m3_encode,
    f32_div_rn,
    i8_decode,
    i8_encode,
)
from .paged import (
    copy_blocks,
    gather_kv,
    paged_attention_decode,
    paged_attention_decode_seq,
    paged_attention_prefill,
    paged_attention_prefill_seq,
    head_scales,
    reshape_and_cache,
    swap_blocks,
)

__all__ = [
    "DTYPES",
    "SCALED",
    "i8_decode",
    "i8_encode",
    "bits_dtype",
    "decode",
    "e4m3_decode",
    "e4m3_encode",
    "f32_div_rn",
    "copy_blocks",
    "gather_kv",
    "head_scales",
    "paged_attention_decode",
    "paged_attention_decode_seq",
    "paged_attention_prefill",
    "paged_attention_prefill_seq",
    "reshape_and_cache",
    "swap_blocks",
]
