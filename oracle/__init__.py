"""CPU oracle for paged grouped-query decode attention and the one-token page append.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check of the entry module
and the CPU-baseline leg of the benchmark use it.  It shares no code, header,
table or helper with the HIP library; the two meet only through the seeded
input arrays the tests hand to both.

Sources (pages of the subject; cited by title and section):

* "6 Hours of YouTube and 85 handtyped pages of notes on LLM Inference - Start
  here" (Hacker News item for the samir-vllm engine, translated README),
  section "features completed so far": one shared BF16 K/V page pool, a block
  table per sequence (and layer), 16 tokens of K and V per physical page,
  decode writes the new token's K/V at its absolute position, and each query
  head streams its own sequence's pages with an FP32 online softmax, without a
  contiguous prefix gather and without storing scores.  Batched decode gives
  every sequence its own page map and attention length.
* "Building an LLM inference engine from scratch: KV cache, operator fusion and
  quantisation practice" (coreui.cn article), section 3.2: single-query
  attention is scores = q K^T, scaled by 1/sqrt(head_dim), softmax with the
  maximum subtracted for stability, then the weighted sum of V; heads are
  computed independently and concatenated.  Section 2.1: the cache holds the K
  and V of every earlier token and the new token's projections are appended.

Every function here is the plain definition, in float64, with explicit Python
loops over sequences and heads so that it can be read against the pages.
"""

from .paged_decode import (  # noqa: F401
    bf16_bits_to_f64,
    gather_sequence,
    attention_one_query,
    decode_attention,
    append_kv,
    fill_kv,
    kv_head_of,
)
from . import admission, kvquant, rope  # noqa: F401,E402
