"""Plain CPU oracle for the FP8 paged MLA decode path.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it shares no code, table or helper with that path.

What it computes, and where the pages define it:

* ``e4m3``: the FP8-E4M3FN byte format the KV pool is stored in
  ("The KV Cache Cast Bottleneck", *The Context*: the pool is
  ``Float8_e4m3fn`` and is cast to BFloat16).  The pages name the format only;
  the bit layout follows the public OCP 8-bit floating point (OFP8) format
  definition.
* ``cast``: the full-pool dtype cast ``get_key_buffer(l).to(q.dtype)``
  ("The KV Cache Cast Bottleneck", *The Context* and *The Message*) and the
  gather-then-cast of only the slots named by ``kv_indices``
  ("The Gather-Then-Cast Pivot", *Reasoning Process*).
* ``encode``: the write path, BF16 rows into the FP8 cache by a dtype copy
  ("When a Faster Kernel Doesn't Speed Up Serving", *Step 3*, CastToFP8),
  with torch's float -> ``Float8_e4m3fn`` rounding rule.
* ``attention``: MLA decode over the absorbed latent cache -- one KV head of
  width 576 = 512 latent + 64 rope shared by all query heads, scores over all
  576 dims, values from the first 512 ("The KV Cache Cast Bottleneck",
  *The Context*; "The Gather-Then-Cast Pivot", *The Subject Message*), with a
  max-subtracted softmax, in float64.
* ``extend``: the same attention with several new query tokens per request
  and a causal mask over the request's cache list, the extend/prefill path
  ("When a Faster Kernel Doesn't Speed Up Serving", *Step 3*, CastFromFP8;
  "The KV Cache Cast Bottleneck", *The Message*).

Pinned by the ``-m "not gpu"`` tests (OCP special values, torch's own FP8
decode, brute force, closed forms and invariants).  The attention numerics at
the full serving shapes have no printed values on the pages; they rest on
those pins.
"""
from .e4m3 import decode_table, e4m3fn_value, bf16_bits_of, cast_table_bf16
from .encode import encode_e4m3fn, scatter_ref
from .cast import cast_ref, gather_ref
from .extend import mla_extend_ref, visible_tokens
from .attention import (
    bf16_bits_to_f64,
    mla_decode_ref,
    mla_decode_partial_ref,
    combine_partials_ref,
    KV_WIDTH,
    V_WIDTH,
)

__all__ = [
    "decode_table",
    "e4m3fn_value",
    "bf16_bits_of",
    "cast_table_bf16",
    "cast_ref",
    "gather_ref",
    "encode_e4m3fn",
    "scatter_ref",
    "bf16_bits_to_f64",
    "mla_decode_ref",
    "mla_extend_ref",
    "visible_tokens",
    "mla_decode_partial_ref",
    "combine_partials_ref",
    "KV_WIDTH",
    "V_WIDTH",
]
