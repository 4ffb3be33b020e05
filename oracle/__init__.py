"""Oracle for MLA decode: TEST INFRASTRUCTURE, not part of the product.

A plain, slow, float64 CPU implementation of what the decode path computes,
written from the pages' formulas in their non-absorbed form: keys and values are
up-projected from the cached latent (k^C = W^UK c^KV, v^C = W^UV c^KV), the
decoupled RoPE key is concatenated to every head's key, and each head runs a
full (two-pass) softmax with scale 1/sqrt(d_h + d_h^R).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP library (``mla_latent_kv_37_amd``)
and never imports it; the only module both sides use is ``synth`` (seeded
random inputs and storage conversions, no attention arithmetic).

Pins (tests/test_oracle.py): brute-force loops on tiny inputs, torch's
scaled_dot_product_attention in float64 as an independent per-head attention,
the absorbed-vs-unabsorbed identity, special cases with closed forms, RoPE
invariants, the exact split/merge identity, the per-token cache sizes the pages
print, and the storage decoders against torch's own bf16 / float8_e4m3fn casts.
Nothing here is "parity unpinned".
"""
from . import mla, storage  # noqa: F401
from .mla import (attend, attend_head, attend_new_tokens, chunk_partials, forward_from_h, merge_partials,  # noqa: F401
                  out_project, prefill_head, project_cache, project_query, rope, rope_theta, softmax_scale,
                  yarn_attention_factor, yarn_theta)
from .storage import (bf16_bits_to_f64, dequantize_rows, e4m3fn_to_f64,  # noqa: F401
                      f32_to_bf16_bits, f64_to_e4m3fn, gather_sequence, quantize_e4m3_groups, stored_rows_f64)
