"""CPU oracle for single-token paged decode attention.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. The
product path (``paged_kv_cache_36_amd``) never imports it and never falls back
to it; the two share no code.

Everything here is plain numpy in float64 and follows the pages' definitions
(the attention formula, the decode step, the paged address map, the online
softmax recurrence). See ``oracle/decode.py`` for the per-function citations;
``oracle/append.py`` holds the KV-append scatter and the page-size rule, and
``oracle/prefill.py`` the causal tail-Q prefill over the cached sequence, and
``oracle/compress.py`` the per-dimension softmax compression of a paged state
window.
"""

from .decode import (  # noqa: F401
    attention_decode,
    decode_batch,
    decode_partials,
    combine_partials,
    online_decode,
    resolve_offsets,
    gather_rows,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
)
