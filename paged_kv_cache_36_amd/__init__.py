"""Paged KV-cache single-token decode attention for AMD MI355X (gfx950).

The compute path is the HIP library ``libpkv.so`` (C ABI in include/pkv.h);
``paged_kv_cache_36_amd.api`` is its thin Python binding. Besides decode, the
library writes new tokens into the paged cache (``append``), runs the causal
tail-Q prefill of one sequence (``prefill``), compresses windows of a paged
state cache and packs the results into KV pages (``compress`` and
``compress_finalize``, or both in one call, ``compress_pack``) and computes
the page-size rule (``page_tokens``).
``synth`` draws the seeded synthetic inputs.
"""

from ._lib import LIB_PATH, LibraryMissing, load  # noqa: F401
from .api import (  # noqa: F401
    PkvError,
    append,
    combine,
    combine_balanced,
    KV_PAGE_BYTES,
    compress,
    compress_finalize,
    compress_pack,
    compress_params,
    compress_splits,
    compress_workspace_bytes,
    debug_gather,
    debug_resolve,
    decode,
    decode_noalloc,
    decode_partials,
    make_params,
    noalloc_scratch_bytes,
    page_tokens,
    plan,
    prefill,
    prefill_key_splits,
    prefill_params,
    prefill_short_blocks,
    prefill_workspace_bytes,
    probe_copy,
    probe_read,
    split,
    split_balanced,
    workspace_bytes,
)
