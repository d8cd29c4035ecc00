"""Python binding of the pkv C ABI (include/pkv.h), same names without the prefix.

Argument marshalling only: tensors are checked for dtype/device/layout, their
device pointers and strides are packed into ``pkv_decode_params`` and the C
entry point is called on torch's current stream (or the one given). Every
step of the computation runs in the HIP kernels of ``libpkv.so``; there is no
Python or CPU fallback.
"""

from __future__ import annotations

import ctypes

import torch

from ._lib import (AppendParams, CompressParams, DecodeParams, FinalizeParams, PlanInfo,
                   PrefillParams, load)

HEAD_SIZE = 256
GROUP = 6


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().pkv_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != 0:
        raise PkvError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")


def _page_stride(cache: torch.Tensor, name: str) -> int:
    """[pages, B, Hkv, D] with each page contiguous; pages may be spaced (unbind view)."""
    _need(cache, name, torch.bfloat16, 4)
    _, b, hkv, d = cache.shape
    if cache.stride(3) != 1 or cache.stride(2) != d or cache.stride(1) != hkv * d:
        raise ValueError(f"{name}: each page must be a contiguous [B, Hkv, D] block, "
                         f"got strides {cache.stride()}")
    return cache.stride(0)


def make_params(q, key_cache, value_cache, block_table, block_size, scale,
                max_seq_len=None, partition_tokens=0) -> DecodeParams:
    _need(q, "q", torch.bfloat16, 3)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [S, Hq, D]")
    ks = _page_stride(key_cache, "key_cache")
    vs = _page_stride(value_cache, "value_cache")
    if key_cache.shape[1:] != value_cache.shape[1:]:
        raise ValueError("key_cache and value_cache pages differ in shape")
    if key_cache.shape[1] != block_size:
        raise ValueError(f"cache pages hold {key_cache.shape[1]} tokens, block_size={block_size}")
    _need(block_table, "block_table", torch.int32, 2)
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous [S, max_blocks]")
    s, hq, d = q.shape
    if block_table.shape[0] != s:
        raise ValueError("block_table rows != number of sequences")
    hkv = key_cache.shape[2]
    if max_seq_len is None:
        max_seq_len = block_table.shape[1] * block_size
    p = DecodeParams()
    p.num_seqs = s
    p.num_q_heads = hq
    p.num_kv_heads = hkv
    p.head_size = d
    p.block_size = int(block_size)
    p.max_blocks_per_seq = block_table.shape[1]
    p.k_page_stride = ks
    p.v_page_stride = vs
    p.max_seq_len = int(max_seq_len)
    p.partition_tokens = int(partition_tokens)
    p.scale = float(scale)
    return p


def plan(params: DecodeParams) -> dict:
    info = PlanInfo()
    _check(load().pkv_plan(ctypes.byref(params), ctypes.byref(info)), "pkv_plan")
    return {f: getattr(info, f) for f, _ in PlanInfo._fields_}


def workspace_bytes(params: DecodeParams) -> int:
    return int(load().pkv_decode_workspace_bytes(ctypes.byref(params)))


def _seq_lens(seq_lens, s):
    _need(seq_lens, "seq_lens", torch.int32, 1)
    if seq_lens.shape[0] != s or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous int32 [S]")


def decode(q, key_cache, value_cache, block_table, seq_lens, block_size, scale, *,
           max_seq_len=None, partition_tokens=0, out=None, out_f32=None, workspace=None,
           stream=None):
    """o = softmax(q K^T * scale) V per sequence, K/V read through block_table.

    Returns ``out`` (bf16 [S, Hq, D]); allocates it (and the workspace) with
    torch when not given. ``out_f32`` (fp32 [S, Hq, D]), when given, also
    receives the result before the bf16 cast.
    """
    p = make_params(q, key_cache, value_cache, block_table, block_size, scale,
                    max_seq_len, partition_tokens)
    _seq_lens(seq_lens, q.shape[0])
    if out is None:
        out = torch.empty_like(q)
    need = workspace_bytes(p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().pkv_decode(ctypes.byref(p), _ptr(q), _ptr(key_cache), _ptr(value_cache),
                             _ptr(block_table), _ptr(seq_lens), _ptr(out), _ptr(out_f32),
                             _ptr(workspace), ws_bytes, _stream(stream)), "pkv_decode")
    return out


def noalloc_scratch_bytes() -> int:
    return int(load().pkv_noalloc_scratch_bytes())


def decode_noalloc(q, key_cache, value_cache, block_table, seq_lens, block_size, scale, out, *,
                   max_seq_len=None, partition_tokens=0, out_f32=None, stream=None):
    """pkv_decode_noalloc: decode into the caller's ``out`` (bf16 [S, Hq, D])
    and optional ``out_f32`` with the library's static scratch array as the
    workspace; nothing is allocated on either side of the call."""
    p = make_params(q, key_cache, value_cache, block_table, block_size, scale,
                    max_seq_len, partition_tokens)
    _seq_lens(seq_lens, q.shape[0])
    _check(load().pkv_decode_noalloc(ctypes.byref(p), _ptr(q), _ptr(key_cache),
                                     _ptr(value_cache), _ptr(block_table), _ptr(seq_lens),
                                     _ptr(out), _ptr(out_f32), _stream(stream)),
           "pkv_decode_noalloc")
    return out


def decode_partials(q, key_cache, value_cache, block_table, seq_lens, block_size, scale, *,
                    max_seq_len=None, partition_tokens=0, stream=None):
    """Returns (o_partial [S,Hq,n,D] f32, lse_partial [S,Hq,n] f32, out_f32 [S,Hq,D], out bf16)."""
    p = make_params(q, key_cache, value_cache, block_table, block_size, scale,
                    max_seq_len, partition_tokens)
    _seq_lens(seq_lens, q.shape[0])
    n = plan(p)["num_partitions"]
    s, hq, d = q.shape
    o_part = torch.zeros((s, hq, n, d), dtype=torch.float32, device=q.device)
    lse_part = torch.full((s, hq, n), float("nan"), dtype=torch.float32, device=q.device)
    out_f32 = torch.empty((s, hq, d), dtype=torch.float32, device=q.device)
    out = torch.empty_like(q)
    _check(load().pkv_decode_partials(ctypes.byref(p), _ptr(q), _ptr(key_cache),
                                      _ptr(value_cache), _ptr(block_table), _ptr(seq_lens),
                                      _ptr(o_part), _ptr(lse_part), _ptr(out_f32), _ptr(out),
                                      _stream(stream)), "pkv_decode_partials")
    return o_part, lse_part, out_f32, out


def split(params: DecodeParams, q, key_cache, value_cache, block_table, seq_lens, o_partial,
          lse_partial, stream=None):
    """The split-KV partition kernel alone (fp32 partials into caller buffers)."""
    _check(load().pkv_split(ctypes.byref(params), _ptr(q), _ptr(key_cache), _ptr(value_cache),
                            _ptr(block_table), _ptr(seq_lens), _ptr(o_partial),
                            _ptr(lse_partial), _stream(stream)), "pkv_split")


def split_balanced(params: DecodeParams, q, key_cache, value_cache, block_table, seq_lens,
                   workspace, stream=None):
    """First half of decode() with the balanced split: partials into workspace."""
    _check(load().pkv_split_balanced(ctypes.byref(params), _ptr(q), _ptr(key_cache),
                                     _ptr(value_cache), _ptr(block_table), _ptr(seq_lens),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)), "pkv_split_balanced")


def combine_balanced(params: DecodeParams, seq_lens, workspace, *, out=None, out_f32=None,
                     stream=None):
    """Second half of decode() with the balanced split."""
    _check(load().pkv_combine_balanced(ctypes.byref(params), _ptr(seq_lens), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _ptr(out),
                                       _ptr(out_f32), _stream(stream)), "pkv_combine_balanced")
    return out, out_f32


def combine(params: DecodeParams, o_partial, lse_partial, seq_lens, *, out=None, out_f32=None,
            stream=None):
    _check(load().pkv_combine(ctypes.byref(params), _ptr(o_partial), _ptr(lse_partial),
                              _ptr(seq_lens), _ptr(out), _ptr(out_f32), _stream(stream)),
           "pkv_combine")
    return out, out_f32


def debug_resolve(params: DecodeParams, kv_head, block_table, seq_lens, stream=None):
    offs = torch.empty((params.num_seqs, params.max_seq_len), dtype=torch.int64,
                       device=block_table.device)
    _check(load().pkv_debug_resolve(ctypes.byref(params), int(kv_head), _ptr(block_table),
                                    _ptr(seq_lens), _ptr(offs), _stream(stream)),
           "pkv_debug_resolve")
    return offs


def debug_gather(params: DecodeParams, which, cache, block_table, seq_lens, fill=0, stream=None):
    dense = torch.full((params.num_seqs, params.max_seq_len, params.num_kv_heads, HEAD_SIZE),
                       fill, dtype=torch.int16, device=cache.device).view(torch.bfloat16)
    _check(load().pkv_debug_gather(ctypes.byref(params), int(which), _ptr(cache),
                                   _ptr(block_table), _ptr(seq_lens), _ptr(dense),
                                   _stream(stream)), "pkv_debug_gather")
    return dense


def _new_rows(t: torch.Tensor, name: str, n: int, row: int) -> int:
    """[N, Hkv, D] (or [N, Hkv*D]) bf16 with each row contiguous; rows may be spaced."""
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.device.type != "cuda":
        raise TypeError(f"{name} must be a bf16 device tensor")
    if t.shape[0] != n or t[0].numel() != row:
        raise ValueError(f"{name} must be [{n}, ...] with {row} elements per token, "
                         f"got {tuple(t.shape)}")
    inner = t[0]
    if not inner.is_contiguous():
        raise ValueError(f"{name}: each token row must be contiguous")
    return t.stride(0) if n > 1 else row


def append(k_new, v_new, slot_mapping, key_cache, value_cache, stream=None):
    """Write the new tokens' K/V rows into the paged caches at their slots
    (page = slot // B, offset = slot % B; negative slots are padding)."""
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    if not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous")
    n = slot_mapping.shape[0]
    k_stride = _page_stride(key_cache, "key_cache")
    v_stride = _page_stride(value_cache, "value_cache")
    if key_cache.shape != value_cache.shape:
        raise ValueError("key_cache and value_cache shapes differ")
    pages, bsz, hkv, d = key_cache.shape
    p = AppendParams()
    p.num_tokens = n
    p.num_kv_heads = hkv
    p.head_size = d
    p.block_size = bsz
    p.num_pages = pages
    p.k_page_stride = k_stride
    p.v_page_stride = v_stride
    p.k_new_stride = _new_rows(k_new, "k_new", n, hkv * d) if n else hkv * d
    p.v_new_stride = _new_rows(v_new, "v_new", n, hkv * d) if n else hkv * d
    _check(load().pkv_append(ctypes.byref(p), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping),
                             _ptr(key_cache), _ptr(value_cache), _stream(stream)), "pkv_append")


def prefill_params(q, key_cache, value_cache, block_table, seq_len, block_size, scale,
                   key_splits=0):
    """pkv_prefill_params for q [Q, Hq, D] over caches [pages, B, Hkv, D]."""
    nq, hq, d = q.shape
    _, bsz, hkv, _ = key_cache.shape
    p = PrefillParams()
    p.num_q_tokens = nq
    p.num_q_heads = hq
    p.num_kv_heads = hkv
    p.head_size = d
    p.block_size = block_size
    p.max_blocks = block_table.shape[0]
    p.k_page_stride = _page_stride(key_cache, "key_cache")
    p.v_page_stride = _page_stride(value_cache, "value_cache")
    p.seq_len = int(seq_len)
    p.scale = float(scale)
    p.key_splits = int(key_splits)
    return p


def prefill_key_splits(params):
    """The key splits pkv_prefill makes for these params (raises on invalid ones)."""
    n = load().pkv_prefill_key_splits(ctypes.byref(params))
    _check(min(n, 0), "pkv_prefill_key_splits")
    return n


def prefill_short_blocks(params):
    """How many of the shortest query blocks take one key split fewer (raises
    on invalid params)."""
    n = load().pkv_prefill_short_blocks(ctypes.byref(params))
    _check(min(n, 0), "pkv_prefill_short_blocks")
    return n


def prefill_workspace_bytes(params):
    """Workspace bytes pkv_prefill needs for these params (0 for one split)."""
    return int(load().pkv_prefill_workspace_bytes(ctypes.byref(params)))


def prefill(q, key_cache, value_cache, block_table, seq_len, block_size, scale, *, out=None,
            out_f32=None, want_bf16=True, key_splits=0, workspace=None, stream=None):
    """Causal attention of one sequence's last q tokens (q: [Q, Hq, D] bf16)
    over its seq_len cached tokens; returns (out, out_f32). key_splits = 0
    lets the library choose; the workspace is allocated with torch when the
    call needs one and none is given."""
    _need(q, "q", torch.bfloat16, 3)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    _need(block_table, "block_table", torch.int32, 1)
    if not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous")
    bsz = key_cache.shape[1]
    if bsz != block_size:
        raise ValueError(f"block_size {block_size} does not match the cache ({bsz})")
    if out is None and want_bf16:
        out = torch.empty_like(q)
    p = prefill_params(q, key_cache, value_cache, block_table, seq_len, block_size, scale,
                       key_splits)
    need = prefill_workspace_bytes(p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().pkv_prefill(ctypes.byref(p), _ptr(q), _ptr(key_cache), _ptr(value_cache),
                              _ptr(block_table), _ptr(out), _ptr(out_f32), _ptr(workspace),
                              ws_bytes, _stream(stream)),
           "pkv_prefill")
    return out, out_f32


def compress_params(state_cache, token_to_req, boundary_token_indices, block_table,
                    compress_ratio, num_splits=0):
    """pkv_compress_params for a state cache [blocks, B, 2D] (fp32, any block
    stride, rows contiguous within a block)."""
    _need(state_cache, "state_cache", torch.float32, 3)
    nblk, bsz, row = state_cache.shape
    if state_cache.stride(2) != 1 or state_cache.stride(1) != row:
        raise ValueError("state_cache rows must be contiguous within a block")
    p = CompressParams()
    p.num_outputs = boundary_token_indices.shape[0]
    p.num_tokens = token_to_req.shape[0]
    p.num_reqs = block_table.shape[0]
    p.max_blocks = block_table.shape[1]
    p.head_dim = row // 2
    p.block_size = bsz
    p.compress_ratio = int(compress_ratio)
    p.num_splits = int(num_splits)
    p.block_stride = state_cache.stride(0)
    p.row_stride = state_cache.stride(1)
    return p


def compress_splits(p) -> int:
    return int(load().pkv_compress_splits(ctypes.byref(p)))


def compress_workspace_bytes(p) -> int:
    return int(load().pkv_compress_workspace_bytes(ctypes.byref(p)))


def compress(state_cache, token_to_req, positions, boundary_token_indices, block_table,
             compress_ratio, *, num_splits=0, out=None, workspace=None, stream=None):
    """Per-dimension softmax compression of each boundary token's window of
    paged state rows; returns compressed fp32 [N, D] (allocated with torch
    when not given, as is the workspace)."""
    _need(token_to_req, "token_to_req", torch.int32, 1)
    _need(positions, "positions", torch.int64, 1)
    _need(boundary_token_indices, "boundary_token_indices", torch.int64, 1)
    _need(block_table, "block_table", torch.int32, 2)
    for t, name in ((token_to_req, "token_to_req"), (positions, "positions"),
                    (boundary_token_indices, "boundary_token_indices"),
                    (block_table, "block_table")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if positions.shape[0] != token_to_req.shape[0]:
        raise ValueError("positions and token_to_req differ in length")
    p = compress_params(state_cache, token_to_req, boundary_token_indices, block_table,
                        compress_ratio, num_splits)
    n = p.num_outputs
    if out is None:
        out = torch.empty((n, p.head_dim), dtype=torch.float32, device=state_cache.device)
    need = int(load().pkv_compress_workspace_bytes(ctypes.byref(p)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=state_cache.device)
    _check(load().pkv_compress(ctypes.byref(p), _ptr(state_cache), _ptr(token_to_req),
                               _ptr(positions), _ptr(boundary_token_indices), _ptr(block_table),
                               _ptr(out), _ptr(workspace),
                               0 if workspace is None else workspace.numel(), _stream(stream)),
           "pkv_compress")
    return out


KV_PAGE_BYTES = 64 * (576 + 8)   # one packed KV page: 64 slots of payload, then their scales


def compress_finalize(compressed, positions, boundary_token_indices, rms_norm_weight,
                      cos_sin_cache, kv_slot_mapping, kv_cache, compress_ratio,
                      rms_norm_eps=1.0e-6, stream=None):
    """Write each output's packed bytes (INT8 NOPE codes, bf16 RoPE, scale
    bytes) into kv_cache (uint8 [pages, page_bytes], rows contiguous)."""
    _need(compressed, "compressed", torch.float32, 2)
    _need(positions, "positions", torch.int64, 1)
    _need(boundary_token_indices, "boundary_token_indices", torch.int64, 1)
    _need(rms_norm_weight, "rms_norm_weight", torch.float32, 1)
    _need(cos_sin_cache, "cos_sin_cache", torch.float32, 2)
    _need(kv_slot_mapping, "kv_slot_mapping", torch.int64, 1)
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    for t, name in ((compressed, "compressed"), (positions, "positions"),
                    (boundary_token_indices, "boundary_token_indices"),
                    (rms_norm_weight, "rms_norm_weight"), (cos_sin_cache, "cos_sin_cache"),
                    (kv_slot_mapping, "kv_slot_mapping")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if kv_cache.stride(1) != 1:
        raise ValueError("kv_cache pages must be contiguous bytes")
    if compressed.shape[1] != 512 or rms_norm_weight.shape[0] != 512 or cos_sin_cache.shape[1] != 64:
        raise ValueError("compressed [N, 512], rms_norm_weight [512], cos_sin_cache [rows, 64]")
    if kv_slot_mapping.shape[0] != positions.shape[0]:
        raise ValueError("kv_slot_mapping and positions differ in length")
    p = _finalize_params(compressed.shape[0], positions, cos_sin_cache, kv_cache,
                         compress_ratio, rms_norm_eps)
    _check(load().pkv_compress_finalize(ctypes.byref(p), _ptr(compressed), _ptr(positions),
                                        _ptr(boundary_token_indices), _ptr(rms_norm_weight),
                                        _ptr(cos_sin_cache), _ptr(kv_slot_mapping), _ptr(kv_cache),
                                        _stream(stream)), "pkv_compress_finalize")
    return kv_cache


def compress_pack(state_cache, token_to_req, positions, boundary_token_indices, block_table,
                  compress_ratio, rms_norm_weight, cos_sin_cache, kv_slot_mapping, kv_cache,
                  rms_norm_eps=1.0e-6, *, num_splits=0, compressed=None, workspace=None,
                  stream=None):
    """pkv_compress_pack: compress each boundary token's window and pack the
    rows into kv_cache in one call (the finalizer fused into the last kernel).
    kv_cache gets the bytes compress() then compress_finalize() would write;
    ``compressed`` (fp32 [N, 512]), when given, gets compress()'s rows. The
    workspace is allocated with torch when needed and not given."""
    for t, name, dt, nd in ((token_to_req, "token_to_req", torch.int32, 1),
                            (positions, "positions", torch.int64, 1),
                            (boundary_token_indices, "boundary_token_indices", torch.int64, 1),
                            (block_table, "block_table", torch.int32, 2),
                            (rms_norm_weight, "rms_norm_weight", torch.float32, 1),
                            (cos_sin_cache, "cos_sin_cache", torch.float32, 2),
                            (kv_slot_mapping, "kv_slot_mapping", torch.int64, 1)):
        _need(t, name, dt, nd)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _need(kv_cache, "kv_cache", torch.uint8, 2)
    if kv_cache.stride(1) != 1:
        raise ValueError("kv_cache pages must be contiguous bytes")
    if positions.shape[0] != token_to_req.shape[0] or kv_slot_mapping.shape[0] != positions.shape[0]:
        raise ValueError("token_to_req, positions and kv_slot_mapping differ in length")
    if rms_norm_weight.shape[0] != 512 or cos_sin_cache.shape[1] != 64:
        raise ValueError("rms_norm_weight [512], cos_sin_cache [rows, 64]")
    if compressed is not None:
        _need(compressed, "compressed", torch.float32, 2)
    p = compress_params(state_cache, token_to_req, boundary_token_indices, block_table,
                        compress_ratio, num_splits)
    fp = _finalize_params(p.num_outputs, positions, cos_sin_cache, kv_cache, compress_ratio,
                          rms_norm_eps)
    need = int(load().pkv_compress_workspace_bytes(ctypes.byref(p)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=state_cache.device)
    _check(load().pkv_compress_pack(ctypes.byref(p), ctypes.byref(fp), _ptr(state_cache),
                                    _ptr(token_to_req), _ptr(positions),
                                    _ptr(boundary_token_indices), _ptr(block_table),
                                    _ptr(rms_norm_weight), _ptr(cos_sin_cache),
                                    _ptr(kv_slot_mapping), _ptr(kv_cache), _ptr(compressed),
                                    _ptr(workspace),
                                    0 if workspace is None else workspace.numel(),
                                    _stream(stream)), "pkv_compress_pack")
    return kv_cache


def _finalize_params(n, positions, cos_sin_cache, kv_cache, compress_ratio, rms_norm_eps):
    p = FinalizeParams()
    p.num_outputs = n
    p.num_tokens = positions.shape[0]
    p.compress_ratio = int(compress_ratio)
    p.cos_sin_rows = cos_sin_cache.shape[0]
    p.num_kv_pages = kv_cache.shape[0]
    p.kv_page_stride = kv_cache.stride(0)
    p.rms_norm_eps = float(rms_norm_eps)
    return p


def page_tokens(state_page_bytes: int, attn_bytes_per_token: int, alignment_tokens: int) -> int:
    """Page-size rule: ceil(state / (alignment * bytes per token)) * alignment (host only)."""
    return int(load().pkv_page_tokens(state_page_bytes, attn_bytes_per_token, alignment_tokens))


def probe_sink_floats() -> int:
    return int(load().pkv_probe_sink_floats())


def probe_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    _check(load().pkv_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(stream)), "pkv_probe_read")


def probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None):
    _check(load().pkv_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                                 _stream(stream)), "pkv_probe_copy")
