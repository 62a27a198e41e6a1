"""Torch-tensor front end of libpa: argument marshalling only.

Each function checks that the tensors are on the GPU, contiguous and of the
types the C ABI expects, takes their device pointers and the current HIP
stream, and calls the library.  All computation happens in the HIP kernels;
there is no CPU fallback.  Outputs and workspaces are allocated with torch
when the caller does not pass them.
"""

import math

import torch

from . import _lib

_DTYPES = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16}


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or "
                        "bfloat16") from None


def _need_gpu(*tensors):
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("libpa operates on GPU tensors only")
        if not t.is_contiguous():
            raise ValueError("libpa needs contiguous tensors")


def _check_out(out, q):
    """A caller's output buffer must be exactly the result's: the kernels
    write q.numel() elements of q's dtype to it, so a smaller buffer, another
    dtype or another device would be written past or misread."""
    if out is None:
        return
    if out.device != q.device:
        raise ValueError(f"out is on {out.device}, q on {q.device}")
    if out.dtype != q.dtype:
        raise TypeError(f"out dtype {out.dtype} differs from q dtype {q.dtype}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out shape {tuple(out.shape)} differs from q shape "
                         f"{tuple(q.shape)}")


def _check_workspace(workspace, q):
    """The workspace must sit on q's device (its size is checked by the
    library against the query)."""
    if workspace is not None and workspace.device != q.device:
        raise ValueError(f"workspace is on {workspace.device}, q on {q.device}")


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _stream(t):
    return ctypes_void(torch.cuda.current_stream(t.device).cuda_stream)


def ctypes_void(x):
    return x if x else None


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() else None


def store_kv(k, v, k_cache, v_cache, slot_mapping):
    """Write rows of k / v ([T, Hkv, D]) to flat slots of the caches
    ([NB, bs, Hkv, D]); negative slots are skipped."""
    _need_gpu(k, v, k_cache, v_cache, slot_mapping)
    _i32(slot_mapping, "slot_mapping")
    if k.shape != v.shape or k.dim() != 3:
        raise ValueError("k and v must both be [T, Hkv, D]")
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ValueError("caches must be [NB, bs, Hkv, D]")
    if tuple(k_cache.shape[2:]) != tuple(k.shape[1:]):
        raise ValueError("cache row shape differs from k/v row shape")
    if k.dtype != k_cache.dtype or v.dtype != k.dtype:
        raise TypeError("k, v and caches must share a dtype")
    if slot_mapping.numel() != k.shape[0]:
        raise ValueError("slot_mapping must have one entry per row")
    lib = _lib.load()
    st = lib.pa_store_kv(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                         _ptr(slot_mapping), k.shape[0], k.shape[1],
                         k.shape[2], k_cache.shape[0] * k_cache.shape[1],
                         _dtype_code(k), _stream(k))
    _lib.check("pa_store_kv", st)


def copy_blocks(k_cache, v_cache, block_pairs):
    """Copy whole blocks of both caches ([NB, ...], same shape): for each row
    (src, dst) of block_pairs (int32 [P, 2]), block dst becomes a copy of
    block src.  Pairs naming a block outside the pool copy nothing."""
    _need_gpu(k_cache, v_cache, block_pairs)
    _i32(block_pairs, "block_pairs")
    if k_cache.shape != v_cache.shape or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache must match in shape and dtype")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [P, 2]")
    if not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("caches must be contiguous")
    num_blocks = k_cache.shape[0]
    block_bytes = k_cache.numel() // max(num_blocks, 1) * k_cache.element_size()
    lib = _lib.load()
    st = lib.pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_pairs),
                            block_pairs.shape[0], block_bytes, num_blocks,
                            _stream(k_cache))
    _lib.check("pa_copy_blocks", st)


def decode_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                           max_context_len):
    return int(_lib.load().pa_decode_workspace_bytes(
        num_seqs, num_heads, num_kv_heads, head_dim, max_context_len))


def decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
           scale=None, out=None, workspace=None):
    """Paged decode attention.  q [B, Hq, D]; caches [NB, 16, Hkv, D];
    block_tables int32 [B, W]; context_lens int32 [B] (counting the new
    token); max_context_len a host-side upper bound.  Returns out [B, Hq, D].
    """
    _check_out(out, q)
    _check_workspace(workspace, q)
    _need_gpu(q, k_cache, v_cache, block_tables, context_lens, out, workspace)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    b, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, W]")
    if context_lens.numel() != b:
        raise ValueError("context_lens must be [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(b, hq, hkv, d, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() \
        if workspace is not None else 0
    lib = _lib.load()
    st = lib.pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), nb,
                       bs, _ptr(block_tables), block_tables.shape[1],
                       _ptr(context_lens), int(max_context_len), b, hq, hkv,
                       d, scale, _ptr(workspace), ws_bytes, _dtype_code(q),
                       _stream(q))
    _lib.check("pa_decode", st)
    return out


DECODE_SCRATCH_BYTES = 32 << 20   # the library's static decode scratch


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens,
                   max_context_len, scale=None, out=None):
    """decode() without a workspace: the library keeps the partial results
    in its static per-GPU scratch (32 MiB), so the C call allocates nothing.
    Calls that overlap on one GPU race on that scratch.  With ``out`` given,
    this function allocates nothing either."""
    _check_out(out, q)
    _need_gpu(q, k_cache, v_cache, block_tables, context_lens, out)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    b, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, W]")
    if context_lens.numel() != b:
        raise ValueError("context_lens must be [B]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    lib = _lib.load()
    st = lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache),
                               _ptr(v_cache), nb, bs, _ptr(block_tables),
                               block_tables.shape[1], _ptr(context_lens),
                               int(max_context_len), b, hq, hkv, d, scale,
                               _dtype_code(q), _stream(q))
    _lib.check("pa_decode_noalloc", st)
    return out


def shared_prefix_workspace_bytes(num_seqs, num_heads, num_kv_heads,
                                  head_dim, max_suffix_len, max_prefix_len,
                                  num_groups, max_group_size):
    return int(_lib.load().pa_decode_shared_prefix_workspace_bytes(
        num_seqs, num_heads, num_kv_heads, head_dim, max_suffix_len,
        max_prefix_len, num_groups, max_group_size))


def decode_shared_prefix(q, k_cache, v_cache, block_tables, context_lens,
                         prefix_lens, groups, max_suffix_len, max_prefix_len,
                         max_group_size, scale=None, out=None,
                         workspace=None):
    """Decode attention where groups of consecutive sequences share their
    leading blocks (same result as decode()).  prefix_lens int32 [B]
    (shared tokens, 0 outside any group); groups int32 [G, 2] (first
    sequence, count); max_suffix_len / max_prefix_len / max_group_size are
    host-side bounds.  Returns out [B, Hq, D]."""
    _check_out(out, q)
    _check_workspace(workspace, q)
    _need_gpu(q, k_cache, v_cache, block_tables, context_lens, prefix_lens,
              groups, out, workspace)
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"),
                 (prefix_lens, "prefix_lens"), (groups, "groups")):
        _i32(t, n)
    b, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, W]")
    if context_lens.numel() != b or prefix_lens.numel() != b:
        raise ValueError("context_lens and prefix_lens must be [B]")
    if groups.dim() != 2 or groups.shape[1] != 2:
        raise ValueError("groups must be [G, 2]")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    ng = groups.shape[0]
    need = shared_prefix_workspace_bytes(b, hq, hkv, d, max_suffix_len,
                                         max_prefix_len, ng, max_group_size)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() \
        if workspace is not None else 0
    lib = _lib.load()
    st = lib.pa_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), nb, bs,
        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(prefix_lens), int(max_suffix_len), int(max_prefix_len),
        _ptr(groups), ng, int(max_group_size), b, hq, hkv, d, scale,
        _ptr(workspace), ws_bytes, _dtype_code(q), _stream(q))
    _lib.check("pa_decode_shared_prefix", st)
    return out


def store_kv_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale):
    """Quantise rows of k / v ([T, Hkv, D], bf16 or fp32) into 8-bit E4M3
    caches (uint8 [NB, bs, Hkv, D]) at flat slots; negative slots skipped.
    Each element is stored as the code of x / scale (per cache)."""
    _need_gpu(k, v, k_cache, v_cache, slot_mapping)
    _i32(slot_mapping, "slot_mapping")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("8-bit caches must be uint8 tensors of E4M3 codes")
    t, hkv, d = k.shape
    nb, bs, hkv2, d2 = k_cache.shape
    if (hkv2, d2) != (hkv, d) or v_cache.shape != k_cache.shape or \
            v.shape != k.shape or slot_mapping.numel() != t:
        raise ValueError("shapes of rows, caches and slot_mapping disagree")
    lib = _lib.load()
    st = lib.pa_store_kv_fp8(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                             _ptr(slot_mapping), t, hkv, d, nb * bs,
                             _dtype_code(k), float(k_scale), float(v_scale),
                             _stream(k))
    _lib.check("pa_store_kv_fp8", st)


def decode_fp8(q, k_cache, v_cache, block_tables, context_lens,
               max_context_len, k_scale, v_scale, scale=None, out=None,
               workspace=None):
    """Paged decode over 8-bit E4M3 caches (uint8 [NB, 16, Hkv, 128]):
    K = code * k_scale, V = code * v_scale; q and out bf16 [B, Hq, 128]."""
    _check_out(out, q)
    _check_workspace(workspace, q)
    _need_gpu(q, k_cache, v_cache, block_tables, context_lens, out, workspace)
    _i32(block_tables, "block_tables")
    _i32(context_lens, "context_lens")
    if q.dtype != torch.bfloat16:
        raise TypeError("decode over an 8-bit cache takes bf16 q")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("8-bit caches must be uint8 tensors of E4M3 codes")
    b, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q")
    if block_tables.dim() != 2 or block_tables.shape[0] != b:
        raise ValueError("block_tables must be [B, W]")
    if context_lens.numel() != b:
        raise ValueError("context_lens must be [B]")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(b, hq, hkv, d, max_context_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() \
        if workspace is not None else 0
    lib = _lib.load()
    st = lib.pa_decode_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                           nb, bs, _ptr(block_tables), block_tables.shape[1],
                           _ptr(context_lens), int(max_context_len), b, hq,
                           hkv, d, scale, float(k_scale), float(v_scale),
                           _ptr(workspace), ws_bytes, _stream(q))
    _lib.check("pa_decode_fp8", st)
    return out


def prefill_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                            max_seqlen_q, max_seqlen_k):
    return int(_lib.load().pa_prefill_workspace_bytes(
        num_seqs, num_heads, num_kv_heads, head_dim, max_seqlen_q,
        max_seqlen_k))


def prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                   max_seqlen_q, max_seqlen_k, block_tables, scale=None,
                   causal=True, out=None, workspace=None):
    """Varlen chunked prefill.  q [total_q, Hq, D] packed by cu_seqlens_q;
    keys are the first cu_seqlens_k[b+1]-cu_seqlens_k[b] tokens of each
    sequence's block table.  Returns out [total_q, Hq, D]."""
    _check_out(out, q)
    _check_workspace(workspace, q)
    _need_gpu(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, block_tables,
              out, workspace)
    for t, n in ((cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k"),
                 (block_tables, "block_tables")):
        _i32(t, n)
    total_q, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    num_seqs = cu_seqlens_q.numel() - 1
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("cache shape does not match q")
    if cu_seqlens_k.numel() != num_seqs + 1 or block_tables.shape[0] != num_seqs:
        raise ValueError("cu_seqlens_k / block_tables do not match cu_seqlens_q")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    need = prefill_workspace_bytes(num_seqs, hq, hkv, d, max_seqlen_q,
                                   max_seqlen_k)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() \
        if workspace is not None else 0
    lib = _lib.load()
    st = lib.pa_prefill_varlen(
        _ptr(out), _ptr(q), total_q, _ptr(k_cache), _ptr(v_cache), nb, bs,
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(max_seqlen_q),
        int(max_seqlen_k), _ptr(block_tables), block_tables.shape[1],
        num_seqs, hq, hkv, d, scale, 1 if causal else 0, _ptr(workspace),
        ws_bytes, _dtype_code(q), _stream(q))
    _lib.check("pa_prefill_varlen", st)
    return out
