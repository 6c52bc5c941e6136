"""TurboQuant hot path for AMD MI355X (gfx950).

Python face of libtq.so: quantize key/value vectors into the packed rotated-codebook +
QJL-sign format, run decode attention and inner-product top-k search straight from the
packed bytes.  These wrappers only check shapes/dtypes, allocate outputs with torch and
pass pointers and the current HIP stream to the C ABI declared in include/tq.h; all
arithmetic runs in the library's kernels.  A missing library raises, never falls back.
"""
from __future__ import annotations

import ctypes
import math

import numpy as np

from ._lib import (LIB_PATH, TQ_BF16, TQ_F16, TQ_F32, Format, Tables, TQError, build_codebook,
                   load, c_cache_segment, make_rotation)

__all__ = ["Format", "Tables", "TQError", "build_codebook", "make_rotation", "quantize_kv", "attend_decode",
           "attend_decode_noalloc",
           "attend_decode_segments", "attend_segments_workspace_bytes",
           "ip_search", "requantize", "attend_workspace_bytes", "search_workspace_bytes",
           "requantize_workspace_bytes", "quantize_kv_paged", "attend_decode_paged",
           "prefill_paged", "prefill_workspace_bytes", "LIB_PATH", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    if t.dtype == torch.float16:
        return TQ_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(device) -> ctypes.c_void_p:
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check(code: int, what: str) -> None:
    if code != 0:
        raise TQError(code, what)


def quantize_kv(x, fmt: Format, tables: Tables, counters=None, codes=None, norms=None):
    """Quantize the rows of x ([..., d_in], fp32 / bf16 / fp16 CUDA tensor, unit stride in
    the last dim).  Returns (codes uint8 [n, record_bytes], norms fp16 [n, 2]); pass
    preallocated `codes`/`norms` to write in place.  `counters` (int64 CUDA tensor of 4)
    accumulates the diagnostics documented in tq.h.  With fmt.layout == 1 (token-sliced,
    n a multiple of 32) codes holds the same bytes as groups: [n // 32, 32 * record_bytes]."""
    torch = _torch()
    if not x.is_cuda:
        raise ValueError("x must be a CUDA tensor")
    d_in = x.shape[-1]
    x2 = x.reshape(-1, d_in)
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    n = x2.shape[0]
    rb = fmt.record_bytes()
    if codes is None:
        shape = (n // 32, 32 * rb) if fmt.layout == 1 else (n, rb)
        codes = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if norms is None:
        norms = torch.empty((n, 2), dtype=torch.float16, device=x.device)
    if codes.numel() < n * rb or norms.numel() < 2 * n:
        raise ValueError("output buffers too small")
    f, t = fmt.c(), tables.c()
    rc = load().tq_quantize_kv(ctypes.byref(f), ctypes.byref(t), _ptr(x2), _dtype_code(x2), n,
                               d_in, x2.stride(0) if n > 1 else d_in, _ptr(codes), _ptr(norms),
                               _ptr(counters), _stream(x.device))
    _check(rc, "tq_quantize_kv")
    return codes, norms


def attend_workspace_bytes(batch, hq, hkv, capacity, d=128) -> int:
    n = load().tq_attend_workspace_bytes(batch, hq, hkv, capacity, d)
    if n < 0:
        raise TQError(-2, "tq_attend_workspace_bytes")
    return int(n)


def _decode_args(q, codes_k, norms_k, codes_v, norms_v, seq_lens, fmt_k, fmt_v, scale):
    torch = _torch()
    batch, hq, d = q.shape
    _, hkv, capacity, _ = codes_k.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t, f in ((codes_k, fmt_k), (codes_v, fmt_v)):
        rb = f.record_bytes()
        shape = (batch, hkv, capacity // 32, 32 * rb) if f.layout == 1 else (batch, hkv, capacity, rb)
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"bad packed cache tensor: expected uint8 {shape}")
    for t in (norms_k, norms_v):
        if t.shape != (batch, hkv, capacity, 2) or not t.is_contiguous():
            raise ValueError("bad norms tensor")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != batch:
        raise ValueError("seq_lens must be int32 [batch]")
    return batch, hq, hkv, capacity, d, scale


def attend_decode(q, codes_k, norms_k, codes_v, norms_v, seq_lens, fmt_k: Format,
                  tables_k: Tables, fmt_v: Format = None, tables_v: Tables = None,
                  scale: float = None, tau: float = 0.0, logits: bool = False,
                  skipped=None, workspace=None, out=None):
    """One decode step.  q [batch, hq, d]; codes_k [batch, hkv, capacity, rbk] uint8;
    norms_k [batch, hkv, capacity, 2] fp16; the same for v (token-sliced values, fmt_v.layout
    == 1: codes_v [batch, hkv, capacity // 32, 32 * rbv]); seq_lens int32 [batch] (CUDA).
    Returns out fp32 [batch, hq, d] (and logits fp32 [batch, hq, capacity] if asked)."""
    torch = _torch()
    fmt_v = fmt_k if fmt_v is None else fmt_v
    tables_v = tables_k if tables_v is None else tables_v
    q = q.contiguous()
    batch, hq, hkv, capacity, d, scale = _decode_args(q, codes_k, norms_k, codes_v, norms_v,
                                                      seq_lens, fmt_k, fmt_v, scale)
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    lg = torch.empty((batch, hq, capacity), dtype=torch.float32, device=q.device) if logits else None
    wsb = attend_workspace_bytes(batch, hq, hkv, capacity, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    fk, fv, tk, tv = fmt_k.c(), fmt_v.c(), tables_k.c(), tables_v.c()
    rc = load().tq_attend_decode(ctypes.byref(fk), ctypes.byref(tk), ctypes.byref(fv),
                                 ctypes.byref(tv), _ptr(q), _dtype_code(q), batch, hq, hkv,
                                 _ptr(codes_k), _ptr(norms_k), _ptr(codes_v), _ptr(norms_v),
                                 capacity, _ptr(seq_lens), float(scale), float(tau), _ptr(out),
                                 _ptr(lg), _ptr(skipped), _ptr(workspace), workspace.numel(),
                                 _stream(q.device))
    _check(rc, "tq_attend_decode")
    return (out, lg) if logits else out


def attend_decode_noalloc(q, codes_k, norms_k, codes_v, norms_v, seq_lens, fmt_k: Format,
                          tables_k: Tables, out, fmt_v: Format = None, tables_v: Tables = None,
                          scale: float = None, tau: float = 0.0, logits=None, skipped=None):
    """attend_decode through tq_attend_decode_noalloc: the caller passes every output
    (out fp32 [batch, hq, d], optional logits fp32 [batch, hq, capacity]) and nothing is
    allocated; the split partials live in the library's per-GPU device array.  q must be
    contiguous."""
    fmt_v = fmt_k if fmt_v is None else fmt_v
    tables_v = tables_k if tables_v is None else tables_v
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    batch, hq, hkv, capacity, d, scale = _decode_args(q, codes_k, norms_k, codes_v, norms_v,
                                                      seq_lens, fmt_k, fmt_v, scale)
    fk, fv, tk, tv = fmt_k.c(), fmt_v.c(), tables_k.c(), tables_v.c()
    rc = load().tq_attend_decode_noalloc(ctypes.byref(fk), ctypes.byref(tk), ctypes.byref(fv),
                                         ctypes.byref(tv), _ptr(q), _dtype_code(q), batch, hq,
                                         hkv, _ptr(codes_k), _ptr(norms_k), _ptr(codes_v),
                                         _ptr(norms_v), capacity, _ptr(seq_lens), float(scale),
                                         float(tau), _ptr(out), _ptr(logits), _ptr(skipped),
                                         _stream(q.device))
    _check(rc, "tq_attend_decode_noalloc")
    return out


def attend_segments_workspace_bytes(batch: int, hq: int, hkv: int, capacities, d: int = 128) -> int:
    caps = (ctypes.c_int64 * len(capacities))(*[int(c) for c in capacities])
    n = load().tq_attend_segments_workspace_bytes(batch, hq, hkv, len(capacities), caps, d)
    if n < 0:
        raise ValueError("bad shape")
    return int(n)


def attend_decode_segments(q, segments, scale: float = None, tau: float = 0.0, skipped=None,
                           workspace=None, out=None):
    """One decode step over a cache kept in segments of different formats (older tokens
    re-encoded narrower): each query attends to its tokens of segment 0, then 1, ... with
    one softmax.  segments: sequence of (codes_k, norms_k, codes_v, norms_v, seq_lens,
    fmt_k, tables_k, fmt_v, tables_v) with the tensors laid out as for attend_decode; value
    tables must share one rotation (S and signs).  Returns out fp32 [batch, hq, d]."""
    torch = _torch()
    batch, hq, d = q.shape
    hkv = segments[0][0].shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    keep, segs = [], (c_cache_segment * len(segments))()
    caps = []
    for i, (ck, nk, cv, nv, seq, fk, tk, fv, tv) in enumerate(segments):
        cap = ck.shape[2]
        for t, rb in ((ck, fk.record_bytes()), (cv, fv.record_bytes())):
            if t.dtype != torch.uint8 or t.shape[:3] != (batch, hkv, cap) or t.shape[3] != rb \
                    or not t.is_contiguous():
                raise ValueError(f"segment {i}: bad packed cache tensor")
        for t in (nk, nv):
            if t.shape != (batch, hkv, cap, 2) or not t.is_contiguous():
                raise ValueError(f"segment {i}: bad norms tensor")
        if seq.dtype != torch.int32 or seq.numel() != batch:
            raise ValueError(f"segment {i}: seq_lens must be int32 [batch]")
        c = (fk.c(), tk.c(), fv.c(), tv.c())
        keep.append(c)
        segs[i] = c_cache_segment(ctypes.addressof(c[0]), ctypes.addressof(c[1]),
                                  ctypes.addressof(c[2]), ctypes.addressof(c[3]), _ptr(ck), _ptr(nk),
                                  _ptr(cv), _ptr(nv), cap, _ptr(seq))
        caps.append(cap)
    q = q.contiguous()
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    wsb = attend_segments_workspace_bytes(batch, hq, hkv, caps, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    rc = load().tq_attend_decode_segments(segs, len(segments), _ptr(q), _dtype_code(q), batch, hq,
                                          hkv, float(scale), float(tau), _ptr(out), _ptr(skipped),
                                          _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(rc, "tq_attend_decode_segments")
    return out


def quantize_kv_paged(x, fmt: Format, tables: Tables, slot_mapping, codes_cache, norms_cache,
                      counters=None):
    """Append: quantize new keys or values x [n_tokens, hkv, d_in] (CUDA, fp32 / bf16 / fp16)
    into a paged cache codes_cache [num_pages, hkv, page_size, record_bytes] uint8,
    norms_cache [num_pages, hkv, page_size, 2] fp16, token i going to slot slot_mapping[i]
    (int64, page * page_size + offset; negative: skipped)."""
    torch = _torch()
    n_tokens, hkv, d_in = x.shape
    num_pages, hkv2, page_size, rb = codes_cache.shape
    if hkv2 != hkv or rb != fmt.record_bytes() or not codes_cache.is_contiguous():
        raise ValueError("bad paged cache tensor")
    if norms_cache.shape != (num_pages, hkv, page_size, 2) or not norms_cache.is_contiguous():
        raise ValueError("bad paged norms tensor")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != n_tokens:
        raise ValueError("slot_mapping must be int64 [n_tokens]")
    x2 = x.reshape(n_tokens * hkv, d_in)
    if x2.stride(-1) != 1:
        x2 = x2.contiguous()
    f, t = fmt.c(), tables.c()
    ld = x2.stride(0) if x2.shape[0] > 1 else d_in
    rc = load().tq_quantize_kv_paged(ctypes.byref(f), ctypes.byref(t), _ptr(x2), _dtype_code(x2),
                                     n_tokens, hkv, d_in, ld, _ptr(slot_mapping), page_size,
                                     num_pages, _ptr(codes_cache), _ptr(norms_cache),
                                     _ptr(counters), _stream(x.device))
    _check(rc, "tq_quantize_kv_paged")


def attend_decode_paged(q, codes_k, norms_k, codes_v, norms_v, block_table, seq_lens,
                        fmt_k: Format, tables_k: Tables, fmt_v: Format = None,
                        tables_v: Tables = None, scale: float = None, tau: float = 0.0,
                        logits: bool = False, skipped=None, workspace=None, out=None):
    """One decode step over paged caches: codes_k [num_pages, hkv, page_size, rbk] uint8,
    norms_k [num_pages, hkv, page_size, 2] fp16 (the same for v), block_table int32
    [batch, max_blocks] of page ids, seq_lens int32 [batch].  Returns out fp32 [batch, hq, d]
    (and logits fp32 [batch, hq, max_blocks * page_size] if asked)."""
    torch = _torch()
    fmt_v = fmt_k if fmt_v is None else fmt_v
    tables_v = tables_k if tables_v is None else tables_v
    batch, hq, d = q.shape
    num_pages, hkv, page_size, _ = codes_k.shape
    for t, rb in ((codes_k, fmt_k.record_bytes()), (codes_v, fmt_v.record_bytes())):
        if t.dtype != torch.uint8 or t.shape[:3] != (num_pages, hkv, page_size) or t.shape[3] != rb \
                or not t.is_contiguous():
            raise ValueError("bad paged cache tensor")
    for t in (norms_k, norms_v):
        if t.shape != (num_pages, hkv, page_size, 2) or not t.is_contiguous():
            raise ValueError("bad paged norms tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != batch \
            or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [batch, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != batch:
        raise ValueError("seq_lens must be int32 [batch]")
    max_blocks = block_table.shape[1]
    capacity = max_blocks * page_size
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = q.contiguous()
    if out is None:
        out = torch.empty((batch, hq, d), dtype=torch.float32, device=q.device)
    lg = torch.empty((batch, hq, capacity), dtype=torch.float32, device=q.device) if logits else None
    wsb = attend_workspace_bytes(batch, hq, hkv, capacity, d)
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=q.device)
    fk, fv, tk, tv = fmt_k.c(), fmt_v.c(), tables_k.c(), tables_v.c()
    rc = load().tq_attend_decode_paged(ctypes.byref(fk), ctypes.byref(tk), ctypes.byref(fv),
                                       ctypes.byref(tv), _ptr(q), _dtype_code(q), batch, hq, hkv,
                                       _ptr(codes_k), _ptr(norms_k), _ptr(codes_v), _ptr(norms_v),
                                       page_size, num_pages, _ptr(block_table), max_blocks,
                                       _ptr(seq_lens), float(scale), float(tau), _ptr(out), _ptr(lg),
                                       _ptr(skipped), _ptr(workspace), workspace.numel(),
                                       _stream(q.device))
    _check(rc, "tq_attend_decode_paged")
    return (out, lg) if logits else out


def prefill_workspace_bytes(n_new, hq, hkv, start) -> int:
    n = load().tq_prefill_workspace_bytes(n_new, hq, hkv, start)
    if n < 0:
        raise TQError(-1, "tq_prefill_workspace_bytes")
    return int(n)


def prefill_paged(q, k_new, v_new, start, codes_k, norms_k, codes_v, norms_v, block_table,
                  fmt_k: Format, tables_k: Tables, fmt_v: Format = None, tables_v: Tables = None,
                  scale: float = None, counters=None, workspace=None, out=None):
    """One prefill chunk of one sequence: k_new / v_new [n_new, hkv, 128] are quantized into
    the paged caches at positions start .. start + n_new - 1 (pages from block_table, int32
    [max_blocks]), then q [n_new, hq, 128] attends causally to the cache.  Returns out fp32
    [n_new, hq, 128]."""
    torch = _torch()
    fmt_v = fmt_k if fmt_v is None else fmt_v
    tables_v = tables_k if tables_v is None else tables_v
    n_new, hq, d = q.shape
    num_pages, hkv, page_size, _ = codes_k.shape
    if k_new.shape != (n_new, hkv, d) or v_new.shape != (n_new, hkv, d) or k_new.dtype != v_new.dtype:
        raise ValueError("k_new / v_new must be [n_new, hkv, d] of one dtype")
    for t, rb in ((codes_k, fmt_k.record_bytes()), (codes_v, fmt_v.record_bytes())):
        if t.dtype != torch.uint8 or t.shape[:3] != (num_pages, hkv, page_size) or t.shape[3] != rb \
                or not t.is_contiguous():
            raise ValueError("bad paged cache tensor")
    for t in (norms_k, norms_v):
        if t.shape != (num_pages, hkv, page_size, 2) or not t.is_contiguous():
            raise ValueError("bad paged norms tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 1 or not block_table.is_contiguous():
        raise ValueError("block_table must be contiguous int32 [max_blocks]")
    max_blocks = block_table.shape[0]
    k2, v2 = k_new.reshape(-1, d).contiguous(), v_new.reshape(-1, d).contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = q.contiguous()
    if out is None:
        out = torch.empty((n_new, hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(prefill_workspace_bytes(max(n_new, 1), hq, hkv, int(start)), 16),
                                dtype=torch.uint8, device=q.device)
    fk, fv, tk, tv = fmt_k.c(), fmt_v.c(), tables_k.c(), tables_v.c()
    rc = load().tq_prefill_paged(ctypes.byref(fk), ctypes.byref(tk), ctypes.byref(fv),
                                 ctypes.byref(tv), _ptr(q), _dtype_code(q), n_new, hq, hkv, _ptr(k2),
                                 _ptr(v2), _dtype_code(k2), d, int(start), _ptr(codes_k),
                                 _ptr(norms_k), _ptr(codes_v), _ptr(norms_v), page_size, num_pages,
                                 _ptr(block_table), max_blocks, float(scale), _ptr(out),
                                 _ptr(counters), _ptr(workspace), workspace.numel(),
                                 _stream(q.device))
    _check(rc, "tq_prefill_paged")
    return out


def search_workspace_bytes(n_q, k, n_db, d) -> int:
    n = load().tq_search_workspace_bytes(n_q, k, n_db, d)
    if n < 0:
        raise TQError(-2, "tq_search_workspace_bytes")
    return int(n)


def ip_search(queries, codes_db, norms_db, fmt: Format, tables: Tables, k: int = 10,
              workspace=None):
    """Top-k estimated inner products of fp32 queries [n_q, d_in] against a packed database.
    Returns (ids int64 [n_q, k], scores fp32 [n_q, k])."""
    torch = _torch()
    n_q, d_in = queries.shape
    n_db = codes_db.shape[0]
    queries = queries.contiguous()
    if queries.dtype != torch.float32:
        raise TypeError("queries must be fp32")
    ids = torch.empty((n_q, k), dtype=torch.int64, device=queries.device)
    scores = torch.empty((n_q, k), dtype=torch.float32, device=queries.device)
    wsb = search_workspace_bytes(n_q, k, n_db, fmt.d)
    if workspace is None or workspace.numel() < wsb:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=queries.device)
    f, t = fmt.c(), tables.c()
    rc = load().tq_ip_search(ctypes.byref(f), ctypes.byref(t), _ptr(codes_db), _ptr(norms_db),
                             n_db, _ptr(queries), d_in, n_q, k, _ptr(ids), _ptr(scores),
                             _ptr(workspace), workspace.numel(), _stream(queries.device))
    _check(rc, "tq_ip_search")
    return ids, scores


def requantize_workspace_bytes(n, d=128) -> int:
    m = load().tq_requantize_workspace_bytes(n, d)
    if m < 0:
        raise TQError(-2, "tq_requantize_workspace_bytes")
    return int(m)


def requantize(codes_in, norms_in, fmt_in: Format, tables_in: Tables, fmt_out: Format,
               tables_out: Tables, codes_out=None, norms_out=None, counters=None,
               workspace=None):
    """Re-encode stored vectors (codes_in uint8 [n, record_bytes(fmt_in)], norms_in fp16
    [n, 2]) at fmt_out (temporal decay).  Pass codes_out=codes_in / norms_out=norms_in to
    rewrite in place (narrower or equal records only); the records then occupy the first
    n * record_bytes(fmt_out) bytes.  Returns (codes_out, norms_out)."""
    torch = _torch()
    n = norms_in.numel() // 2
    rb_in, rb_out = fmt_in.record_bytes(), fmt_out.record_bytes()
    if codes_in.numel() < n * rb_in:
        raise ValueError("codes_in too small for the norms given")
    if codes_out is None:
        codes_out = torch.empty((n, rb_out), dtype=torch.uint8, device=codes_in.device)
    if norms_out is None:
        norms_out = torch.empty((n, 2), dtype=torch.float16, device=codes_in.device)
    if codes_out.numel() < n * rb_out or norms_out.numel() < 2 * n:
        raise ValueError("output buffers too small")
    if workspace is None:
        workspace = torch.empty(requantize_workspace_bytes(n, fmt_in.d), dtype=torch.uint8,
                                device=codes_in.device)
    fi, ti, fo, to = fmt_in.c(), tables_in.c(), fmt_out.c(), tables_out.c()
    rc = load().tq_requantize(ctypes.byref(fi), ctypes.byref(ti), _ptr(codes_in), _ptr(norms_in),
                              n, ctypes.byref(fo), ctypes.byref(to), _ptr(codes_out),
                              _ptr(norms_out), _ptr(counters), _ptr(workspace), workspace.numel(),
                              _stream(codes_in.device))
    _check(rc, "tq_requantize")
    return codes_out, norms_out
