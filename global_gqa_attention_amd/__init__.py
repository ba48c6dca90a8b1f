"""MiMo-V2.6-Flash attention on AMD Instinct MI355X (gfx950): thin Python binding of libmimo_attn.so.

Every function here only checks shapes and dtypes, allocates outputs with torch (device memory and
streams are torch's), and passes raw pointers to the C ABI declared in ``include/mimo_attn.h``.  All
arithmetic runs in the HIP kernels of ``csrc/``.  There is no fallback: if the library is missing or the
tensors are not on a GPU, the call raises.

Layer (miles docs "MiMo-V2.6-Flash" sections 1, 5.1, 5.4; miles PR "feat(models): add MiMo-V2.6-Flash-RL
support"): GQA with 192-dim Q/K and 128-dim V, V scaled by 0.707, partial RoPE on the first 64 dims
(base 1e4 on sliding-window layers, 1e7 on global layers), sliding window of the query plus 128 previous
keys with a per-head sink on the sliding-window layers, plain causal attention on global layers, THD
packing through cu_seqlens.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmimo_attn.so")
DQK = 192
DV = 128

MIMO_OK = 0
_lib = None


class MimoAttnError(RuntimeError):
    pass


def lib():
    """The loaded C library (loads it on first use; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MimoAttnError(f"{LIB_PATH} is missing: build it with `python -m global_gqa_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_size_t
        L.mimo_attn_fwd.argtypes = [P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32, P, P, P, P, P, sz, P]
        L.mimo_attn_fwd_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mimo_attn_fwd_workspace_size.restype = sz
        L.mimo_attn_bwd_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mimo_attn_bwd_workspace_size_fast.argtypes = [i32, i32, i32, i32, i32, i32]
        L.mimo_attn_bwd_workspace_size_fast.restype = sz
        L.mimo_attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32, P, P, P, P, P, sz, P]
        L.mimo_attn_decode_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mimo_attn_decode.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, f64, i32, i32, P, P, sz, P]
        L.mimo_attn_cache_append.argtypes = [P, P, P, P, i32, i32, i32, f64, P, P, P]
        L.mimo_attn_decode_paged.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, f64, i32, i32, P, P, sz, P]
        L.mimo_attn_prefill_paged.argtypes = [P, P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f64, i32,
                                              i32, P, P, P, sz, P]
        L.mimo_attn_decode_paged_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, f64, i32, i32, P, P]
        L.mimo_attn_verify_workspace_size.argtypes = [i32, i32, i32, i32, i32]
        L.mimo_attn_verify_workspace_size.restype = sz
        L.mimo_attn_verify_paged.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, f64, i32, i32, P, P, sz, P]
        L.mimo_attn_prefill_cached_workspace_size.argtypes = [i32, i32, i32]
        L.mimo_attn_prefill_cached_workspace_size.restype = sz
        L.mimo_attn_prefill_cached.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, f64, i32,
                                               i32, P, P, P, sz, P]
        L.mimo_attn_status_string.argtypes = [ctypes.c_int]
        L.mimo_attn_last_error.argtypes = []
        L.mimo_attn_release.argtypes = []
        L.mimo_attn_trace_enable.argtypes = [ctypes.c_int]
        L.mimo_attn_trace_count.argtypes = []
        L.mimo_attn_trace_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
        L.mimo_attn_trace_clear.argtypes = []
        L.mimo_attn_trace_enable.restype = ctypes.c_int
        L.mimo_attn_trace_count.restype = i32
        L.mimo_attn_trace_read.restype = ctypes.c_int
        L.mimo_attn_trace_clear.restype = None
        for f in ("mimo_attn_fwd", "mimo_attn_bwd", "mimo_attn_decode", "mimo_attn_prefill_cached",
                  "mimo_attn_cache_append", "mimo_attn_decode_paged", "mimo_attn_prefill_paged",
                  "mimo_attn_verify_paged", "mimo_attn_decode_paged_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        L.mimo_attn_bwd_workspace_size.restype = sz
        L.mimo_attn_decode_workspace_size.restype = sz
        L.mimo_attn_status_string.restype = ctypes.c_char_p
        L.mimo_attn_last_error.restype = ctypes.c_char_p
        L.mimo_attn_release.restype = None
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != MIMO_OK:
        L = lib()
        raise MimoAttnError(f"{what}: {L.mimo_attn_status_string(rc).decode()}: {L.mimo_attn_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise MimoAttnError(f"{name} must be on a GPU (there is no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _layer_checks(q, k, v, sink, cu_seqlens):
    _need(q, "q", torch.bfloat16)
    T, hq = q.shape[0], q.shape[1]
    _need(k, "k", torch.bfloat16)
    hkv = k.shape[1]
    _need(q, "q", torch.bfloat16, (T, hq, DQK))
    _need(k, "k", torch.bfloat16, (T, hkv, DQK))
    _need(v, "v", torch.bfloat16, (T, hkv, DV))
    if sink is not None:
        _need(sink, "sink", torch.float32, (hq,))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor of batch+1 entries")
    return T, hq, hkv, cu_seqlens.numel() - 1


def fwd_workspace_size(total_tokens, n_q_heads, n_kv_heads, window) -> int:
    return int(lib().mimo_attn_fwd_workspace_size(int(total_tokens), int(n_q_heads), int(n_kv_heads), int(window)))


def fwd(q, k, v, sink, cu_seqlens, max_seqlen, window, rope_base, out=None, lse=None, return_lse=True,
        workspace=None, q_rot=None, k_rot=None):
    """Forward of one layer.  Returns (out bf16 [T,hq,128], lse fp32 [hq,T] or None).  A given q_rot (bf16
    [T,hq,192]) receives q with RoPE applied, a given k_rot (bf16 [T,hkv,192]) k with RoPE applied, for the
    backward."""
    T, hq, hkv, batch = _layer_checks(q, k, v, sink, cu_seqlens)
    if workspace is None:
        workspace = torch.empty((max(fwd_workspace_size(T, hq, hkv, window), 1),), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((T, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (T, hq, DV))
    if return_lse and lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (hq, T))
    if q_rot is not None:
        _need(q_rot, "q_rot", torch.bfloat16, (T, hq, DQK))
    if k_rot is not None:
        _need(k_rot, "k_rot", torch.bfloat16, (T, hkv, DQK))
    rc = lib().mimo_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(cu_seqlens), batch, T, int(max_seqlen),
                             int(window), float(rope_base), hq, hkv, _ptr(out), _ptr(lse), _ptr(q_rot),
                             _ptr(k_rot), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(rc, "mimo_attn_fwd")
    return out, lse


def bwd_workspace_size(total_tokens, n_q_heads, n_kv_heads, window, batch=None, max_seqlen=None) -> int:
    """Workspace bytes of the backward: the least size (dQ recomputes S and dP) when batch or max_seqlen is not
    given, else the size that selects the stored-dS path (mimo_attn_bwd_workspace_size_fast)."""
    if batch is None or max_seqlen is None:
        return int(lib().mimo_attn_bwd_workspace_size(int(total_tokens), int(n_q_heads), int(n_kv_heads),
                                                      int(window)))
    return int(lib().mimo_attn_bwd_workspace_size_fast(int(total_tokens), int(batch), int(max_seqlen),
                                                       int(n_q_heads), int(n_kv_heads), int(window)))


def bwd(q, k, v, sink, out, lse, dout, cu_seqlens, max_seqlen, window, rope_base, workspace=None, grads=None,
        q_rot=None, k_rot=None):
    """Backward of one layer.  Returns (dq, dk, dv, dsink or None).  Without a workspace one of the fast size
    (stored dS) is allocated; a given workspace selects the path by its size.  q_rot, k_rot: the forward's
    rotated q and k for the same inputs (each saves one of the backward's rotation passes), or None."""
    T, hq, hkv, batch = _layer_checks(q, k, v, sink, cu_seqlens)
    _need(out, "out", torch.bfloat16, (T, hq, DV))
    _need(dout, "dout", torch.bfloat16, (T, hq, DV))
    _need(lse, "lse", torch.float32, (hq, T))
    if grads is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)
        dsink = torch.empty((hq,), dtype=torch.float32, device=q.device) if sink is not None else None
    else:
        dq, dk, dv, dsink = grads
    if workspace is None:
        need = bwd_workspace_size(T, hq, hkv, window, batch, max_seqlen)
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    if q_rot is not None:
        _need(q_rot, "q_rot", torch.bfloat16, (T, hq, DQK))
    if k_rot is not None:
        _need(k_rot, "k_rot", torch.bfloat16, (T, hkv, DQK))
    rc = lib().mimo_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(sink), _ptr(out), _ptr(lse), _ptr(dout), _ptr(q_rot),
                             _ptr(k_rot), _ptr(cu_seqlens), batch, T, int(max_seqlen), int(window), float(rope_base), hq, hkv,
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dsink), _ptr(workspace), workspace.numel(),
                             _stream(q.device))
    _check(rc, "mimo_attn_bwd")
    return dq, dk, dv, dsink


def decode_workspace_size(batch, max_cache_len, n_q_heads, window) -> int:
    return int(lib().mimo_attn_decode_workspace_size(int(batch), int(max_cache_len), int(n_q_heads), int(window)))


def decode(q, k_new, v_new, k_cache, v_cache, cu_cache, positions, sink, max_cache_len, window, rope_base,
           out=None, workspace=None):
    """One decode step.  Returns out bf16 [batch, hq, 128]."""
    _need(q, "q", torch.bfloat16)
    B, hq = q.shape[0], q.shape[1]
    hkv = k_new.shape[1]
    _need(q, "q", torch.bfloat16, (B, hq, DQK))
    _need(k_new, "k_new", torch.bfloat16, (B, hkv, DQK))
    _need(v_new, "v_new", torch.bfloat16, (B, hkv, DV))
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16)
    if k_cache.dim() != 3 or k_cache.shape[1:] != (hkv, DQK) or v_cache.shape != (k_cache.shape[0], hkv, DV):
        raise ValueError("cache shapes must be [rows, n_kv_heads, 192] and [rows, n_kv_heads, 128]")
    _need(cu_cache, "cu_cache", torch.int32, (B + 1,))
    _need(positions, "positions", torch.int32, (B,))
    if sink is not None:
        _need(sink, "sink", torch.float32, (hq,))
    if out is None:
        out = torch.empty((B, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, hq, DV))
    need = decode_workspace_size(B, max_cache_len, hq, window)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    rc = lib().mimo_attn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(cu_cache),
                                _ptr(positions), _ptr(sink), B, int(max_cache_len), int(window), float(rope_base),
                                hq, hkv, _ptr(out), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(rc, "mimo_attn_decode")
    return out


def prefill_cached_workspace_size(total_tokens, total_cache, n_kv_heads) -> int:
    return int(lib().mimo_attn_prefill_cached_workspace_size(int(total_tokens), int(total_cache), int(n_kv_heads)))


def prefill_cached(q, k, v, k_cache, v_cache, sink, cu_seqlens, cu_cache, positions, max_seqlen, max_position,
                   window, rope_base, out=None, lse=None, return_lse=True, workspace=None):
    """Prefill of new tokens (q, k, v THD-packed by cu_seqlens) over cached prefixes (k_cache rotated, v_cache,
    rows of sequence b: cu_cache[b] .. cu_cache[b+1]-1; first new token at positions[b]).  Returns (out bf16
    [T,hq,128], lse fp32 [hq,T] or None)."""
    T, hq, hkv, batch = _layer_checks(q, k, v, sink, cu_seqlens)
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(v_cache, "v_cache", torch.bfloat16)
    Tc = k_cache.shape[0]
    _need(k_cache, "k_cache", torch.bfloat16, (Tc, hkv, DQK))
    _need(v_cache, "v_cache", torch.bfloat16, (Tc, hkv, DV))
    _need(cu_cache, "cu_cache", torch.int32, (batch + 1,))
    _need(positions, "positions", torch.int32, (batch,))
    if workspace is None:
        workspace = torch.empty((max(prefill_cached_workspace_size(T, Tc, hkv), 1),), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((T, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (T, hq, DV))
    if return_lse and lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (hq, T))
    rc = lib().mimo_attn_prefill_cached(_ptr(q), _ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(sink),
                                        _ptr(cu_seqlens), _ptr(cu_cache), _ptr(positions), batch, T, Tc,
                                        int(max_seqlen), int(max_position), int(window), float(rope_base), hq, hkv,
                                        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(rc, "mimo_attn_prefill_cached")
    return out, lse


def _pool_checks(k_pool, v_pool, hkv):
    _need(k_pool, "k_pool", torch.bfloat16)
    _need(v_pool, "v_pool", torch.bfloat16)
    P = k_pool.shape[0]
    _need(k_pool, "k_pool", torch.bfloat16, (P, hkv, DQK))
    _need(v_pool, "v_pool", torch.bfloat16, (P, hkv, DV))
    return P


def cache_append(k, v, positions, slots, k_pool, v_pool, rope_base):
    """Rotate k (bf16 [n, hkv, 192]) at positions (int32 [n]) and store it with v in pool rows slots (int32 [n])."""
    _need(k, "k", torch.bfloat16)
    n, hkv = k.shape[0], k.shape[1]
    _need(k, "k", torch.bfloat16, (n, hkv, DQK))
    _need(v, "v", torch.bfloat16, (n, hkv, DV))
    _need(positions, "positions", torch.int32, (n,))
    _need(slots, "slots", torch.int32, (n,))
    P = _pool_checks(k_pool, v_pool, hkv)
    rc = lib().mimo_attn_cache_append(_ptr(k), _ptr(v), _ptr(positions), _ptr(slots), n, hkv, P, float(rope_base),
                                      _ptr(k_pool), _ptr(v_pool), _stream(k.device))
    _check(rc, "mimo_attn_cache_append")


def decode_paged(q, k_new, v_new, k_pool, v_pool, page_table, cu_pages, positions, sink, max_cache_len, window,
                 rope_base, out=None, workspace=None):
    """Decode over a paged cache (cache row r of sequence b = pool row page_table[cu_pages[b] + r])."""
    _need(q, "q", torch.bfloat16)
    B, hq = q.shape[0], q.shape[1]
    hkv = k_new.shape[1]
    _need(q, "q", torch.bfloat16, (B, hq, DQK))
    _need(k_new, "k_new", torch.bfloat16, (B, hkv, DQK))
    _need(v_new, "v_new", torch.bfloat16, (B, hkv, DV))
    _pool_checks(k_pool, v_pool, hkv)
    _need(page_table, "page_table", torch.int32)
    _need(cu_pages, "cu_pages", torch.int32, (B + 1,))
    _need(positions, "positions", torch.int32, (B,))
    if sink is not None:
        _need(sink, "sink", torch.float32, (hq,))
    if out is None:
        out = torch.empty((B, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, hq, DV))
    if workspace is None:
        workspace = torch.empty((max(decode_workspace_size(B, max_cache_len, hq, window), 1),), dtype=torch.uint8,
                                device=q.device)
    rc = lib().mimo_attn_decode_paged(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                      _ptr(cu_pages), _ptr(positions), _ptr(sink), B, int(max_cache_len), int(window),
                                      float(rope_base), hq, hkv, _ptr(out), _ptr(workspace), workspace.numel(),
                                      _stream(q.device))
    _check(rc, "mimo_attn_decode_paged")
    return out


def decode_paged_noalloc(q, k_new, v_new, k_pool, v_pool, page_table, cu_pages, positions, sink, max_cache_len,
                         window, rope_base, out):
    """decode_paged with no workspace (the library's per-device scratch array holds the split partials): for
    callers that cannot allocate.  `out` (bf16 [batch, hq, 128]) must be given; nothing is allocated here."""
    _need(q, "q", torch.bfloat16)
    B, hq = q.shape[0], q.shape[1]
    hkv = k_new.shape[1]
    _need(q, "q", torch.bfloat16, (B, hq, DQK))
    _need(k_new, "k_new", torch.bfloat16, (B, hkv, DQK))
    _need(v_new, "v_new", torch.bfloat16, (B, hkv, DV))
    _pool_checks(k_pool, v_pool, hkv)
    _need(page_table, "page_table", torch.int32)
    _need(cu_pages, "cu_pages", torch.int32, (B + 1,))
    _need(positions, "positions", torch.int32, (B,))
    if sink is not None:
        _need(sink, "sink", torch.float32, (hq,))
    _need(out, "out", torch.bfloat16, (B, hq, DV))
    rc = lib().mimo_attn_decode_paged_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                              _ptr(page_table), _ptr(cu_pages), _ptr(positions), _ptr(sink), B,
                                              int(max_cache_len), int(window), float(rope_base), hq, hkv, _ptr(out),
                                              _stream(q.device))
    _check(rc, "mimo_attn_decode_paged_noalloc")
    return out


def prefill_paged(q, k, v, k_pool, v_pool, page_table, sink, cu_seqlens, cu_pages, positions, max_seqlen, max_position,
                  window, rope_base, out=None, lse=None, return_lse=True, workspace=None):
    """prefill_cached over a paged cache (the multi-token verify step with short chunks)."""
    T, hq, hkv, batch = _layer_checks(q, k, v, sink, cu_seqlens)
    _pool_checks(k_pool, v_pool, hkv)
    _need(page_table, "page_table", torch.int32)
    _need(cu_pages, "cu_pages", torch.int32, (batch + 1,))
    _need(positions, "positions", torch.int32, (batch,))
    npg = page_table.numel()
    if workspace is None:
        workspace = torch.empty((max(prefill_cached_workspace_size(T, npg, hkv), 1),), dtype=torch.uint8,
                                device=q.device)
    if out is None:
        out = torch.empty((T, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (T, hq, DV))
    if return_lse and lse is None:
        lse = torch.empty((hq, T), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (hq, T))
    rc = lib().mimo_attn_prefill_paged(_ptr(q), _ptr(k), _ptr(v), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                       _ptr(sink), _ptr(cu_seqlens), _ptr(cu_pages), _ptr(positions), batch, T, npg,
                                       int(max_seqlen), int(max_position), int(window), float(rope_base), hq, hkv,
                                       _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(rc, "mimo_attn_prefill_paged")
    return out, lse


def verify_workspace_size(batch, n_query, max_cache_len, n_q_heads, window) -> int:
    return int(lib().mimo_attn_verify_workspace_size(int(batch), int(n_query), int(max_cache_len), int(n_q_heads),
                                                     int(window)))


def verify_paged(q, k_pool, v_pool, page_table, cu_pages, positions, sink, n_query, max_cache_len, window, rope_base,
                 out=None, workspace=None):
    """Verify n_query draft tokens per sequence (their keys already appended as the last n_query entries of
    each page-table list).  q: bf16 [batch * n_query, hq, 192].  Returns out bf16 [batch * n_query, hq, 128]."""
    _need(q, "q", torch.bfloat16)
    R, hq = q.shape[0], q.shape[1]
    if n_query < 1 or R % n_query:
        raise ValueError("q must hold n_query rows per sequence")
    B = R // n_query
    hkv = k_pool.shape[1] if k_pool.dim() == 3 else 0
    _need(q, "q", torch.bfloat16, (R, hq, DQK))
    _pool_checks(k_pool, v_pool, hkv)
    _need(page_table, "page_table", torch.int32)
    _need(cu_pages, "cu_pages", torch.int32, (B + 1,))
    _need(positions, "positions", torch.int32, (B,))
    if sink is not None:
        _need(sink, "sink", torch.float32, (hq,))
    if out is None:
        out = torch.empty((R, hq, DV), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (R, hq, DV))
    if workspace is None:
        workspace = torch.empty((max(verify_workspace_size(B, n_query, max_cache_len, hq, window), 1),),
                                dtype=torch.uint8, device=q.device)
    rc = lib().mimo_attn_verify_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(cu_pages),
                                      _ptr(positions), _ptr(sink), B, int(n_query), int(max_cache_len), int(window),
                                      float(rope_base), hq, hkv, _ptr(out), _ptr(workspace), workspace.numel(),
                                      _stream(q.device))
    _check(rc, "mimo_attn_verify_paged")
    return out


def release():
    """Free the library's cached RoPE tables."""
    lib().mimo_attn_release()


def trace_enable(on: bool = True):
    """Record a HIP event pair around every kernel the library launches (on the caller's stream)."""
    _check(lib().mimo_attn_trace_enable(1 if on else 0), "mimo_attn_trace_enable")


def trace_read(clear: bool = True):
    """[(kernel name, milliseconds)] for every kernel launched while tracing was on (waits for them)."""
    L = lib()
    out = []
    for i in range(L.mimo_attn_trace_count()):
        name, ms = ctypes.c_char_p(), ctypes.c_float()
        _check(L.mimo_attn_trace_read(i, ctypes.byref(name), ctypes.byref(ms)), "mimo_attn_trace_read")
        out.append((name.value.decode(), float(ms.value)))
    if clear:
        L.mimo_attn_trace_clear()
    return out
