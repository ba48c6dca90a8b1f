"""fp64 CPU oracle for the MiMo-V2.6-Flash attention layer (test infrastructure only).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may import this package.  The
arithmetic lives in ``mimo_oracle.c`` (plain C, IEEE double); this module builds it with gcc and marshals
numpy / torch-CPU arrays into it.  It imports nothing from the HIP library and the HIP library imports
nothing from it.

Sources (titles of the pages the oracle follows, with the section):
  * miles pull request "feat(models): add MiMo-V2.6-Flash-RL support" -- PR body and commit messages:
    per-layer KV heads, 192/128 head dims, sink on sliding-window layers, V scaled by 0.707,
    129-key window (query + 128 previous keys).
  * miles docs "MiMo-V2.6-Flash" -- section 1 (hybrid attention, RoPE bases, partial RoPE 64 of 192),
    section 5.1 (THD packing), section 5.4 (window_size = (128, 0)).
  * Megatron-Bridge API docs "mimo_v2_flash_bridge" -- module summary (partial rotary, dual bases).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mimo_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmimo_oracle.so")
_lib = None

DQK = 192
DV = 128


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/libmimo_oracle.so (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-D_GNU_SOURCE",
               _SRC, "-o", tmp, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_prefill_rows.argtypes = [P, P, P, P, P, i32, i64, i32, f64, i32, i32, P, i64, P, P, i32, i32]
        lib.oracle_prefill_bwd.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, f64, i32, i32, P, P, P, P, i32,
                                           i32]
        lib.oracle_bwd_dq_rows.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, f64, i32, i32, P, i64, P, i32, i32]
        lib.oracle_bwd_dkv_rows.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, f64, i32, i32, P, i64, P, P, i32,
                                            i32]
        lib.oracle_bwd_dsink_heads.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, f64, i32, i32, P, i32, P, i32,
                                               i32]
        lib.oracle_decode_rows.argtypes = [P, P, P, P, P, P, P, P, i32, i32, f64, i32, i32, P, i64, P, P, i32,
                                           i32]
        lib.oracle_prefill_cached_rows.argtypes = [P, P, P, P, P, P, P, P, P, i32, i32, f64, i32, i32, P, i64,
                                                   P, P, i32, i32]
        lib.oracle_rope.argtypes = [P, P, i64, f64, i32, P]
        for name in ("oracle_prefill_rows", "oracle_prefill_bwd", "oracle_bwd_dq_rows", "oracle_bwd_dkv_rows",
                     "oracle_bwd_dsink_heads", "oracle_decode_rows", "oracle_prefill_cached_rows", "oracle_rope"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
    return _lib


# ----------------------------------------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------------------------------------
def _elem(x):
    """(array, f64 flag) for a tensor argument: bf16 data becomes uint16 bit patterns (flag 0), float64 data
    stays float64 (flag 1).  Accepts torch tensors (any device) and numpy arrays."""
    if isinstance(x, np.ndarray):
        if x.dtype == np.uint16:
            return np.ascontiguousarray(x), 0
        if x.dtype == np.float64:
            return np.ascontiguousarray(x), 1
        raise TypeError("numpy data must be uint16 bf16 bit patterns or float64")
    import torch  # local: the oracle itself needs no torch

    if x.dtype == torch.bfloat16:
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16), 0
    if x.dtype == torch.float64:
        return x.detach().cpu().contiguous().numpy(), 1
    raise TypeError(f"expected bfloat16 or float64, got {x.dtype}")


def _same(*pairs):
    """Arrays of several tensors that must share one element type; returns (arrays..., flag)."""
    arrs, flags = [], set()
    for p in pairs:
        if p is None:
            arrs.append(None)
            continue
        a, f = _elem(p)
        arrs.append(a)
        flags.add(f)
    if len(flags) > 1:
        raise TypeError("all tensors of one call must be bf16, or all float64")
    return (*arrs, flags.pop() if flags else 0)


def bf16_bits(x) -> np.ndarray:
    a, f = _elem(x)
    if f:
        raise TypeError("expected bf16 data")
    return a


def _f64(x):
    if x is None:
        return None
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.float64)
    return x.detach().cpu().contiguous().double().numpy()


def _i32(x):
    if isinstance(x, np.ndarray):
        return np.ascontiguousarray(x, dtype=np.int32)
    if hasattr(x, "detach"):
        return x.detach().cpu().contiguous().numpy().astype(np.int32)
    return np.ascontiguousarray(np.asarray(x), dtype=np.int32)


def _i64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.int64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle rejected the arguments (rc={rc})")


def _layer(q, k, v, sink, cu_seqlens, dout=None, out_given=None):
    qb, kb, vb, dob, og, f64 = _same(q, k, v, dout, out_given)
    cu = _i32(cu_seqlens)
    T = qb.shape[0]
    hq, hkv = qb.shape[1], kb.shape[1]
    if qb.shape[2] != DQK or kb.shape[2] != DQK or vb.shape[2] != DV:
        raise ValueError("head dims must be 192 (Q/K) and 128 (V)")
    return qb, kb, vb, dob, og, f64, _f64(sink), cu, len(cu) - 1, T, hq, hkv


# ----------------------------------------------------------------------------------------------------------
# public oracle functions.  Tensors are bf16 (torch or uint16 numpy) or float64 (all of one call alike);
# sink is any float array of n_q_heads values (used in fp64) or None.
# ----------------------------------------------------------------------------------------------------------
def prefill_rows(q, k, v, sink, cu_seqlens, window, rope_base, rows=None, nthreads=0):
    """Forward rows.  rows: None (all, in token-major order) or an int array of token*n_q_heads + head.
    Returns (out [n,128] fp64, lse [n] fp64)."""
    qb, kb, vb, _, _, f64, sk, cu, B, T, hq, hkv = _layer(q, k, v, sink, cu_seqlens)
    r = None if rows is None else _i64(rows)
    n = T * hq if r is None else len(r)
    out = np.zeros((n, DV), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_prefill_rows(_p(qb), _p(kb), _p(vb), _p(sk), _p(cu), B, T, int(window), float(rope_base),
                                     hq, hkv, _p(r), n, _p(out), _p(lse), f64, int(nthreads))
    _check(rc, "prefill_rows")
    return out, lse


def prefill(q, k, v, sink, cu_seqlens, window, rope_base, nthreads=0):
    """Full forward: out [T,hq,128], lse [hq,T] (fp64)."""
    T, hq = q.shape[0], q.shape[1]
    out, lse = prefill_rows(q, k, v, sink, cu_seqlens, window, rope_base, None, nthreads)
    return out.reshape(T, hq, DV), lse.reshape(T, hq).T.copy()


def prefill_bwd(q, k, v, sink, dout, cu_seqlens, window, rope_base, out_given=None, nthreads=0):
    """Full backward.  out_given: the O used for D = dO.O, or None for the exact O.
    Returns dq [T,hq,192], dk [T,hkv,192], dv [T,hkv,128], dsink [hq] or None (fp64)."""
    qb, kb, vb, dob, og, f64, sk, cu, B, T, hq, hkv = _layer(q, k, v, sink, cu_seqlens, dout, out_given)
    dq = np.zeros((T, hq, DQK), np.float64)
    dk = np.zeros((T, hkv, DQK), np.float64)
    dv = np.zeros((T, hkv, DV), np.float64)
    ds = np.zeros((hq,), np.float64) if sk is not None else None
    rc = _load().oracle_prefill_bwd(_p(qb), _p(kb), _p(vb), _p(sk), _p(og), _p(dob), _p(cu), B, T, int(window),
                                    float(rope_base), hq, hkv, _p(dq), _p(dk), _p(dv), _p(ds), f64, int(nthreads))
    _check(rc, "prefill_bwd")
    return dq, dk, dv, ds


def bwd_dq_rows(q, k, v, sink, dout, cu_seqlens, window, rope_base, rows, out_given=None, nthreads=0):
    """dq for rows token*n_q_heads + head: [n,192] fp64."""
    qb, kb, vb, dob, og, f64, sk, cu, B, T, hq, hkv = _layer(q, k, v, sink, cu_seqlens, dout, out_given)
    r = _i64(rows)
    dq = np.zeros((len(r), DQK), np.float64)
    rc = _load().oracle_bwd_dq_rows(_p(qb), _p(kb), _p(vb), _p(sk), _p(og), _p(dob), _p(cu), B, T, int(window),
                                    float(rope_base), hq, hkv, _p(r), len(r), _p(dq), f64, int(nthreads))
    _check(rc, "bwd_dq_rows")
    return dq


def bwd_dkv_rows(q, k, v, sink, dout, cu_seqlens, window, rope_base, key_rows, out_given=None, nthreads=0):
    """dk, dv for key rows token*n_kv_heads + kv head: ([n,192], [n,128]) fp64."""
    qb, kb, vb, dob, og, f64, sk, cu, B, T, hq, hkv = _layer(q, k, v, sink, cu_seqlens, dout, out_given)
    r = _i64(key_rows)
    dk = np.zeros((len(r), DQK), np.float64)
    dv = np.zeros((len(r), DV), np.float64)
    rc = _load().oracle_bwd_dkv_rows(_p(qb), _p(kb), _p(vb), _p(sk), _p(og), _p(dob), _p(cu), B, T, int(window),
                                     float(rope_base), hq, hkv, _p(r), len(r), _p(dk), _p(dv), f64, int(nthreads))
    _check(rc, "bwd_dkv_rows")
    return dk, dv


def bwd_dsink_heads(q, k, v, sink, dout, cu_seqlens, window, rope_base, heads, out_given=None, nthreads=0):
    """dsink for the listed Q heads (summed over every token): [n] fp64."""
    qb, kb, vb, dob, og, f64, sk, cu, B, T, hq, hkv = _layer(q, k, v, sink, cu_seqlens, dout, out_given)
    hs = _i32(heads)
    ds = np.zeros((len(hs),), np.float64)
    rc = _load().oracle_bwd_dsink_heads(_p(qb), _p(kb), _p(vb), _p(sk), _p(og), _p(dob), _p(cu), B, T,
                                        int(window), float(rope_base), hq, hkv, _p(hs), len(hs), _p(ds), f64,
                                        int(nthreads))
    _check(rc, "bwd_dsink_heads")
    return ds


def decode_rows(q, k_new, v_new, k_cache, v_cache, cu_cache, positions, sink, window, rope_base, rows=None,
                nthreads=0):
    """Decode.  rows: None (all b*hq+h) or a list.  Returns (out [n,128], lse [n]) in fp64."""
    qb, knb, vnb, kcb, vcb, f64 = _same(q, k_new, v_new, k_cache, v_cache)
    cuc, pos, sk = _i32(cu_cache), _i32(positions), _f64(sink)
    B, hq, hkv = qb.shape[0], qb.shape[1], knb.shape[1]
    r = None if rows is None else _i64(rows)
    n = B * hq if r is None else len(r)
    out = np.zeros((n, DV), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_decode_rows(_p(qb), _p(knb), _p(vnb), _p(kcb), _p(vcb), _p(cuc), _p(pos), _p(sk), B,
                                    int(window), float(rope_base), hq, hkv, _p(r), n, _p(out), _p(lse), f64,
                                    int(nthreads))
    _check(rc, "decode_rows")
    return out, lse


def prefill_cached_rows(q, k, v, k_cache, v_cache, cu_seqlens_q, cu_cache, positions, sink, window, rope_base,
                        rows=None, nthreads=0):
    """Prefill of new tokens over a cached prefix.  rows: None (all t*hq+h) or a list.  Returns (out [n,128],
    lse [n]) in fp64."""
    qb, kb, vb, kcb, vcb, f64 = _same(q, k, v, k_cache, v_cache)
    cuq, cuc, pos, sk = _i32(cu_seqlens_q), _i32(cu_cache), _i32(positions), _f64(sink)
    T, hq, hkv = qb.shape[0], qb.shape[1], kb.shape[1]
    B = len(cuq) - 1
    r = None if rows is None else _i64(rows)
    n = T * hq if r is None else len(r)
    out = np.zeros((n, DV), np.float64)
    lse = np.zeros((n,), np.float64)
    rc = _load().oracle_prefill_cached_rows(_p(qb), _p(kb), _p(vb), _p(kcb), _p(vcb), _p(cuq), _p(cuc), _p(pos),
                                            _p(sk), B, int(window), float(rope_base), hq, hkv, _p(r), n, _p(out),
                                            _p(lse), f64, int(nthreads))
    _check(rc, "prefill_cached_rows")
    return out, lse


def rope(x, positions, rope_base):
    """Rotate rows of 192 values (shape [n,192], bf16 or float64) at the given positions; fp64 [n,192]."""
    xb, f64 = _elem(x)
    xb = xb.reshape(-1, DQK)
    pos = _i32(positions)
    out = np.zeros(xb.shape, np.float64)
    _check(_load().oracle_rope(_p(xb), _p(pos), xb.shape[0], float(rope_base), f64, _p(out)), "rope")
    return out
