"""CPU oracle for the paged KV-cache decode operator (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never does; the two share no code.

The arithmetic lives in ``oracle.cpp`` (plain fp64 C++17, built into
``liboracle.so`` by :func:`build`); this module only marshals numpy arrays.
Each routine cites the page passage it follows in ``oracle.cpp``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# dtype codes of this module's C interface
F16, BF16, E4M3 = 0, 1, 2
_DTYPE_CODES = {"f16": F16, "bf16": BF16, "e4m3": E4M3}


def dtype_code(name: str) -> int:
    return _DTYPE_CODES[name]


def build(force: bool = True) -> str:
    """Compile liboracle.so with g++ (no GPU toolchain involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        c = ctypes
        vp, i32p, dp = c.c_void_p, c.POINTER(c.c_int32), c.c_void_p
        L.or_f16_to_f64.argtypes = [c.c_uint16]; L.or_f16_to_f64.restype = c.c_double
        L.or_bf16_to_f64.argtypes = [c.c_uint16]; L.or_bf16_to_f64.restype = c.c_double
        L.or_e4m3_to_f64.argtypes = [c.c_uint8]; L.or_e4m3_to_f64.restype = c.c_double
        L.or_f64_to_f16.argtypes = [c.c_double]; L.or_f64_to_f16.restype = c.c_uint16
        L.or_f64_to_bf16.argtypes = [c.c_double]; L.or_f64_to_bf16.restype = c.c_uint16
        L.or_f32_to_e4m3.argtypes = [c.c_float]; L.or_f32_to_e4m3.restype = c.c_uint8
        L.or_f64_to_dtype_array.argtypes = [vp, c.c_size_t, c.c_int, vp]
        L.or_dequant_array.argtypes = [vp, c.c_size_t, c.c_int, c.c_float, vp]
        L.or_build_tables.argtypes = [vp, vp, c.c_int32, c.c_int32, vp, vp, vp, c.c_int32,
                                      c.c_int32, vp, vp, c.c_int32]
        L.or_build_tables.restype = c.c_int
        L.or_free_rows.argtypes = [vp, vp, vp, c.c_int32, c.c_int32, vp, vp]
        L.or_scatter.argtypes = [vp, c.c_int, vp, c.c_int, vp, c.c_int32, vp, vp, c.c_int32,
                                 c.c_int32, c.c_int32, c.c_int32, c.c_float]
        dec = [vp, c.c_int, vp, vp, c.c_int, c.c_float, c.c_float, vp, vp,
               c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_int32, c.c_float]
        L.or_decode.argtypes = dec + [vp, c.c_int32, c.c_int32, vp, vp]
        L.or_decode_online.argtypes = dec + [vp, vp]
        L.or_decode_partitioned.argtypes = dec + [c.c_int32, vp]
        L.or_decode_multi.argtypes = dec + [c.c_int32, vp, c.c_int32, vp]
        L.or_kv_bytes_per_token.argtypes = [c.c_int32] * 4
        L.or_kv_bytes_per_token.restype = c.c_uint64
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- conversions
def f16_to_f64(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().or_dequant_array(_p(bits), bits.size, F16, 1.0, _p(out))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().or_dequant_array(_p(bits), bits.size, BF16, 1.0, _p(out))
    return out


def e4m3_to_f64(bits, scale: float = 1.0) -> np.ndarray:
    """Dequantize e4m3 codes: float(code value) * float(scale) in binary32, widened."""
    bits = _c(bits, np.uint8)
    out = np.empty(bits.shape, np.float64)
    lib().or_dequant_array(_p(bits), bits.size, E4M3, float(scale), _p(out))
    return out


def to_f64(bits, dtype: int, scale: float = 1.0) -> np.ndarray:
    if dtype == F16:
        return f16_to_f64(bits)
    if dtype == BF16:
        return bf16_to_f64(bits)
    return e4m3_to_f64(bits, scale)


def round_to(x, dtype: int) -> np.ndarray:
    """fp64 -> dtype bits, round to nearest even (e4m3: via binary32, saturating)."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8 if dtype == E4M3 else np.uint16)
    lib().or_f64_to_dtype_array(_p(x), x.size, dtype, _p(out))
    return out


def f32_to_e4m3(x) -> np.ndarray:
    x = _c(x, np.float32).astype(np.float64)  # exact widening; encoder narrows back to binary32
    return round_to(x, E4M3)


# ---------------------------------------------------------------- block tables
def build_tables(num_blocks: int, block_size: int, free_order, context_lens, max_blocks: int,
                 prefix_group=None, prefix_lens=None):
    """O1.  Returns (status, tables[S, MB], refcounts[NB], remaining free list)."""
    fl = _c(free_order, np.int32).copy()
    cnt = np.array([fl.size], np.int32)
    ctx = _c(context_lens, np.int32)
    S = ctx.size
    pg = None if prefix_group is None else _c(prefix_group, np.int32)
    pl = None if prefix_lens is None else _c(prefix_lens, np.int32)
    ng = 0 if pl is None else pl.size
    tables = np.full((S, max_blocks), -1, np.int32)
    ref = np.zeros(num_blocks, np.int32)
    st = lib().or_build_tables(_p(fl), _p(cnt), block_size, S, _p(ctx), _p(pg), _p(pl), ng,
                               max_blocks, _p(tables), _p(ref), num_blocks)
    return st, tables, ref, fl[: cnt[0]].copy()


def free_rows(free_list, tables, rows, refcounts, num_blocks: int):
    """Release table rows; returns (new free list, new refcounts)."""
    fl = np.empty(num_blocks, np.int32)
    fl[: len(free_list)] = free_list
    cnt = np.array([len(free_list)], np.int32)
    ref = _c(refcounts, np.int32).copy()
    t = _c(tables, np.int32)
    r = _c(rows, np.int32)
    lib().or_free_rows(_p(fl), _p(cnt), _p(t), t.shape[1], r.size, _p(r), _p(ref))
    return fl[: cnt[0]].copy(), ref


# ---------------------------------------------------------------- scatter
def scatter(src_bits, src_dtype: int, cache, cache_dtype: int, tables, seq_ids, positions,
            block_size: int, inv_scale: float = 1.0):
    """O2, in place on `cache` ([NB, Hkv, B, d] bits)."""
    src_bits = _c(src_bits, np.uint16)
    T, Hkv, d = src_bits.shape
    assert cache.flags.c_contiguous
    t = _c(tables, np.int32)
    lib().or_scatter(_p(src_bits), src_dtype, _p(cache), cache_dtype, _p(t), t.shape[1],
                     _p(_c(seq_ids, np.int32)), _p(_c(positions, np.int32)), T, Hkv, d,
                     block_size, float(inv_scale))
    return cache


# ---------------------------------------------------------------- decode
def _dec_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables, context_lens,
              num_kv_heads, block_size, scale):
    q = np.ascontiguousarray(q)
    S, Hq, d = q.shape
    t = _c(tables, np.int32)
    ctx = _c(context_lens, np.int32)
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    return (q, t, ctx), [_p(q), q_dtype, _p(k_cache), _p(v_cache), kv_dtype, float(k_scale),
                         float(v_scale), _p(t), _p(ctx), S, Hq, num_kv_heads, d, block_size,
                         t.shape[1], float(scale)]


def decode(q, q_dtype, k_cache, v_cache, kv_dtype, tables, context_lens, num_kv_heads,
           block_size, scale, k_scale=1.0, v_scale=1.0, rows=None, threads=None,
           want_weights=False):
    """O4.  Returns out [S, Hq, d] fp64 (only `rows` filled when given; NaN elsewhere)
    and, if asked, the weights [S, Hq, MB*B]."""
    keep, args = _dec_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables,
                           context_lens, num_kv_heads, block_size, scale)
    S, Hq, d = keep[0].shape
    MB = keep[1].shape[1]
    out = np.full((S, Hq, d), np.nan)
    w = np.zeros((S, Hq, MB * block_size)) if want_weights else None
    rr = None if rows is None else _c(rows, np.int32).reshape(-1, 2)
    nthreads = threads if threads is not None else (os.cpu_count() or 1)
    lib().or_decode(*args, _p(rr), 0 if rr is None else rr.shape[0], nthreads, _p(out), _p(w))
    return (out, w) if want_weights else out


def decode_online(q, q_dtype, k_cache, v_cache, kv_dtype, tables, context_lens, num_kv_heads,
                  block_size, scale, k_scale=1.0, v_scale=1.0, block_orders=None):
    keep, args = _dec_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables,
                           context_lens, num_kv_heads, block_size, scale)
    S, Hq, d = keep[0].shape
    out = np.zeros((S, Hq, d))
    bo = None if block_orders is None else _c(block_orders, np.int32)
    lib().or_decode_online(*args, _p(bo), _p(out))
    return out


def decode_partitioned(q, q_dtype, k_cache, v_cache, kv_dtype, tables, context_lens,
                       num_kv_heads, block_size, scale, partition_size, k_scale=1.0,
                       v_scale=1.0):
    keep, args = _dec_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, tables,
                           context_lens, num_kv_heads, block_size, scale)
    S, Hq, d = keep[0].shape
    out = np.zeros((S, Hq, d))
    lib().or_decode_partitioned(*args, int(partition_size), _p(out))
    return out


def decode_multi(q, q_dtype, k_cache, v_cache, kv_dtype, tables, context_lens, num_kv_heads,
                 block_size, scale, k_scale=1.0, v_scale=1.0, tree_masks=None, threads=None):
    """Multi-token queries q [S, T, Hq, d] (the last T positions of each sequence);
    tree_masks [S, T] uint32 or None (causal).  Returns out [S, T, Hq, d] fp64."""
    q = np.ascontiguousarray(q)
    S, T, Hq, d = q.shape
    keep, args = _dec_args(q.reshape(S, T * Hq, d), q_dtype, k_cache, v_cache, kv_dtype,
                           k_scale, v_scale, tables, context_lens, num_kv_heads, block_size,
                           scale)
    args[10] = Hq  # _dec_args read Hq from the flattened shape
    tm = None if tree_masks is None else _c(tree_masks, np.uint32).reshape(S, T)
    out = np.zeros((S, T, Hq, d))
    nthreads = threads if threads is not None else (os.cpu_count() or 1)
    lib().or_decode_multi(*args, int(T), _p(tm), nthreads, _p(out))
    return out


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, kv_dtype: int) -> int:
    return int(lib().or_kv_bytes_per_token(num_layers, num_kv_heads, head_dim, kv_dtype))
