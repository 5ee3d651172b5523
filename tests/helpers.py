"""Test-side helpers: build oracle inputs from a seeded case and compare results."""
from __future__ import annotations

import os

import numpy as np

import oracle
import workloads

DT = {"f16": oracle.F16, "bf16": oracle.BF16, "e4m3": oracle.E4M3}


def oracle_tables(case):
    sp = case.spec
    st, tables, ref, free_left = oracle.build_tables(
        sp.num_blocks, sp.block_size, case.free_order, case.context_lens, sp.max_blocks,
        case.prefix_group, case.prefix_lens)
    assert st == 0, st
    return tables, ref, free_left


def oracle_caches(case, tables, poison=True):
    """K and V pools filled by the oracle scatter from the case's token writes."""
    sp = case.spec
    k = workloads.empty_cache(sp, poison)
    v = workloads.empty_cache(sp, poison)
    src = DT[sp.src_dtype]
    dst = DT[sp.kv_dtype]
    oracle.scatter(case.k_src, src, k, dst, tables, case.seq_ids, case.positions, sp.block_size,
                   case.k_inv_scale)
    oracle.scatter(case.v_src, src, v, dst, tables, case.seq_ids, case.positions, sp.block_size,
                   case.v_inv_scale)
    return k, v


def oracle_decode(case, tables, k, v, **kw):
    sp = case.spec
    return oracle.decode(case.q, DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables, case.context_lens,
                         sp.num_kv_heads, sp.block_size, sp.scale, case.k_scale, case.v_scale, **kw)


def half_ulp(r: np.ndarray, dtype: str | None) -> np.ndarray:
    """Half a unit in the last place of `dtype` at |r| (0 when dtype is None): the most
    that the final round-to-nearest into the output dtype can move a result."""
    if dtype is None:
        return np.zeros_like(r)
    mant, emin = {"f16": (10, -14), "bf16": (7, -126)}[dtype]
    a = np.abs(r)
    with np.errstate(divide="ignore"):
        e = np.where(a > 0, np.floor(np.log2(np.where(a > 0, a, 1.0))), emin)
    e = np.maximum(e, emin)
    return np.ldexp(1.0, (e - mant - 1).astype(np.int64))


def compare(gpu_out_f64: np.ndarray, ref_f64: np.ndarray, atol: float, rtol_row: float | None,
            out_dtype: str | None = None):
    """Tolerance gates against the unrounded fp64 oracle.

    Gate 1: |g - r| <= atol for every element (2e-3 for fp16/bf16 caches, 2e-2 for
    e4m3), with one allowance: a bf16 output also gets half an ulp of bf16 at |r|, since the
    final round-to-nearest into bf16 alone moves a result by up to 2^-9 |r|, more than 2e-3
    once |r| > 1.  fp16 outputs (half an ulp <= 4.9e-4 below |r| = 2) take the bar as is.
    Gate 2: per (s, h) row, ||g - r||_inf / ||r||_inf <= rtol_row.
    Returns (max_abs, max_row_rel)."""
    g = np.asarray(gpu_out_f64, np.float64)
    r = np.asarray(ref_f64, np.float64)
    assert g.shape == r.shape
    assert np.isfinite(g).all(), "non-finite output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    bar = atol + half_ulp(r, "bf16" if out_dtype == "bf16" else None)
    worst = float((err - bar).max()) if err.size else -1.0
    rn = np.abs(r).max(axis=-1)
    en = err.max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(rn > 0, en / np.where(rn > 0, rn, 1), en)
    max_rel = float(rel.max()) if rel.size else 0.0
    assert worst <= 0, (f"max abs err {max_abs} exceeds {atol}"
                        + (" + half an ulp of bf16" if out_dtype == "bf16" else ""))
    if rtol_row is not None:
        assert max_rel <= rtol_row, f"max row rel err {max_rel} > {rtol_row}"
    return max_abs, max_rel


def host_threads() -> int:
    """Oracle threads: the CPUs this process may run on, at most 16 (a GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


# ------------------------------------------------------------------ GPU-side helpers
TOL = {"f16": (2e-3, 1e-2), "bf16": (2e-3, 1e-2), "e4m3": (2e-2, None)}


def tolerance(spec):
    """(max abs, max row-relative) bar for the spec's KV dtype."""
    return TOL[spec.kv_dtype]


def to_dev(bits: np.ndarray, dtype: str):
    """Storage bits (numpy) -> device tensor of the matching torch dtype."""
    import torch
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def to_bits(t) -> np.ndarray:
    """Device tensor -> storage bits (numpy), exact."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.uint8,):
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
