"""Test-side helpers: build oracle inputs from a seeded case and compare results."""
from __future__ import annotations

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


def compare(gpu_out_f64: np.ndarray, ref_f64: np.ndarray, atol: float, rtol_row: float | None):
    """Tolerance gates: max |g - r| over all elements <= atol, and per (s, h) row
    ||g - r||_inf / ||r||_inf <= rtol_row.  Returns (max_abs, max_row_rel)."""
    g = np.asarray(gpu_out_f64, np.float64)
    r = np.asarray(ref_f64, np.float64)
    assert g.shape == r.shape
    assert np.isfinite(g).all(), "non-finite output"
    err = np.abs(g - r)
    max_abs = float(err.max()) if err.size else 0.0
    rn = np.abs(r).max(axis=-1)
    en = err.max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(rn > 0, en / np.where(rn > 0, rn, 1), en)
    max_rel = float(rel.max()) if rel.size else 0.0
    assert max_abs <= atol, f"max abs err {max_abs} > {atol}"
    if rtol_row is not None:
        assert max_rel <= rtol_row, f"max row rel err {max_rel} > {rtol_row}"
    return max_abs, max_rel
