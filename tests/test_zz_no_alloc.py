"""pa_decode_noalloc against pa_decode (needs an MI355X).

The no-allocation decode launches the same kernels as pa_decode with the partition
partials in the library's fixed device array instead of a caller workspace.  Each case
calls both entry points through the C ABI on the same inputs: the outputs must be
bit-identical, and both within the oracle's bar.  Two calls in a row reuse the array, the
second with a smaller input (fewer rows, fewer partitions), so a partial left behind by the
first call would show up in the second.  Oversized plans are refused before any launch.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import workloads
import paged_kv_cache_89_amd as pa
from helpers import (compare, dev_i32, oracle_caches, oracle_decode, oracle_tables, to_bits,
                     to_dev, tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()  # fail loudly when the library is not built
    yield
    torch.cuda.synchronize()


def _run_both(case, tables, k, v, P, rows=None):
    """pa_decode (own workspace) and pa_decode_noalloc on rows [0, rows) of the case."""
    sp = case.spec
    n = sp.num_seqs if rows is None else rows
    ctx = case.context_lens[:n]
    q = to_dev(case.q[:n], sp.q_dtype)
    kd, vd = to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype)
    td, cd = dev_i32(tables[:n]), dev_i32(ctx)
    mc = int(ctx.max())
    need = pa.decode_workspace_size(n, sp.num_heads, sp.num_kv_heads, sp.head_dim,
                                    sp.block_size, mc, P)
    assert 0 < need <= pa.NOALLOC_SCRATCH_BYTES, need  # the case must use the array
    ref_out = pa.decode(q, kd, vd, td, cd, mc, sp.scale, case.k_scale, case.v_scale,
                        partition_size=P)
    out = torch.full_like(q, float("nan"))
    pa.decode_noalloc(q, kd, vd, td, cd, mc, sp.scale, case.k_scale, case.v_scale,
                      partition_size=P, out=out)
    torch.cuda.synchronize()
    return to_bits(ref_out), to_bits(out), out.double().cpu().numpy()


CASES = [("long_split", 512, 256, 1), ("gqa_llama", 256, 128, 2), ("fp8_prefix", 256, 128, 4),
         ("opt13b_layer", 256, 512, 3),
         # library-chosen splits: the flat split (fp16/bf16) on both calls
         ("opt13b_layer", 0, 0, 3), ("gqa_llama", 0, 0, 2)]


@pytest.mark.parametrize("name,P1,P2,rows2", CASES)
def test_noalloc_matches_decode_on_two_calls(name, P1, P2, rows2):
    """First call: the whole reduced workload; second call: its first rows2 sequences with
    another partition size, so fewer partials than the first call left in the array."""
    case = workloads.generate(workloads.SMALL[name], 8900 + 40)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    atol, rrel = tolerance(case.spec)
    for P, rows in ((P1, None), (P2, rows2)):
        a, b, got = _run_both(case, tables, k, v, P, rows)
        assert np.array_equal(a, b), (name, P, rows)
        n = got.shape[0]
        compare(got, ref[:n], atol, rrel, case.spec.q_dtype)


def test_noalloc_refuses_plans_beyond_the_array():
    """A plan whose partials exceed the array is refused before anything is launched (the
    pointers are never touched, so NULL is fine here)."""
    S, Hq, Hkv, D, B, ctx = 512, 64, 8, 128, 16, 32768
    need = pa.decode_workspace_size(S, Hq, Hkv, D, B, ctx, 512)
    assert need > pa.NOALLOC_SCRATCH_BYTES
    st = pa.lib().pa_decode_noalloc(None, None, None, None, None, None, S, Hq, Hkv, D, B,
                                    ctx // B, 1 << 20, ctx, ctypes.c_float(0.088), pa.F16,
                                    pa.F16, ctypes.c_float(1.0), ctypes.c_float(1.0), 512, 0,
                                    None)
    assert st == -2  # PA_ERR_UNSUPPORTED
    assert b"scratch" in pa.lib().pa_last_error()


def test_noalloc_takes_fixed_partitions_when_the_flat_split_does_not_fit():
    """128 sequences x 32 query heads under an 8192-token bound: the flat split's partials
    (33 slots a row) exceed the array, its fixed 1024-token partitions (8 slots) fit, so the
    call gives exactly pa_decode's output with those partitions, twice in a row."""
    S, Hq, Hkv, D, B, mc = 128, 32, 8, 128, 16, 8192
    flat = pa.decode_workspace_size(S, Hq, Hkv, D, B, mc, 0)
    fixed = pa.decode_workspace_size(S, Hq, Hkv, D, B, mc, 1024)
    assert fixed <= pa.NOALLOC_SCRATCH_BYTES < flat
    assert pa.decode_plan(S, Hq, Hkv, D, B, mc, 0, pa.BF16)[:2] == (0, 33)
    rng = np.random.default_rng(8900 + 41)
    lens = rng.integers(1, 1500, S).astype(np.int32)
    lens[3] = 0
    nb = int(sum((n + B - 1) // B for n in lens))
    perm = rng.permutation(nb + 5).astype(np.int32)
    tables = np.full((S, mc // B), -1, np.int32)
    k = 0
    for s, n in enumerate(lens):
        m = (int(n) + B - 1) // B
        tables[s, :m] = perm[k:k + m]
        k += m
    g = torch.Generator(device="cuda")
    g.manual_seed(8900 + 42)
    kd = torch.randn((nb + 5, Hkv, B, D), generator=g, device="cuda").to(torch.bfloat16)
    vd = torch.randn((nb + 5, Hkv, B, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((S, Hq, D), generator=g, device="cuda").to(torch.bfloat16)
    td, cd = dev_i32(tables), dev_i32(lens)
    ref = pa.decode(q, kd, vd, td, cd, mc, 0.088, partition_size=1024)
    for _ in range(2):
        out = torch.full_like(q, float("nan"))
        pa.decode_noalloc(q, kd, vd, td, cd, mc, 0.088, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
