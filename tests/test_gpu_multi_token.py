"""GPU parity of the multi-token decode, pa_decode_multi (draft verification: several query
tokens per sequence with causal or tree masks), against the oracle's multi-token decode."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_89_amd as pa
import workloads
from helpers import (DT, compare, dev_i32, host_threads, oracle_caches, oracle_tables, to_bits,
                     to_dev, tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


def _case(G, T, d, qd, kvd, lens, seed):
    B, Hkv = 16, 2
    sp = workloads.Spec("multi", len(lens), G * Hkv, Hkv, d, B, 0, 0,
                        sum(math.ceil(n / B) for n in lens) + 5, math.ceil(max(lens) / B) + 2,
                        qd, kvd, 1 / math.sqrt(d))
    case = workloads.generate(sp, seed, context_lens=lens)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    rng = np.random.default_rng(seed)
    qm = workloads._round_bits(rng.standard_normal((len(lens), T, G * Hkv, d), dtype=np.float32), qd)
    return case, tables, k, v, qm


def _run(case, tables, k, v, qm, masks, **kw):
    sp = case.spec
    out = pa.decode_multi(to_dev(qm, sp.q_dtype), to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype),
                          dev_i32(tables), dev_i32(case.context_lens), int(case.context_lens.max()),
                          sp.scale, case.k_scale, case.v_scale,
                          tree_masks=None if masks is None else dev_i32(masks.view(np.int32)), **kw)
    torch.cuda.synchronize()
    return out.double().cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3"),
                                ("f16", "e4m3")])
def test_multi_token_matches_oracle_all_variants(d, dt):
    """Every compiled variant and column count (G heads x T draft tokens in {2, 4, 8, 16});
    lengths 0, below and at T, around block and partition edges; causal and random tree
    masks (some rows see only the committed prefix, some nothing at all); library,
    one-block and four-block partitions; both load policies."""
    qd, kvd = dt
    lens = [0, 1, 3, 4, 16, 17, 33, 300, 513]
    for G, T in ((1, 2), (1, 4), (1, 16), (2, 1), (2, 2), (2, 8), (4, 1), (4, 4), (8, 2)):
        case, tables, k, v, qm = _case(G, T, d, qd, kvd, lens, 300 + 17 * G + T + d)
        rng = np.random.default_rng(G * 100 + T)
        tree = rng.integers(0, 1 << T, (len(lens), T)).astype(np.uint32)
        tree[1, :] = 0      # n = 1: its one position is a draft nobody sees -> zero rows
        tree[5, 0] = 0      # n = 17: query 0 sees the committed positions only
        atol, rrel = tolerance(case.spec)
        for masks in (None, tree):
            ref = oracle.decode_multi(qm, DT[qd], k, v, DT[kvd], tables, case.context_lens,
                                      case.spec.num_kv_heads, 16, case.spec.scale, case.k_scale,
                                      case.v_scale, tree_masks=masks)
            for P in (0, 16, 64):
                for flags in (0, pa.DECODE_SHARED_KV):
                    out = _run(case, tables, k, v, qm, masks, partition_size=P, flags=flags)
                    assert (out[0] == 0).all(), "n = 0 must give zero rows"
                    compare(out.reshape(-1, d), ref.reshape(-1, d), atol, rrel, qd)


def test_flat_merge_of_more_rows_than_resident_wavefronts():
    """255 sequences x 4 draft tokens x 9 heads = 9,180 rows under the flat split, more
    than the merge's wavefronts an MI355X holds at once."""
    B, Hkv, T, d = 16, 9, 4, 64
    rng = np.random.default_rng(8960)
    lens = rng.integers(3, 401, 255).tolist()
    lens[0] = 0
    sp = workloads.Spec("rows", len(lens), Hkv, Hkv, d, B, 0, 0,
                        sum(math.ceil(n / B) for n in lens) + 5, math.ceil(max(lens) / B) + 2,
                        "bf16", "bf16", 1 / math.sqrt(d))
    case = workloads.generate(sp, 8961, context_lens=lens)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    qm = workloads._round_bits(rng.standard_normal((len(lens), T, Hkv, d), dtype=np.float32), "bf16")
    assert pa.decode_plan(len(lens), Hkv, Hkv, d, B, max(lens), 0, pa.BF16)[2] > 0
    ref = oracle.decode_multi(qm, DT["bf16"], k, v, DT["bf16"], tables, case.context_lens, Hkv, B,
                              sp.scale, case.k_scale, case.v_scale, tree_masks=None)
    out = _run(case, tables, k, v, qm, None)
    assert (out[0] == 0).all()
    compare(out.reshape(-1, d), ref.reshape(-1, d), *tolerance(sp), "bf16")


def test_multi_token_causal_row_equals_plain_decode_of_truncated_length():
    """Query token t of a causal draft gives what pa_decode gives for the same query with
    context length n - T + 1 + t, to rounding."""
    G, T, d = 4, 4, 128
    lens = [40, 100, 257, 700]
    case, tables, k, v, qm = _case(G, T, d, "bf16", "bf16", lens, 11)
    out = _run(case, tables, k, v, qm, None)
    sp = case.spec
    for t in range(T):
        lt = (case.context_lens - T + 1 + t).astype(np.int32)
        ref = pa.decode(to_dev(qm[:, t].copy(), "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                        dev_i32(tables), dev_i32(lt), int(lt.max()), sp.scale)
        torch.cuda.synchronize()
        # both results are rounded to bf16: allow one bf16 ulp besides the kernel error
        compare(out[:, t], ref.double().cpu().numpy(), 1e-2, 2e-2, "bf16")


@pytest.mark.parametrize("name", ["opt13b_layer", "gqa_llama", "fp8_prefix"])
def test_full_size_multi_token_all_sequences(name):
    """Four causal draft tokens per sequence over each workload at full size, launched as
    the benchmark's multi-token path launches it; the threaded oracle computes every query
    row of every sequence."""
    T = 4
    sp = workloads.SPECS[name]
    seed = 8900 + list(workloads.SPECS).index(name)
    ctx, free = workloads.draw_lengths(sp, seed)
    pg, pl = workloads.prefix_groups(sp)
    st, tables, _, _ = oracle.build_tables(sp.num_blocks, sp.block_size, free, ctx,
                                           sp.max_blocks, pg, pl)
    assert st == 0 and ctx.min() >= T
    _, kd, vd, ks, vs = workloads.device_pool(sp, seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 7)
    qt = torch.float16 if sp.q_dtype == "f16" else torch.bfloat16
    qm = torch.randn((sp.num_seqs, T, sp.num_heads, sp.head_dim), generator=g,
                     device="cuda").to(qt)
    flags = pa.DECODE_SHARED_KV if sp.group_size else 0
    out = pa.decode_multi(qm, kd, vd, dev_i32(tables), dev_i32(ctx), int(ctx.max()), sp.scale,
                          ks, vs, partition_size=sp.partition_size, flags=flags)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    qb = qm.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    kb, vb = to_bits(kd), to_bits(vd)
    del kd, vd
    ref = oracle.decode_multi(qb, DT[sp.q_dtype], kb, vb, DT[sp.kv_dtype], tables, ctx,
                              sp.num_kv_heads, sp.block_size, sp.scale, ks, vs,
                              threads=host_threads())
    atol, rrel = tolerance(sp)
    compare(got, ref, atol, rrel, sp.q_dtype)
