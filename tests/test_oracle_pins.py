"""Pins of the CPU oracle against facts fixed outside it (CPU only).

Each test checks the oracle against the pages' worked examples and closed forms,
library conversions, brute force on the logical (unpaged) arrays, or invariants
of the mathematics, chosen so that a dropped term, a wrong index or a transposed
operand in the oracle fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import DT, oracle_caches, oracle_decode, oracle_tables

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))


# ------------------------------------------------------------------ number formats
def test_f16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f64(codes)
    ref = codes.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_encode_matches_numpy(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000)
    # exact ties between neighbouring fp16 values, subnormal through the top of the range
    codes = np.arange(0, 0x7BFF, 7, dtype=np.uint16)
    lo = codes.view(np.float16).astype(np.float64)
    hi = (codes + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2, [65504.0, 65519.0, 65520.0, 1e6, -1e6,
                                                            0.0, -0.0, 2.0 ** -25, 2.0 ** -26]])
    ours = orc.round_to(x, orc.F16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_decode_all_codes(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.bf16_to_f64(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()


def test_bf16_encode_matches_torch(orc):
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(50000) * 10.0 ** rng.integers(-30, 30, 50000)).astype(np.float32)
    # exact midpoints between neighbouring bf16 values (representable in binary32)
    b = rng.integers(0, 0x7F7F, 5000).astype(np.uint32)
    mid = ((b << 16) | 0x8000).view(np.float32)
    x32 = np.concatenate([x32, mid, -mid, np.array([0.0, -0.0, 1e-40, 3e38], np.float32)])
    ours = orc.round_to(x32.astype(np.float64), orc.BF16)
    ref = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    ours = orc.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    # closed forms of the OCP E4M3 definition
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_e4m3_encode_matches_torch_in_range(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-464, 464, 40000),
                        rng.standard_normal(40000) * 10.0 ** rng.integers(-4, 2, 40000)]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    vals = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)  # exact ties
    x = np.concatenate([x, mids, -mids])
    ours = orc.f32_to_e4m3(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates(orc):
    x = np.array([465.0, 480.0, 1e30, np.inf, -500.0, -np.inf], np.float32)
    assert orc.f32_to_e4m3(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.f32_to_e4m3(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


def test_e4m3_dequant_is_binary32_product(orc):
    codes = np.arange(256, dtype=np.uint8)
    scale = np.float32(0.0123456)
    ours = orc.e4m3_to_f64(codes, float(scale))
    ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy() * scale).astype(np.float64)
    nan = np.isnan(ref)
    assert (ours[~nan] == ref[~nan]).all()


# ------------------------------------------------------------------ footprint (closed form)
def test_footprint_closed_form(orc):
    g = GOLDEN["footprint"]
    L, dm = g["num_layers"], g["d_model"]
    # d_model = Hkv * d for any head split of OPT-13B's 5120-wide model
    for heads, d in ((40, 128), (80, 64), (20, 256)):
        assert heads * d == dm
        assert orc.kv_bytes_per_token(L, heads, d, orc.F16) == g["bytes_per_token"]
    assert orc.kv_bytes_per_token(L, 40, 128, orc.F16) * 2048 == g["tokens_2048_bytes"]
    assert orc.kv_bytes_per_token(1, 40, 128, orc.F16) == 20480            # one layer
    assert orc.kv_bytes_per_token(1, 32, 128, orc.E4M3) == 8192            # e4m3 halves it
    assert orc.kv_bytes_per_token(1, 8, 128, orc.BF16) == 4096


# ------------------------------------------------------------------ block tables (O1)
def test_block_table_worked_example(orc):
    g = GOLDEN["block_table_figure"]
    B, n = g["block_size"], g["context_len"]
    NB = 24
    rest = [i for i in range(NB) if i not in g["free_order_prefix"]]
    free = np.array(g["free_order_prefix"] + rest, np.int32)
    st, tables, ref, left = orc.build_tables(NB, B, free, [n], 8)
    assert st == 0
    nblk = math.ceil(n / B)
    assert tables[0, :nblk].tolist() == g["expected_row"]
    assert (tables[0, nblk:] == -1).all()
    filled = [min(B, n - j * B) for j in range(nblk)]
    assert filled == g["expected_filled"]
    tp = g["token_probe"]
    assert tables[0, tp["token"] // B] == tp["phys"] and tp["token"] % B == tp["slot"]
    assert left.tolist() == rest
    assert ref[g["expected_row"]].tolist() == [1, 1, 1] and ref.sum() == 3


def test_contiguous_vs_paged_example(orc):
    g = GOLDEN["contiguous_vs_paged_figure"]
    B = 16
    free = np.array(g["free_order_prefix"] + [0, 2, 3], np.int32)
    st, tables, _, _ = orc.build_tables(15, B, free, [2 * B + 5], 4)
    assert st == 0 and tables[0, :3].tolist() == g["expected_row"]


def test_shared_prompt_refcounts(orc):
    g = GOLDEN["parallel_sampling_figure"]
    B = 4
    K = g["num_samples"]
    free = np.array(g["prompt_blocks"] + [3, 0, 2, 4, 5, 6], np.int32)
    # prompt of two full blocks shared by K samples, then one private token each
    st, tables, ref, left = orc.build_tables(8, B, free, [2 * B + 1] * K, 4,
                                             prefix_group=[0] * K, prefix_lens=[2 * B])
    assert st == 0
    for s in range(K):
        assert tables[s, :2].tolist() == g["prompt_blocks"]
    assert ref[g["prompt_blocks"]].tolist() == [g["expected_refcount"]] * 2
    assert tables[0, 2] == 3 and tables[1, 2] == 0   # private blocks in free-list order
    # releasing one sample drops the shared counts by one and frees only its private block
    fl, ref2 = orc.free_rows(left, tables, [0], ref, 8)
    assert ref2[g["prompt_blocks"]].tolist() == [1, 1] and fl[-1] == 3
    fl, ref3 = orc.free_rows(fl, tables, [1], ref2, 8)
    assert (ref3 == 0).all() and fl[-3:].tolist() == [7, 1, 0]


def test_tables_failures_leave_state(orc):
    free = np.arange(4, dtype=np.int32)
    st, _, _, left = orc.build_tables(4, 4, free, [8, 9], 8)   # needs 2 + 3 = 5 > 4
    assert st == -3 and left.tolist() == [0, 1, 2, 3]
    st, _, _, left = orc.build_tables(4, 4, free, [17], 4)     # 5 blocks > max_blocks 4
    assert st == -4 and left.tolist() == [0, 1, 2, 3]


@pytest.mark.parametrize("name", list(workloads.SPECS))
def test_table_invariants_full_specs(orc, name):
    """Distinct ids, refcount = number of referencing rows, free + used = NB, and the
    waste bound of the allocation lifecycle (at most B-1 empty slots per sequence)."""
    sp = workloads.SPECS[name]
    ctx, free = workloads.draw_lengths(sp, 8900)
    pg, pl = workloads.prefix_groups(sp)
    st, tables, ref, left = orc.build_tables(sp.num_blocks, sp.block_size, free, ctx,
                                             sp.max_blocks, pg, pl)
    assert st == 0
    used = tables[tables >= 0]
    uniq = np.unique(used)
    assert uniq.size + left.size == sp.num_blocks
    assert np.intersect1d(uniq, left).size == 0
    counts = np.bincount(used, minlength=sp.num_blocks)
    assert np.array_equal(counts, ref)
    for s in range(sp.num_seqs):
        nb = math.ceil(ctx[s] / sp.block_size)
        assert (tables[s, :nb] >= 0).all() and (tables[s, nb:] == -1).all()
    waste = int(np.sum(np.ceil(ctx / sp.block_size) * sp.block_size - ctx))
    assert waste <= sp.num_seqs * (sp.block_size - 1)
    if sp.group_size:
        shared = sp.prompt_len // sp.block_size
        for s in range(sp.num_seqs):
            leader = (s // sp.group_size) * sp.group_size
            assert np.array_equal(tables[s, :shared], tables[leader, :shared])
        assert (ref[tables[:, :shared]] == sp.group_size).all()
    # private blocks come off the free list in order
    gb = GOLDEN["waste_bound"]
    assert gb["max_waste_slots"] == gb["block_size"] - 1


def test_private_blocks_follow_free_order(orc):
    sp = workloads.SPECS["opt13b_layer"]
    ctx, free = workloads.draw_lengths(sp, 8902)
    st, tables, _, left = orc.build_tables(sp.num_blocks, sp.block_size, free, ctx, sp.max_blocks)
    row_major = tables[tables >= 0]  # row order s, then j
    assert np.array_equal(row_major, free[: row_major.size])
    assert np.array_equal(left, free[row_major.size:])


# ------------------------------------------------------------------ scatter (O2)
@pytest.mark.parametrize("name", ["tiny_mha", "fp8_prefix"])
def test_scatter_inverts_through_table(orc, name):
    case = workloads.generate(workloads.SMALL[name], 8900 + 1)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    B = sp.block_size
    written = np.zeros(k.shape[:1] + k.shape[2:3], bool)  # [NB, B]
    for s in range(sp.num_seqs):
        n = int(case.context_lens[s])
        t = np.arange(n)
        blk = tables[s, t // B]
        for which, cache, scale in (("k", k, case.k_inv_scale), ("v", v, case.v_inv_scale)):
            got = cache[blk, :, t % B, :]           # [n, Hkv, d]
            src = case.logical(s, which)
            if sp.kv_dtype == "e4m3":
                x = workloads.bits_to_f32(src, sp.src_dtype) * np.float32(scale)
                exp = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            else:
                exp = src
            assert np.array_equal(got, exp)
        written[blk, t % B] = True
    # every other slot still holds the poison pattern
    poison = workloads.poison_bits(sp.kv_dtype)
    assert (k.transpose(0, 2, 1, 3)[~written] == poison).all()
    assert (v.transpose(0, 2, 1, 3)[~written] == poison).all()


# ------------------------------------------------------------------ decode (O4)
def _brute(case, s, h):
    """Contiguous attention on the logical arrays: library conversions and numpy only."""
    sp = case.spec
    G = sp.num_heads // sp.num_kv_heads
    g = h // G

    def deq(bits, which):
        if sp.kv_dtype == "e4m3":
            inv = case.k_inv_scale if which == "k" else case.v_inv_scale
            sc = case.k_scale if which == "k" else case.v_scale
            x = workloads.bits_to_f32(bits, sp.src_dtype) * np.float32(inv)
            c = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
            return (c * np.float32(sc)).astype(np.float64)
        return workloads.bits_to_f32(bits, sp.kv_dtype).astype(np.float64)

    K = deq(case.logical(s, "k")[:, g, :], "k")
    V = deq(case.logical(s, "v")[:, g, :], "v")
    q = workloads.bits_to_f32(case.q[s, h], sp.q_dtype).astype(np.float64)
    z = np.float64(np.float32(sp.scale)) * (K @ q)
    w = np.exp(z - z.max())
    a = w / w.sum()
    return a @ V


@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_decode_matches_brute_force(orc, name):
    case = workloads.generate(workloads.SMALL[name], 8900 + 7)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out = oracle_decode(case, tables, k, v)
    rng = np.random.default_rng(0)
    pairs = [(s, h) for s in range(sp.num_seqs) for h in range(sp.num_heads)]
    if len(pairs) > 12:
        pairs = [pairs[i] for i in rng.choice(len(pairs), 12, replace=False)]
    for s, h in pairs:
        ref = _brute(case, s, h)
        assert np.abs(out[s, h] - ref).max() <= 1e-12


@pytest.mark.parametrize("B", [1, 4, 16])
def test_decode_hand_cases_vs_brute(orc, B):
    for n in sorted({1, max(B - 1, 1), B, B + 1, 3 * B + 2}):
        sp = workloads.Spec("hand", 3, 4, 2, 64, B, n, n, 3 * math.ceil(n / B) + 5,
                            math.ceil(n / B) + 1, "f16", "f16", 0.125)
        case = workloads.generate(sp, 100 + n)
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        out = oracle_decode(case, tables, k, v)
        for s in range(sp.num_seqs):
            for h in range(sp.num_heads):
                assert np.abs(out[s, h] - _brute(case, s, h)).max() <= 1e-12


def test_single_token_returns_v1_exactly(orc):
    for kvd, qd in (("f16", "f16"), ("bf16", "bf16"), ("e4m3", "bf16"), ("e4m3", "f16")):
        sp = workloads.Spec("n1", 5, 8, 4, 128, 16, 1, 1, 16, 2, qd, kvd, 0.0883883)
        case = workloads.generate(sp, 11)
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        out = oracle_decode(case, tables, k, v)
        for s in range(sp.num_seqs):
            blk = tables[s, 0]
            for h in range(sp.num_heads):
                v1 = oracle.to_f64(v[blk, h // 2, 0], DT[kvd], case.v_scale)
                assert np.array_equal(out[s, h], v1)


@pytest.mark.parametrize("name", ["tiny_mha", "gqa_llama", "fp8_prefix"])
def test_weights_sum_to_one(orc, name):
    case = workloads.generate(workloads.SMALL[name], 8900 + 3)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    _, w = oracle_decode(case, tables, k, v, want_weights=True)
    sums = w.sum(axis=-1)
    assert np.abs(sums - 1.0).max() <= 1e-12
    # weights live only on the first n slots
    n = case.context_lens
    for s in range(case.spec.num_seqs):
        assert (w[s, :, n[s]:] == 0).all() and (w[s, :, : n[s]] > 0).all()


def test_zero_query_gives_mean_of_values(orc):
    case = workloads.generate(workloads.SMALL["opt13b_layer"], 8900 + 4)
    case.q[:] = 0
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out = oracle_decode(case, tables, k, v)
    for s in range(case.spec.num_seqs):
        V = workloads.bits_to_f32(case.logical(s, "v"), "f16").astype(np.float64)  # [n, Hkv, d]
        assert np.abs(out[s] - V.mean(axis=0)).max() <= 1e-12


def test_zero_length_row_is_zero(orc):
    sp = workloads.SMALL["tiny_mha"]
    case = workloads.generate(sp, 5, context_lens=[0, 5, 0, 17])
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out = oracle_decode(case, tables, k, v)
    assert (out[0] == 0).all() and (out[2] == 0).all() and np.isfinite(out).all()


@pytest.mark.parametrize("name", ["tiny_mha", "long_split", "fp8_prefix"])
def test_physical_permutation_invariance(orc, name):
    """Moving every block to a new physical id and remapping the table leaves the
    output bit-identical: the table is pure indirection."""
    case = workloads.generate(workloads.SMALL[name], 8900 + 5)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out = oracle_decode(case, tables, k, v)
    perm = np.random.default_rng(9).permutation(sp.num_blocks).astype(np.int32)
    k2 = np.empty_like(k); k2[perm] = k
    v2 = np.empty_like(v); v2[perm] = v
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = oracle_decode(case, t2, k2, v2)
    assert np.array_equal(out, out2)


@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_online_recurrence_equals_definition(orc, name):
    """The pages' block-at-a-time online softmax, in any block order, equals the
    two-pass definition."""
    case = workloads.generate(workloads.SMALL[name].replace(num_seqs=min(4, workloads.SMALL[name].num_seqs)
                                                            if not workloads.SMALL[name].group_size else 4),
                              8900 + 6)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    on = oracle.decode_online(case.q, DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables,
                              case.context_lens, sp.num_kv_heads, sp.block_size, sp.scale,
                              case.k_scale, case.v_scale)
    assert np.abs(on - ref).max() <= 1e-12
    rng = np.random.default_rng(1)
    orders = np.zeros((sp.num_seqs, sp.max_blocks), np.int32)
    for s in range(sp.num_seqs):
        nb = math.ceil(case.context_lens[s] / sp.block_size)
        orders[s, :nb] = rng.permutation(nb)
    on2 = oracle.decode_online(case.q, DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables,
                               case.context_lens, sp.num_kv_heads, sp.block_size, sp.scale,
                               case.k_scale, case.v_scale, block_orders=orders)
    assert np.abs(on2 - ref).max() <= 1e-12


@pytest.mark.parametrize("P_blocks", [1, 2, 5, 32])
def test_partition_merge_equals_definition(orc, P_blocks):
    case = workloads.generate(workloads.SMALL["long_split"].replace(num_seqs=1, num_heads=1,
                                                                   num_kv_heads=1, ctx_lo=3000,
                                                                   ctx_hi=5000, num_blocks=160),
                              8900 + 8)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    part = oracle.decode_partitioned(case.q, DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables,
                                     case.context_lens, sp.num_kv_heads, sp.block_size, sp.scale,
                                     P_blocks * sp.block_size)
    assert np.abs(part - ref).max() <= 1e-12


def test_shared_prefix_equals_private_copies(orc):
    """Sharing prompt blocks by reference count gives the same output as giving every
    sample its own copy of the prompt."""
    case = workloads.generate(workloads.SMALL["fp8_prefix"], 8900 + 9)
    sp = case.spec
    tables, ref, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out = oracle_decode(case, tables, k, v)
    shared = sp.prompt_len // sp.block_size
    assert (ref[tables[:, :shared]] == sp.group_size).all()
    # private layout: no groups; every sequence writes its whole logical context
    priv = workloads.Case(sp.replace(group_size=0, num_blocks=sp.num_seqs * sp.max_blocks),
                          case.context_lens,
                          np.random.default_rng(3).permutation(sp.num_seqs * sp.max_blocks).astype(np.int32),
                          None, None, case.q,
                          np.repeat(np.arange(sp.num_seqs), case.context_lens).astype(np.int32),
                          np.concatenate([np.arange(n) for n in case.context_lens]).astype(np.int32),
                          np.concatenate([case.logical(s, "k") for s in range(sp.num_seqs)]),
                          np.concatenate([case.logical(s, "v") for s in range(sp.num_seqs)]),
                          case.token_index, case.k_scale, case.v_scale, case.k_inv_scale,
                          case.v_inv_scale)
    t2, r2, _ = oracle_tables(priv)
    assert r2.max() == 1
    k2, v2 = oracle_caches(priv, t2)
    out2 = oracle_decode(priv, t2, k2, v2)
    assert np.array_equal(out, out2)


# ------------------------------------------------------------------ multi-token queries
def _multi_case(T, kv="f16", q="f16", seed=3, lens=(1, 2, 5, 16, 17, 40, 64)):
    sp = workloads.Spec("multi", len(lens), 8, 4, 64, 16, 1, 1,
                        sum(math.ceil(n / 16) for n in lens) + 4, math.ceil(max(lens) / 16) + 1,
                        q, kv, 0.125)
    case = workloads.generate(sp, seed, context_lens=list(lens))
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    rng = np.random.default_rng(seed)
    qm = workloads._round_bits(rng.standard_normal((len(lens), T, 8, 64), dtype=np.float32), q)
    return case, tables, k, v, qm


def _multi(case, tables, k, v, qm, masks=None):
    sp = case.spec
    return oracle.decode_multi(qm, DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables,
                               case.context_lens, sp.num_kv_heads, sp.block_size, sp.scale,
                               case.k_scale, case.v_scale, tree_masks=masks)


def test_multi_single_token_equals_decode(orc):
    """T = 1 with the causal mask is the plain decode (a different oracle routine)."""
    case, tables, k, v, qm = _multi_case(1)
    sp = case.spec
    out = _multi(case, tables, k, v, qm)
    ref = oracle.decode(qm[:, 0], DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables,
                        case.context_lens, sp.num_kv_heads, sp.block_size, sp.scale)
    assert np.abs(out[:, 0] - ref).max() <= 1e-13


@pytest.mark.parametrize("T", [2, 4])
def test_multi_causal_equals_truncated_decode(orc, T):
    """Causal query t of a sequence of n tokens sees exactly its first n - T + 1 + t
    positions: the plain decode with that length."""
    case, tables, k, v, qm = _multi_case(T, seed=5 + T)
    sp = case.spec
    out = _multi(case, tables, k, v, qm)
    for t in range(T):
        lens = np.maximum(case.context_lens - T + 1 + t, 0).astype(np.int32)
        ref = oracle.decode(qm[:, t], DT[sp.q_dtype], k, v, DT[sp.kv_dtype], tables, lens,
                            sp.num_kv_heads, sp.block_size, sp.scale)
        assert np.abs(out[:, t] - ref).max() <= 1e-13


def test_multi_tree_mask_vs_dense_numpy(orc):
    """Arbitrary tree masks: dense attention over the visible logical rows in numpy."""
    T = 4
    case, tables, k, v, qm = _multi_case(T, kv="bf16", q="bf16", seed=9)
    sp = case.spec
    rng = np.random.default_rng(1)
    masks = rng.integers(0, 1 << T, (sp.num_seqs, T)).astype(np.uint32)
    masks[0, :] = 0                       # n = 1: query 0..3 see nothing or the one token
    out = _multi(case, tables, k, v, qm, masks)
    G = sp.num_heads // sp.num_kv_heads
    for s in range(sp.num_seqs):
        n = int(case.context_lens[s])
        K = workloads.bits_to_f32(case.logical(s, "k"), "bf16").astype(np.float64)
        V = workloads.bits_to_f32(case.logical(s, "v"), "bf16").astype(np.float64)
        for t in range(T):
            vis = [p for p in range(n) if p < n - T or (masks[s, t] >> (p - (n - T))) & 1]
            for h in range(sp.num_heads):
                if not vis:
                    assert (out[s, t, h] == 0).all()
                    continue
                qv = workloads.bits_to_f32(qm[s, t, h], "bf16").astype(np.float64)
                z = np.float64(np.float32(sp.scale)) * (K[vis, h // G] @ qv)
                w = np.exp(z - z.max())
                ref = (w / w.sum()) @ V[vis, h // G]
                assert np.abs(out[s, t, h] - ref).max() <= 1e-12
