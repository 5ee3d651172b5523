"""GPU parity of libpaged_attn against the CPU oracle (needs an MI355X).

Every case builds its inputs from a seeded generator, runs the HIP path through
the C ABI (via the thin Python binding) and compares with the oracle:
  * block tables and the KV write scatter: bit-exact;
  * fp16/bf16 KV decode: max |gpu - oracle| <= 2e-3 and per-row
    ||gpu - oracle||_inf / ||oracle||_inf <= 1e-2;
  * e4m3 KV decode: max |gpu - oracle| <= 2e-2 against an oracle that dequantises
    the same bytes with the same per-tensor scale.
The oracle output is fp64 and unrounded; every unused cache slot and free block is
NaN-poisoned, so a read past a sequence's end shows up as a NaN.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import paged_kv_cache_89_amd as pa
from helpers import (DT, compare, dev_i32, host_threads, oracle_caches, oracle_decode,
                     oracle_tables, to_bits, to_dev, tolerance)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()  # fail loudly when the library is not built
    yield
    torch.cuda.synchronize()


def _flags(spec):
    """The decode flags a caller would pass: shared prompt blocks -> PA_DECODE_SHARED_KV."""
    return pa.DECODE_SHARED_KV if spec.group_size else 0


def _gpu_decode(case, tables, k, v, partition_size=None, max_ctx=None, flags=None):
    sp = case.spec
    q = to_dev(case.q, sp.q_dtype)
    kd, vd = to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype)
    P = sp.partition_size if partition_size is None else partition_size
    mc = int(case.context_lens.max()) if max_ctx is None else max_ctx
    out = pa.decode(q, kd, vd, dev_i32(tables), dev_i32(case.context_lens), mc, sp.scale,
                    case.k_scale, case.v_scale, partition_size=P,
                    flags=_flags(sp) if flags is None else flags)
    torch.cuda.synchronize()
    return out


def _f64(out):
    return out.double().cpu().numpy()


# ------------------------------------------------------------------ KV write scatter
@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_write_kv_bit_exact(name):
    case = workloads.generate(workloads.SMALL[name], 8900 + 20)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k_ref, v_ref = oracle_caches(case, tables)
    kd = to_dev(workloads.empty_cache(sp), sp.kv_dtype)
    vd = to_dev(workloads.empty_cache(sp), sp.kv_dtype)
    pa.write_kv(to_dev(case.k_src, sp.src_dtype), to_dev(case.v_src, sp.src_dtype), kd, vd,
                dev_i32(tables), dev_i32(case.seq_ids), dev_i32(case.positions),
                case.k_inv_scale, case.v_inv_scale)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kd), k_ref)
    assert np.array_equal(to_bits(vd), v_ref)


def test_write_kv_e4m3_every_code_path():
    """Quantise values across the whole e4m3 range (subnormals, ties, saturation) and
    compare every byte with the oracle's encoder."""
    rng = np.random.default_rng(4)
    sp = workloads.Spec("q", 1, 2, 2, 128, 16, 64, 64, 8, 4, "f16", "e4m3", 0.1)
    T = 64
    mags = np.concatenate([rng.uniform(0, 2 ** -6, T * 64), rng.uniform(2 ** -6, 600, T * 64),
                           rng.standard_normal(T * 128) * 100])
    x = (mags[: T * 2 * 128] * np.where(rng.random(T * 2 * 128) < 0.5, -1, 1)).astype(np.float32)
    for src_dtype, qd in (("f16", "f16"), ("bf16", "bf16")):
        src = workloads._round_bits(x.reshape(T, 2, 128), src_dtype)
        case = workloads.Case(sp.replace(q_dtype=qd), np.array([T], np.int32),
                              np.arange(8, dtype=np.int32), None, None,
                              np.zeros((1, 2, 128), np.uint16), np.zeros(T, np.int32),
                              np.arange(T, dtype=np.int32), src, src,
                              np.arange(T, dtype=np.int32)[None], 1.0, 1.0, 0.75, 1.0)
        tables, _, _ = oracle_tables(case)
        k_ref, v_ref = oracle_caches(case, tables)
        kd = to_dev(workloads.empty_cache(sp), "e4m3")
        vd = to_dev(workloads.empty_cache(sp), "e4m3")
        pa.write_kv(to_dev(src, src_dtype), to_dev(src, src_dtype), kd, vd, dev_i32(tables),
                    dev_i32(case.seq_ids), dev_i32(case.positions), 0.75, 1.0)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(kd), k_ref) and np.array_equal(to_bits(vd), v_ref)


def test_write_kv_skips_bad_rows():
    """Tokens whose sequence, position or table entry is out of range are skipped."""
    sp = workloads.Spec("w", 2, 4, 4, 64, 8, 8, 8, 6, 2, "f16", "f16", 0.1)
    tables = np.array([[0, -1], [1, 99]], np.int32)
    seq_ids = np.array([0, 0, 1, 5, -1, 1], np.int32)
    pos = np.array([3, 9, 2, 0, 0, 12], np.int32)  # row 1: entry -1; row 5: entry 99
    src = workloads._round_bits(np.random.default_rng(0).standard_normal((6, 4, 64),
                                                                          dtype=np.float32), "f16")
    kd = to_dev(workloads.empty_cache(sp), "f16")
    vd = to_dev(workloads.empty_cache(sp), "f16")
    pa.write_kv(to_dev(src, "f16"), to_dev(src, "f16"), kd, vd, dev_i32(tables),
                dev_i32(seq_ids), dev_i32(pos))
    torch.cuda.synchronize()
    k = to_bits(kd)
    expect = workloads.empty_cache(sp)
    expect[0, :, 3, :] = src[0]
    expect[1, :, 2, :] = src[2]
    assert np.array_equal(k, expect)


# ------------------------------------------------------------------ decode parity
@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_decode_matches_oracle(name):
    case = workloads.generate(workloads.SMALL[name], 8900 + 21)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    out = _gpu_decode(case, tables, k, v)
    atol, rrel = tolerance(case.spec)
    compare(_f64(out), ref, atol, rrel, case.spec.q_dtype)


@pytest.mark.parametrize("name", list(workloads.SMALL))
def test_end_to_end_block_manager_write_decode(name):
    """Tables from the library's block manager, cache filled by pa_write_kv, then
    pa_decode: the whole path against the oracle's own tables/scatter/decode."""
    case = workloads.generate(workloads.SMALL[name], 8900 + 22)
    sp = case.spec
    t_or, _, _ = oracle_tables(case)
    k_ref, v_ref = oracle_caches(case, t_or)
    ref = oracle_decode(case, t_or, k_ref, v_ref)
    bm = pa.BlockManager(sp.num_blocks, sp.block_size, case.free_order)
    tables, _ = bm.alloc_tables(case.context_lens, sp.max_blocks, case.prefix_group,
                                case.prefix_lens)
    assert np.array_equal(tables, t_or)
    kd = to_dev(workloads.empty_cache(sp), sp.kv_dtype)
    vd = to_dev(workloads.empty_cache(sp), sp.kv_dtype)
    td = dev_i32(tables)
    pa.write_kv(to_dev(case.k_src, sp.src_dtype), to_dev(case.v_src, sp.src_dtype), kd, vd, td,
                dev_i32(case.seq_ids), dev_i32(case.positions), case.k_inv_scale,
                case.v_inv_scale)
    out = pa.decode(to_dev(case.q, sp.q_dtype), kd, vd, td, dev_i32(case.context_lens),
                    int(case.context_lens.max()), sp.scale, case.k_scale, case.v_scale,
                    partition_size=sp.partition_size, flags=_flags(sp))
    torch.cuda.synchronize()
    atol, rrel = tolerance(sp)
    compare(_f64(out), ref, atol, rrel, case.spec.q_dtype)


@pytest.mark.parametrize("B", [8, 16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", [("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3"),
                                ("f16", "e4m3")])
def test_decode_ragged_lengths_all_variants(B, d, dt):
    """Every compiled (head_dim, block size, dtype) variant on lengths around block and
    partition edges, including 0 and 1, with GQA groups 1, 2, 4 and 8 (16-token fp16/bf16
    blocks with G >= 2 run on the matrix-core kernel, the rest on the vector kernel)."""
    qd, kvd = dt
    lens = [0, 1, B - 1, B, B + 1, 2 * B + 3, 97, 300, 513]
    for G in (1, 2, 4, 8):
        sp = workloads.Spec("rag", len(lens), 4 * G, 4, d, B, 1, 1,
                            sum(math.ceil(n / B) for n in lens) + 7,
                            math.ceil(max(lens) / B) + 2, qd, kvd, 1 / math.sqrt(d))
        case = workloads.generate(sp, 1000 + B + d + G, context_lens=lens)
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        ref = oracle_decode(case, tables, k, v)
        atol, rrel = tolerance(sp)
        for P in (0, B, 4 * B):
            for flags in (0, pa.DECODE_SHARED_KV):  # streaming and cacheable K/V loads
                out = _f64(_gpu_decode(case, tables, k, v, partition_size=P, flags=flags))
                assert (out[0] == 0).all(), "n = 0 must give a zero row"
                compare(out, ref, atol, rrel, qd)


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_few_dominant_tokens_with_distant_values(qd):
    """A handful of tokens share the weight and their values are far apart (+-4): the
    output then amplifies any rounding of the weights, which must stay within the bar on
    the matrix-core path (bf16 has only 8 significant bits for P)."""
    lens = [2, 3, 5, 7, 16, 19]
    for G in (2, 4, 8):
        sp = workloads.Spec("few", len(lens), 4 * G, 4, 128, 16, 1, 1, 40, 3, qd, qd,
                            1 / math.sqrt(128))
        case = workloads.generate(sp, 77 + G, context_lens=lens)
        rng = np.random.default_rng(G)
        signs = rng.choice([-4.0, 4.0], case.v_src.shape).astype(np.float32)
        case.v_src = workloads._round_bits(signs, qd)
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        ref = oracle_decode(case, tables, k, v)
        compare(_f64(_gpu_decode(case, tables, k, v, partition_size=0)), ref, 2e-3, 1e-2, qd)


@pytest.mark.parametrize("qd", ["bf16", "f16"])
def test_e4m3_sink_token_with_many_small_weights(qd):
    """Position 0 of every sequence scores about 9 (natural log units) above the rest for
    one query head per KV head, so each other token weighs ~2^-13 of it, yet together they
    carry about a third of the mass.  On the fp8 matrix-core path those small weights
    must keep their precision (they are lifted per block before rounding to e4m3), not
    fall below e4m3's range; the vector kernel (G = 1) runs the same case."""
    lens = [1500, 700, 33]
    for G in (1, 4):
        sp = workloads.Spec("sink", len(lens), 4 * G, 4, 128, 16, 1, 1,
                            sum(math.ceil(n / 16) for n in lens) + 5, 96, qd, "e4m3",
                            1 / math.sqrt(128))
        case = workloads.generate(sp, 500 + G, context_lens=lens)
        src = sp.src_dtype
        q = workloads.bits_to_f32(case.q, qd).astype(np.float64)
        k32 = workloads.bits_to_f32(case.k_src, src)
        for row in np.nonzero(case.positions == 0)[0]:
            s = case.seq_ids[row]
            for g in range(4):
                qh = q[s, g * G]
                k32[row, g] = (9.0 * math.sqrt(128) * qh / (qh @ qh)).astype(np.float32)
        case.k_src = workloads._round_bits(k32, src)
        amax = np.float32(np.abs(workloads.bits_to_f32(case.k_src, src)).max())
        case.k_scale = float(np.float32(amax / np.float32(448.0)))
        case.k_inv_scale = float(np.float32(1.0) / np.float32(case.k_scale))
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        ref = oracle_decode(case, tables, k, v)
        for P in (0, 1024):
            out = _f64(_gpu_decode(case, tables, k, v, partition_size=P))
            compare(out, ref, 2e-2, None, qd)


def test_single_token_returns_v1_bit_exact():
    for qd, kvd in (("f16", "f16"), ("bf16", "bf16"), ("bf16", "e4m3"), ("f16", "e4m3")):
        sp = workloads.Spec("n1", 6, 8, 2, 128, 16, 1, 1, 12, 2, qd, kvd, 0.0883883)
        case = workloads.generate(sp, 31)
        tables, _, _ = oracle_tables(case)
        k, v = oracle_caches(case, tables)
        out = to_bits(_gpu_decode(case, tables, k, v))
        ref = oracle.round_to(oracle_decode(case, tables, k, v), DT[qd])
        assert np.array_equal(out, ref), (qd, kvd)


def test_e4m3_decoder_matches_ocp_definition():
    """n = 1 with v_scale = 1 returns the decoded value of every e4m3 code (all of them
    are exact in bf16): pins the in-register fp8 decode to the OCP E4M3 format."""
    sp = workloads.Spec("codes", 2, 1, 1, 128, 16, 1, 1, 2, 1, "bf16", "e4m3", 0.1)
    case = workloads.generate(sp, 3)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    k = np.zeros((2, 1, 16, 128), np.uint8)
    v = np.zeros((2, 1, 16, 128), np.uint8)
    v[0, 0, 0] = codes[0]
    v[1, 0, 0] = codes[1]
    tables = np.array([[0], [1]], np.int32)
    case.v_scale = 1.0
    out = _f64(_gpu_decode(case, tables, k, v))
    ref = oracle.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert (np.isnan(out[:, 0]) == nan).all() and (out[:, 0][~nan] == ref[~nan]).all()


def test_physical_permutation_bit_identical():
    case = workloads.generate(workloads.SMALL["opt13b_layer"], 8900 + 23)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    out1 = to_bits(_gpu_decode(case, tables, k, v))
    perm = np.random.default_rng(5).permutation(sp.num_blocks).astype(np.int32)
    k2 = np.empty_like(k); k2[perm] = k
    v2 = np.empty_like(v); v2[perm] = v
    t2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1).astype(np.int32)
    out2 = to_bits(_gpu_decode(case, t2, k2, v2))
    assert np.array_equal(out1, out2)


@pytest.mark.parametrize("name", ["opt13b_layer", "fp8_prefix"])
def test_load_policy_flag_gives_identical_results(name):
    """At a given partition size PA_DECODE_SHARED_KV only changes cache hints and the order
    units are visited: every unit computes the same thing, so the output is bit-identical.
    Under the library's choice the flag also keeps fixed partitions where fp16/bf16 caches
    would take the flat split: both then agree with the oracle."""
    case = workloads.generate(workloads.SMALL[name], 8900 + 26)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    for P in (256, 512):
        a = to_bits(_gpu_decode(case, tables, k, v, partition_size=P, flags=0))
        b = to_bits(_gpu_decode(case, tables, k, v, partition_size=P, flags=pa.DECODE_SHARED_KV))
        assert np.array_equal(a, b)
    ref = oracle_decode(case, tables, k, v)
    atol, rrel = tolerance(case.spec)
    for flags in (0, pa.DECODE_SHARED_KV):
        out = _f64(_gpu_decode(case, tables, k, v, partition_size=0, flags=flags))
        compare(out, ref, atol, rrel, case.spec.q_dtype)


@pytest.mark.parametrize("qd", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 4])
def test_merge_of_many_partitions(qd, G):
    """One-block partitions over long rows: up to 200 partials per row, so the merge walks
    several 64-slot chunks and a ragged last one; rows of 0 and 1 partials beside them."""
    B = 16
    lens = [3200, 1100, 17, 0, 2049, 1024, 16]
    sp = workloads.Spec("many", len(lens), 2 * G, 2, 128, B, 1, 1,
                        sum(math.ceil(n / B) for n in lens) + 5, math.ceil(max(lens) / B) + 1,
                        qd, qd, 1 / math.sqrt(128))
    case = workloads.generate(sp, 8900 + 26 + G, context_lens=lens)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    assert pa.decode_plan(sp.num_seqs, sp.num_heads, sp.num_kv_heads, 128, B, max(lens), B)[1] == 200
    out = _f64(_gpu_decode(case, tables, k, v, partition_size=B))
    assert (out[3] == 0).all()
    compare(out, ref, *tolerance(sp), qd)


def test_merge_of_more_rows_than_resident_wavefronts():
    """8,195 rows of at most three partitions, more than the merge's wavefronts an MI355X
    holds at once (two rounds of them, the last workgroup partly filled); rows of 0, 1, 2
    and 3 partials."""
    B, P = 8, 32
    rng = np.random.default_rng(8950)
    lens = rng.integers(0, 97, 8195).tolist()
    lens[:4] = [0, 32, 33, 96]
    sp = workloads.Spec("rows", len(lens), 1, 1, 64, B, 1, 1,
                        sum(math.ceil(n / B) for n in lens) + 5, math.ceil(96 / B) + 1,
                        "f16", "f16", 1 / 8)
    case = workloads.generate(sp, 8951, context_lens=lens)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    assert pa.decode_plan(sp.num_seqs, 1, 1, 64, B, 96, P)[1] == 3
    out = _f64(_gpu_decode(case, tables, k, v, partition_size=P))
    assert (out[0] == 0).all()
    compare(out, ref, *tolerance(sp), "f16")


def test_partition_size_invariance_and_determinism():
    case = workloads.generate(workloads.SMALL["long_split"], 8900 + 24)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    outs = {}
    for P in (0, 32, 256, 512, 4096):
        outs[P] = _f64(_gpu_decode(case, tables, k, v, partition_size=P))
        compare(outs[P], ref, 2e-3, 1e-2, sp.q_dtype)
    again = _f64(_gpu_decode(case, tables, k, v, partition_size=512))
    assert np.array_equal(again, outs[512])


def test_max_context_len_clamps_lengths():
    """Lengths above max_context_len are treated as max_context_len."""
    case = workloads.generate(workloads.SMALL["tiny_mha"], 8900 + 25)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    cap = int(np.sort(case.context_lens)[1])
    clipped = workloads.Case(**{**case.__dict__, "context_lens": np.minimum(case.context_lens, cap)})
    ref = oracle_decode(clipped, tables, k, v)
    out = _f64(_gpu_decode(case, tables, k, v, max_ctx=cap))
    compare(out, ref, 2e-3, 1e-2, "f16")


# ------------------------------------------------------------------ full-size workloads
@pytest.mark.parametrize("name", list(workloads.SPECS))
def test_full_size_all_rows(name):
    """Each workload at its full size, launched as the benchmark launches it; the threaded
    oracle computes every (sequence, head) row from the same device-drawn bits."""
    sp = workloads.SPECS[name]
    seed = 8900 + list(workloads.SPECS).index(name)
    ctx, free = workloads.draw_lengths(sp, seed)
    pg, pl = workloads.prefix_groups(sp)
    st, tables, _, _ = oracle.build_tables(sp.num_blocks, sp.block_size, free, ctx,
                                           sp.max_blocks, pg, pl)
    assert st == 0
    q, kd, vd, ks, vs = workloads.device_pool(sp, seed)
    out = pa.decode(q, kd, vd, dev_i32(tables), dev_i32(ctx), int(ctx.max()), sp.scale, ks, vs,
                    partition_size=sp.partition_size, flags=_flags(sp))
    torch.cuda.synchronize()
    got = _f64(out)
    qb, kb, vb = to_bits(q), to_bits(kd), to_bits(vd)
    del kd, vd
    ref = oracle.decode(qb, DT[sp.q_dtype], kb, vb, DT[sp.kv_dtype], tables, ctx,
                        sp.num_kv_heads, sp.block_size, sp.scale, ks, vs,
                        threads=host_threads())
    atol, rrel = tolerance(sp)
    compare(got, ref, atol, rrel, sp.q_dtype)


@pytest.mark.parametrize("kv,q,G", [("f16", "f16", 1), ("bf16", "bf16", 4), ("e4m3", "bf16", 1),
                                    ("e4m3", "bf16", 4)])
def test_pools_beyond_4_gib(kv, q, G):
    """Every block the batch uses lies above byte 2^32 of pools larger than 4 GiB: the KV
    write, the batched block copy and the decode (vector kernel for G = 1, matrix cores for
    G = 4) must form 64-bit addresses.  The oracle sees the same blocks renumbered from 0."""
    Hkv, d, B = 8, 128, 16
    e = 1 if kv == "e4m3" else 2
    block_bytes = Hkv * B * d * e
    used = 64
    nb_big = (1 << 32) // block_bytes + used          # pool of more than 4 GiB
    base = nb_big - used                              # first block above byte 2^32
    assert base * block_bytes >= 1 << 32
    lens = np.array([37, 300, 16, 1], np.int32)
    S, MB = lens.size, 24
    small = np.full((S, MB), -1, np.int32)
    nxt = 0
    for s_, n in enumerate(lens):
        nb = -(-int(n + 1) // B)                      # room for one appended token
        small[s_, :nb] = np.arange(nxt, nxt + nb)
        nxt += nb
    spare = used - 1                                  # destination of the block copy
    assert nxt < spare
    big = np.where(small >= 0, small + base, -1).astype(np.int32)
    sp = workloads.Spec("big", S, Hkv * G, Hkv, d, B, 1, 1, used, MB, q, kv, 1 / math.sqrt(d))
    rng = np.random.default_rng(21 + G)
    src = sp.src_dtype
    seq_ids = np.concatenate([np.full(n, i, np.int32) for i, n in enumerate(lens)])
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    rows = {w: workloads._round_bits(rng.standard_normal((seq_ids.size, Hkv, d),
                                                         dtype=np.float32), src) for w in "kv"}
    scale, inv = 1.0, 1.0
    if kv == "e4m3":
        scale = float(np.float32(4.0 / 448.0))
        inv = float(np.float32(1.0) / np.float32(scale))
    k_or, v_or = workloads.empty_cache(sp), workloads.empty_cache(sp)
    oracle.scatter(rows["k"], DT[src], k_or, DT[kv], small, seq_ids, pos, B, inv)
    oracle.scatter(rows["v"], DT[src], v_or, DT[kv], small, seq_ids, pos, B, inv)
    valid = np.zeros((used, B), bool)                 # slots holding a token (small ids)
    for s_, n in enumerate(lens):
        for t in range(int(n)):
            valid[small[s_, t // B], t % B] = True
    valid[spare] = valid[small[1, 0]]
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "e4m3": torch.uint8}[kv]
    kd = torch.empty((nb_big, Hkv, B, d), dtype=tdt, device="cuda")
    vd = torch.empty_like(kd)
    try:
        pa.write_kv(to_dev(rows["k"], src), to_dev(rows["v"], src), kd, vd, dev_i32(big),
                    dev_i32(seq_ids), dev_i32(pos), inv, inv)
        # copy the first block of sequence 1 to the spare block and point the table at it
        pa.copy_blocks(kd, vd, dev_i32([[big[1, 0], base + spare]]))
        k_or[spare], v_or[spare] = k_or[small[1, 0]], v_or[small[1, 0]]
        small[1, 0], big[1, 0] = spare, base + spare
        torch.cuda.synchronize()
        ids = torch.arange(base, nb_big, device="cuda")
        for dev_pool, ref_pool in ((kd, k_or), (vd, v_or)):
            got = to_bits(dev_pool.index_select(0, ids)).transpose(0, 2, 1, 3)  # [blk, B, H, d]
            want = ref_pool.transpose(0, 2, 1, 3)
            assert np.array_equal(got[valid], want[valid])   # every written (and copied) slot
        qd = to_dev(workloads._round_bits(rng.standard_normal((S, Hkv * G, d), dtype=np.float32),
                                          q), q)
        out = pa.decode(qd, kd, vd, dev_i32(big), dev_i32(lens), int(lens.max()), sp.scale,
                        scale, scale, partition_size=64)
        torch.cuda.synchronize()
        ref = oracle.decode(to_bits(qd), DT[q], k_or, v_or, DT[kv], small, lens, Hkv, B,
                            sp.scale, scale, scale)
        atol, rrel = (2e-2, None) if kv == "e4m3" else (2e-3, 1e-2)
        compare(_f64(out), ref, atol, rrel, q)
        # the appending decode stores above 2^32 too: one more token per sequence, equal
        # bit for bit to the KV write of that token followed by the decode
        grown = lens + 1
        kn, vn = (to_dev(workloads._round_bits(rng.standard_normal((S, Hkv, d), dtype=np.float32),
                                               q), q) for _ in range(2))
        saved = (kd[base:].clone(), vd[base:].clone())
        pa.write_kv(kn, vn, kd, vd, dev_i32(big), dev_i32(np.arange(S, dtype=np.int32)),
                    dev_i32(lens), inv, inv)
        want = pa.decode(qd, kd, vd, dev_i32(big), dev_i32(grown), int(grown.max()), sp.scale,
                         scale, scale, partition_size=64)
        torch.cuda.synchronize()
        want_pools = (to_bits(kd[base:]), to_bits(vd[base:]))
        kd[base:], vd[base:] = saved
        got = pa.decode_append(qd, kn, vn, kd, vd, dev_i32(big), dev_i32(grown), int(grown.max()),
                               sp.scale, scale, scale, inv, inv, partition_size=64)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert np.array_equal(to_bits(kd[base:]), want_pools[0])
        assert np.array_equal(to_bits(vd[base:]), want_pools[1])
    finally:
        del kd, vd
        torch.cuda.empty_cache()


@pytest.mark.parametrize("S", [128, 129])
def test_grouped_queries_skewed_rows_over_xcds(S):
    """Matrix-core decodes spread row-partitions over the XCDs by their blocks (at most 128
    rows; 129 take contiguous ranges): a few long rows among many short or empty ones, so
    the ranges cut rows apart; every row must still be decoded once and only once."""
    rng = np.random.default_rng(S)
    lens = rng.integers(0, 40, S)
    lens[rng.choice(S, 5, replace=False)] = [3000, 2047, 1500, 777, 3001]
    lens[rng.choice(S, 10, replace=False)] = 0
    B, d, G = 16, 128, 4
    sp = workloads.Spec("skew", S, 2 * G, 2, d, B, 1, 1,
                        int(sum(math.ceil(n / B) for n in lens)) + 5,
                        math.ceil(int(lens.max()) / B) + 1, "bf16", "bf16", 1 / math.sqrt(d))
    case = workloads.generate(sp, 5200 + S, context_lens=lens.tolist())
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    for P in (0, 256):
        out = _f64(_gpu_decode(case, tables, k, v, partition_size=P))
        assert (out[lens == 0] == 0).all()
        compare(out, ref, 2e-3, 1e-2, "bf16")
