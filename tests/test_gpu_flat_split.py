"""The flat split against the CPU oracle (needs an MI355X).

With fp16/bf16 caches, at most 256 sequences and a split left to the library, pa_decode
cuts the stream of all sequences' blocks (one sequence after another) into equal chunks;
a unit is (chunk, KV head), and a chunk that crosses sequence boundaries leaves one
partial per sequence, merged like any other partitions.  The cases below put chunk
boundaries everywhere a mistake would show: inside sequences, between empty sequences,
across several whole short sequences; chunks at the shortest length and longer ones; the
largest batch the split takes and the first it leaves to fixed partitions; a batch with
no token at all.  Bars as in the other parity tests ([P1] sec. 3 defines the output).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import workloads
import paged_kv_cache_89_amd as pa
from helpers import compare, dev_i32, oracle_caches, oracle_decode, oracle_tables, to_dev, tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


def _spec(lens, G, Hkv, d, B, qd, max_ctx=None):
    mc = max(lens) if max_ctx is None else max_ctx
    return workloads.Spec("flat", len(lens), G * Hkv, Hkv, d, B, 1, 1,
                          sum(math.ceil(n / B) for n in lens) + 5, math.ceil(mc / B) + 1,
                          qd, qd, 1 / math.sqrt(d))


def _run(sp, lens, seed, max_ctx=None, expect_flat=True):
    """Oracle vs GPU for one batch; checks which split the library takes."""
    case = workloads.generate(sp, seed, context_lens=lens)
    mc = int(max(lens)) if max_ctx is None else max_ctx
    plan = pa.decode_plan(sp.num_seqs, sp.num_heads, sp.num_kv_heads, sp.head_dim,
                          sp.block_size, mc, 0, pa.F16 if sp.kv_dtype == "f16" else pa.BF16)
    assert (plan[2] > 0) == expect_flat, plan
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    ref = oracle_decode(case, tables, k, v)
    q = to_dev(case.q, sp.q_dtype)
    kd, vd = to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype)
    td, cd = dev_i32(tables), dev_i32(case.context_lens)
    out = pa.decode(q, kd, vd, td, cd, mc, sp.scale)
    again = pa.decode(q, kd, vd, td, cd, mc, sp.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, again), "the same call must give the same bits"
    got = out.double().cpu().numpy()
    atol, rrel = tolerance(sp)
    compare(got, ref, atol, rrel, sp.q_dtype)
    for s, n in enumerate(lens):
        if n == 0:
            assert (got[s] == 0).all(), "n = 0 must give a zero row"
    return got


@pytest.mark.parametrize("qd", ["f16", "bf16"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_chunks_cross_short_and_empty_sequences(qd, G):
    """Few blocks in all (the chunk takes its shortest length, 16 blocks): chunks begin
    and end inside long sequences and run over several whole short and empty ones.
    G = 1 runs the vector kernel, G >= 2 the matrix-core kernel."""
    lens = [0, 700, 1, 0, 15, 16, 17, 33, 5, 0, 2000, 31, 64, 250, 0, 3, 1023, 9, 256, 257]
    for d in (64, 128):
        _run(_spec(lens, G, 2, d, 16, qd), lens, 4100 + 10 * G + d)


@pytest.mark.parametrize("qd", ["f16", "bf16"])
def test_eight_token_blocks(qd):
    lens = [0, 9, 8, 7, 1500, 0, 64, 65, 1, 800]
    _run(_spec(lens, 1, 4, 64, 8, qd), lens, 4200)


def test_chunks_longer_than_the_shortest_vector():
    """Enough blocks per wavefront that the chunk grows past 16 blocks (32 KV heads)."""
    rng = np.random.default_rng(4300)
    lens = rng.integers(1000, 3001, 20).tolist()
    lens[3] = 0
    lens[11] = 1
    _run(_spec(lens, 1, 32, 64, 16, "f16"), lens, 4301)


def test_chunks_longer_than_the_shortest_matrix_core():
    rng = np.random.default_rng(4400)
    lens = rng.integers(2000, 4001, 24).tolist()
    lens[0] = 17
    lens[7] = 0
    _run(_spec(lens, 4, 8, 128, 16, "bf16"), lens, 4401)


def test_largest_flat_batch_and_the_first_with_fixed_partitions():
    rng = np.random.default_rng(4500)
    lens = rng.integers(100, 601, 257).tolist()
    lens[5] = 0
    _run(_spec(lens[:256], 1, 2, 64, 16, "f16"), lens[:256], 4501)
    _run(_spec(lens, 1, 2, 64, 16, "f16"), lens, 4502, expect_flat=False)
    _run(_spec(lens[:256], 4, 2, 64, 16, "bf16"), lens[:256], 4503)


def test_no_token_in_the_batch():
    """Every length 0 under a bound that makes the library split: zero rows."""
    lens = [0, 0, 0, 0, 0]
    for G in (1, 4):
        sp = _spec(lens, G, 2, 128, 16, "bf16", max_ctx=1000)
        _run(sp, lens, 4600 + G, max_ctx=1000)


def test_one_sequence():
    lens = [5000]
    for G in (1, 8):
        _run(_spec(lens, G, 2, 128, 16, "f16"), lens, 4700 + G)
