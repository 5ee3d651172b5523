"""GPU tests of the block lifecycle path: batched copy-on-write kernel and a parallel
sampling run (fork, append with copy-on-write, KV write, decode) through the library,
checked against the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_89_amd as pa
import workloads
from helpers import DT, compare, dev_i32, to_bits, to_dev
from oracle.lifecycle import LifecycleOracle, copy_blocks

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("kv", ["f16", "e4m3"])
def test_copy_blocks_bit_exact(kv):
    rng = np.random.default_rng(3)
    sp = workloads.Spec("c", 1, 8, 8, 128, 16, 1, 1, 64, 4, "bf16", kv, 0.1)
    k = workloads.empty_cache(sp, poison=False)
    v = workloads.empty_cache(sp, poison=False)
    k[:] = rng.integers(0, 1 << (8 * k.itemsize), k.shape, dtype=np.uint64).astype(k.dtype)
    v[:] = rng.integers(0, 1 << (8 * v.itemsize), v.shape, dtype=np.uint64).astype(v.dtype)
    perm = rng.permutation(64)
    pairs = np.stack([perm[:20], perm[20:40]], 1).astype(np.int32)
    pairs_bad = np.concatenate([pairs, [[70, 1], [2, -1]]]).astype(np.int32)  # skipped
    kd, vd = to_dev(k, kv), to_dev(v, kv)
    pa.copy_blocks(kd, vd, dev_i32(pairs_bad))
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(kd), copy_blocks(k.copy(), pairs.tolist()))
    assert np.array_equal(to_bits(vd), copy_blocks(v.copy(), pairs.tolist()))


@pytest.mark.parametrize("kv,q", [("f16", "f16"), ("bf16", "bf16"), ("e4m3", "bf16")])
def test_parallel_sampling_copy_on_write_end_to_end(kv, q):
    """Prefill a prompt whose last block is partial, fork it into 4 samples, then decode 24
    steps: each step appends a slot per sample (copy-on-write of the shared partial block on
    the first step), runs the batched copy, writes the new rows and decodes.  Tables,
    copies and the final caches match the oracle bit for bit; every step's output matches
    the oracle decode."""
    rng = np.random.default_rng(5)
    B, Hkv, Hq, d, NB, MB, K = 16, 4, 8, 128, 64, 8, 4
    prompt_len, steps = 45, 24
    sp = workloads.Spec("l", K, Hq, Hkv, d, B, 1, 1, NB, MB, q, kv, 1 / np.sqrt(d))
    free = rng.permutation(NB)
    o = LifecycleOracle.create(NB, B, free)
    bm = pa.BlockManager(NB, B, free)
    src = sp.src_dtype

    def draw(n):
        return workloads._round_bits(rng.standard_normal((n, Hkv, d), dtype=np.float32), src)

    pk, pv = draw(prompt_len), draw(prompt_len)
    scale_k = scale_v = inv_k = inv_v = 1.0
    if kv == "e4m3":
        scale_k = scale_v = float(np.float32(4.0 / 448.0))
        inv_k = inv_v = float(np.float32(1.0) / np.float32(scale_k))
    [po] = o.alloc([prompt_len])
    t_dev_np, hb = bm.alloc_tables([prompt_len], MB)
    k_or, v_or = workloads.empty_cache(sp), workloads.empty_cache(sp)
    kd, vd = to_dev(k_or, kv), to_dev(v_or, kv)
    t_or, _ = o.table([po], MB)
    pos = np.arange(prompt_len, dtype=np.int32)
    zeros = np.zeros(prompt_len, np.int32)
    oracle.scatter(pk, DT[src], k_or, DT[kv], t_or, zeros, pos, B, inv_k)
    oracle.scatter(pv, DT[src], v_or, DT[kv], t_or, zeros, pos, B, inv_v)
    pa.write_kv(to_dev(pk, src), to_dev(pv, src), kd, vd, dev_i32(t_dev_np), dev_i32(zeros),
                dev_i32(pos), inv_k, inv_v)
    so = o.fork(po, K)
    sb = bm.fork(int(hb[0]), K)
    assert sb.tolist() == so
    o.free_seqs([po])
    bm.free(hb)
    qd = to_dev(workloads._round_bits(rng.standard_normal((K, Hq, d), dtype=np.float32), q), q)
    qb = to_bits(qd)
    for step in range(steps):
        blk_o, slot_o, cp_o = o.append(so)
        blk_b, slot_b, cp_b = bm.append(sb)
        assert blk_b.tolist() == blk_o and slot_b.tolist() == slot_o
        assert [tuple(c) for c in cp_b.tolist()] == cp_o
        if step == 0:
            assert len(cp_o) == K - 1  # the shared partial prompt block, once per sample but one
        copy_blocks(k_or, cp_o)
        copy_blocks(v_or, cp_o)
        if len(cp_b):
            pa.copy_blocks(kd, vd, dev_i32(cp_b))
        tables, lens = bm.table(sb, MB)
        nk, nv = draw(K), draw(K)
        seq_ids = np.arange(K, dtype=np.int32)
        positions = (lens - 1).astype(np.int32)
        oracle.scatter(nk, DT[src], k_or, DT[kv], tables, seq_ids, positions, B, inv_k)
        oracle.scatter(nv, DT[src], v_or, DT[kv], tables, seq_ids, positions, B, inv_v)
        td = dev_i32(tables)
        pa.write_kv(to_dev(nk, src), to_dev(nv, src), kd, vd, td, dev_i32(seq_ids),
                    dev_i32(positions), inv_k, inv_v)
        out = pa.decode(qd, kd, vd, td, dev_i32(lens), int(lens.max()), sp.scale, scale_k,
                        scale_v, flags=pa.DECODE_SHARED_KV)
        torch.cuda.synchronize()
        ref = oracle.decode(qb, DT[q], k_or, v_or, DT[kv], tables, lens, Hkv, B, sp.scale,
                            scale_k, scale_v)
        atol, rrel = (2e-2, None) if kv == "e4m3" else (2e-3, 1e-2)
        compare(out.double().cpu().numpy(), ref, atol, rrel, q)
    assert np.array_equal(to_bits(kd), k_or) and np.array_equal(to_bits(vd), v_or)
