"""HIP graph capture of the hot path.

Every device entry point only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronisation), so one decode step -- pa_write_kv, then pa_decode with its
partition merge, the shared-prefix decode or the multi-token decode -- can be captured once
and replayed.  Each replay, with other eager GPU work and synchronisations in between,
must reproduce the eager result bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_89_amd as pa
import workloads
from helpers import dev_i32, oracle_caches, oracle_tables, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pa.lib()
    yield
    torch.cuda.synchronize()


def _replays_match_eager(step, outs, replays=4):
    step()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(replays):
        for o in outs:
            o.fill_(float(i + 3))              # eager work between replays
        torch.randn(1 << 20, device="cuda").sum().item()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o, r), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("name,P", [("opt13b_layer", 32), ("gqa_llama", 0), ("fp8_prefix", 16)])
def test_write_and_decode_step_replays(name, P):
    case = workloads.generate(workloads.SMALL[name], 8900 + 50)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    q, kd, vd = to_dev(case.q, sp.q_dtype), to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype)
    ks, vs = to_dev(case.k_src, sp.src_dtype), to_dev(case.v_src, sp.src_dtype)
    td, cd = dev_i32(tables), dev_i32(case.context_lens)
    sid, pos = dev_i32(case.seq_ids), dev_i32(case.positions)
    mc = int(case.context_lens.max())
    S, Hq, D = q.shape
    NB, Hkv, B, _ = kd.shape
    assert pa.decode_plan(S, Hq, Hkv, D, B, mc, P)[1] >= 1
    ws = torch.empty(max(pa.decode_workspace_size(S, Hq, Hkv, D, B, mc, P), 1),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)

    def step():
        pa.write_kv(ks, vs, kd, vd, td, sid, pos, case.k_inv_scale, case.v_inv_scale)
        pa.decode(q, kd, vd, td, cd, mc, sp.scale, case.k_scale, case.v_scale,
                  partition_size=P, out=out, workspace=ws)

    _replays_match_eager(step, [out])


def test_appending_decode_replays():
    """pa_decode_append in a graph: each replay stores the same new rows and gives the
    eager output and pools."""
    case = workloads.generate(workloads.SMALL["gqa_llama"], 8900 + 52)
    sp = case.spec
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    q, kd, vd = to_dev(case.q, sp.q_dtype), to_dev(k, sp.kv_dtype), to_dev(v, sp.kv_dtype)
    td, cd = dev_i32(tables), dev_i32(case.context_lens)
    mc = int(case.context_lens.max())
    S, Hq, D = q.shape
    NB, Hkv, B, _ = kd.shape
    g = torch.Generator(device="cuda")
    g.manual_seed(8900 + 53)
    kn = torch.randn((S, Hkv, D), generator=g, device="cuda").to(q.dtype)
    vn = torch.randn((S, Hkv, D), generator=g, device="cuda").to(q.dtype)
    P = B
    assert pa.decode_plan(S, Hq, Hkv, D, B, mc, P)[1] > 1
    ws = torch.empty(pa.decode_workspace_size(S, Hq, Hkv, D, B, mc, P), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)

    def step():
        pa.decode_append(q, kn, vn, kd, vd, td, cd, mc, sp.scale, case.k_scale, case.v_scale,
                         1.0, 1.0, partition_size=P, out=out, workspace=ws)

    k0, v0 = kd.clone(), vd.clone()
    step()
    torch.cuda.synchronize()
    ref = (out.clone(), to_bits(kd), to_bits(vd))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for i in range(4):
        out.fill_(float(i + 3))        # eager work between replays; the pools go back to
        kd.copy_(k0)                   # their state before the new rows, so each replay
        vd.copy_(v0)                   # must store them again
        torch.randn(1 << 20, device="cuda").sum().item()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]), f"replay {i} differs from the eager result"
        assert np.array_equal(to_bits(kd), ref[1]) and np.array_equal(to_bits(vd), ref[2])


@pytest.mark.parametrize("Hq", [4, 2])
def test_shared_prefix_and_multi_token_replay(Hq):
    """Hq = 4 over 2 KV heads: the cascade's two decode launches; Hq = 2: its one launch
    (e4m3 cache, one query head per KV head)."""
    K, B, prompt = 4, 16, 64
    lens = [70, 90, 64, 100, 80, 65, 120, 66]
    S = len(lens)
    need = (S // K) * (prompt // B) + sum(max(0, math.ceil(n / B) - prompt // B) for n in lens) + 5
    sp = workloads.Spec("casc", S, Hq, 2, 128, B, 0, 0, need, 10, "bf16", "e4m3",
                        1 / math.sqrt(128), group_size=K, prompt_len=prompt)
    case = workloads.generate(sp, 8900 + 51, context_lens=lens)
    tables, _, _ = oracle_tables(case)
    k, v = oracle_caches(case, tables)
    q, kd, vd = to_dev(case.q, "bf16"), to_dev(k, "e4m3"), to_dev(v, "e4m3")
    td, cd = dev_i32(tables), dev_i32(case.context_lens)
    pb = dev_i32(np.full(S // K, prompt // B, np.int32))
    Hkv, D, mc, T = 2, 128, max(lens), 2
    ws_sp = torch.empty(pa.decode_shared_prefix_workspace_size(S, Hq, Hkv, D, B, mc, prompt // B),
                        dtype=torch.uint8, device="cuda")
    out_sp = torch.empty_like(q)
    qm = torch.randn((S, T, Hq, D), device="cuda").to(torch.bfloat16)
    ws_m = torch.empty(max(pa.decode_multi_workspace_size(S, T, Hq, Hkv, D, B, mc, 32), 1),
                       dtype=torch.uint8, device="cuda")
    out_m = torch.empty_like(qm)

    def step():
        pa.decode_shared_prefix(q, kd, vd, td, cd, pb, K, mc, prompt // B, sp.scale, case.k_scale,
                                case.v_scale, out=out_sp, workspace=ws_sp)
        pa.decode_multi(qm, kd, vd, td, cd, mc, sp.scale, case.k_scale, case.v_scale,
                        partition_size=32, out=out_m, workspace=ws_m)

    _replays_match_eager(step, [out_sp, out_m])


def test_block_copy_replays():
    NB, Hkv, B, d = 32, 2, 16, 64
    k = torch.randn((NB, Hkv, B, d), device="cuda").half()
    v = torch.randn((NB, Hkv, B, d), device="cuda").half()
    pairs = dev_i32(np.array([[1, 2], [3, 4], [5, 30]], np.int32))
    dst = torch.tensor([2, 4, 30], device="cuda")

    def step():
        pa.copy_blocks(k, v, pairs)

    step()
    torch.cuda.synchronize()
    ref_k, ref_v = k.clone(), v.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        k[dst] = float(i)
        v[dst] = float(-i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(k, ref_k) and torch.equal(v, ref_v)
