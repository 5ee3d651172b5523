"""Seeded synthetic inputs for the paged decode operator.

Shared by the tests, the smoke check and the benchmark.  This module holds none
of the operator's arithmetic: it draws random numbers, rounds them to a storage
dtype with numpy/torch library conversions, shuffles free lists and lays out the
list of tokens a caller would write.  Block tables, cache scatters and attention
outputs are computed elsewhere (by the library under test, or by the oracle).

Workloads (the five decode shapes the operator is measured on):

* ``tiny_mha``      4 seqs, 8 heads, d 64, B 16, n ~ U[1,256], fp16, 64 blocks, scale 1/8
* ``opt13b_layer``  64 seqs, 40 heads, d 128, B 16, n ~ U[512,2048], fp16, 8192 blocks
* ``gqa_llama``     128 seqs, 32 q heads / 8 KV heads, d 128, B 16, n ~ U[1024,8192], bf16
* ``long_split``    8 seqs, 32 heads, d 128, B 32, n = 32768, fp16, partitions of 512
* ``fp8_prefix``    64 prompts x 4 samples, 32 heads, d 128, B 16, prompt 1024 shared +
                    U[0,512] private tokens, bf16 Q, e4m3 K/V with per-tensor scales

Draw order for a seed: context lengths, free-list permutation, Q, K, V.
Values are N(0,1) in binary32 rounded to nearest even into the storage dtype;
an e4m3 cache gets per-tensor scale = amax / 448 over its source values.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

DTYPE_BYTES = {"f16": 2, "bf16": 2, "e4m3": 1}


@dataclass(frozen=True)
class Spec:
    name: str
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    ctx_lo: int            # inclusive range of context lengths (private part for prefix workloads)
    ctx_hi: int
    num_blocks: int
    max_blocks: int
    q_dtype: str
    kv_dtype: str
    scale: float
    partition_size: int = 0     # 0: let the library choose
    group_size: int = 0         # samples sharing one prompt (0: no sharing)
    prompt_len: int = 0

    @property
    def src_dtype(self) -> str:
        """dtype of the new K/V rows handed to the cache writer."""
        return self.q_dtype if self.kv_dtype == "e4m3" else self.kv_dtype

    def replace(self, **kw) -> "Spec":
        return dataclasses.replace(self, **kw)


SPECS = {
    "tiny_mha": Spec("tiny_mha", 4, 8, 8, 64, 16, 1, 256, 64, 16, "f16", "f16", 1.0 / 8),
    "opt13b_layer": Spec("opt13b_layer", 64, 40, 40, 128, 16, 512, 2048, 8192, 128,
                         "f16", "f16", 1.0 / math.sqrt(128)),
    "gqa_llama": Spec("gqa_llama", 128, 32, 8, 128, 16, 1024, 8192, 65536, 512,
                      "bf16", "bf16", 1.0 / math.sqrt(128)),
    "long_split": Spec("long_split", 8, 32, 32, 128, 32, 32768, 32768, 8192, 1024,
                       "f16", "f16", 1.0 / math.sqrt(128), partition_size=512),
    "fp8_prefix": Spec("fp8_prefix", 256, 32, 32, 128, 16, 0, 512, 12288, 96,
                       "bf16", "e4m3", 1.0 / math.sqrt(128), group_size=4, prompt_len=1024),
}

# Reduced shapes that keep each workload's head_dim, block size, grouping, dtypes and
# length mix (several tiles and a ragged tail) but that the CPU oracle finishes in seconds.
SMALL = {
    "tiny_mha": SPECS["tiny_mha"],
    "opt13b_layer": SPECS["opt13b_layer"].replace(num_seqs=6, num_heads=4, num_kv_heads=4,
                                                  num_blocks=6 * 128 + 16),
    "gqa_llama": SPECS["gqa_llama"].replace(num_seqs=4, num_heads=8, num_kv_heads=2,
                                            num_blocks=4 * 512 + 8),
    "long_split": SPECS["long_split"].replace(num_seqs=2, num_heads=2, num_kv_heads=2,
                                              num_blocks=2 * 1024),
    "fp8_prefix": SPECS["fp8_prefix"].replace(num_seqs=8, num_heads=4, num_kv_heads=4,
                                              num_blocks=2 * 64 + 8 * 32),
}


def _round_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """binary32 -> fp16/bf16 storage bits (library round-to-nearest-even)."""
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16) \
            .numpy().view(np.uint16)
    raise ValueError(dtype)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """fp16/bf16 storage bits -> binary32 (exact widening, library routines)."""
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


@dataclass
class Case:
    """One seeded batch.  All arrays are numpy, storage dtypes as raw bits."""
    spec: Spec
    context_lens: np.ndarray        # int32 [S]
    free_order: np.ndarray          # int32 [NB], a permutation
    prefix_group: np.ndarray | None  # int32 [S] (-1 none) or None
    prefix_lens: np.ndarray | None   # int32 [num_groups] or None
    q: np.ndarray                   # uint16 [S, Hq, d]
    seq_ids: np.ndarray             # int32 [T]   the token writes that fill the cache
    positions: np.ndarray           # int32 [T]
    k_src: np.ndarray               # uint16 [T, Hkv, d] in spec.src_dtype
    v_src: np.ndarray
    token_index: np.ndarray         # int32 [S, max n]: write-list row of logical token t (-1 pad)
    k_scale: float = 1.0
    v_scale: float = 1.0
    k_inv_scale: float = 1.0
    v_inv_scale: float = 1.0

    def logical(self, s: int, which: str = "k") -> np.ndarray:
        """Sequence s's logical rows [n_s, Hkv, d] (source bits), before any paging."""
        src = self.k_src if which == "k" else self.v_src
        n = int(self.context_lens[s])
        return src[self.token_index[s, :n]]


def generate(spec: Spec, seed: int, context_lens=None) -> Case:
    """Seeded batch for `spec` (draw order: lengths, free list, Q, K, V)."""
    rng = np.random.default_rng(seed)
    S, Hq, Hkv, d, B = spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    drawn = rng.integers(spec.ctx_lo, spec.ctx_hi + 1, size=S).astype(np.int32)
    if context_lens is None:
        ctx = drawn + spec.prompt_len
    else:
        ctx = np.asarray(context_lens, np.int32)
    ctx = ctx.astype(np.int32)
    free_order = rng.permutation(spec.num_blocks).astype(np.int32)
    q32 = rng.standard_normal((S, Hq, d), dtype=np.float32)
    q = _round_bits(q32, spec.q_dtype)

    prefix_group = prefix_lens = None
    shared_tok = 0
    if spec.group_size:
        assert S % spec.group_size == 0
        ngroups = S // spec.group_size
        prefix_group = (np.arange(S) // spec.group_size).astype(np.int32)
        prefix_lens = np.full(ngroups, spec.prompt_len, np.int32)
        shared_tok = (spec.prompt_len // B) * B

    # Token write list: each group's prompt rows are drawn once; tokens that live in the
    # group's shared blocks are written once (by the group's first sequence), the rest of
    # the prompt is written into every member's own blocks; private tokens follow.
    seq_ids, positions, rows_of = [], [], []
    token_index = np.full((S, int(ctx.max()) if S else 0), -1, np.int32)
    prompt_row = {}
    nrows = 0
    if prefix_group is None:  # no sharing: every sequence's tokens in order, all new rows
        lens = np.maximum(ctx, 0).astype(np.int64)
        seq_ids = np.repeat(np.arange(S), lens).tolist()
        positions = np.concatenate([np.arange(n) for n in lens]).tolist() if S else []
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]) if S else np.zeros(0, np.int64)
        for s in range(S):
            token_index[s, :lens[s]] = starts[s] + np.arange(lens[s])
        nrows = int(lens.sum())
        rows_of = [("new", None)] * nrows
    for s in (range(S) if prefix_group is not None else ()):
        n = int(ctx[s])
        g = -1 if prefix_group is None else int(prefix_group[s])
        for t in range(n):
            if g >= 0 and t < spec.prompt_len:
                key = (g, t)
                if t < shared_tok and key in prompt_row:
                    token_index[s, t] = prompt_row[key]
                    continue
                if key in prompt_row:          # partial prompt block: same values, own slot
                    rows_of.append(("copy", prompt_row[key]))
                else:
                    rows_of.append(("new", None))
                    prompt_row[key] = nrows
            else:
                rows_of.append(("new", None))
            seq_ids.append(s)
            positions.append(t)
            token_index[s, t] = nrows
            nrows += 1
    T = nrows
    n_new = sum(1 for kind, _ in rows_of if kind == "new")
    k32_new = rng.standard_normal((n_new, Hkv, d), dtype=np.float32)
    v32_new = rng.standard_normal((n_new, Hkv, d), dtype=np.float32)
    k32 = np.empty((T, Hkv, d), np.float32)
    v32 = np.empty((T, Hkv, d), np.float32)
    j = 0
    if n_new == T:  # every row new: the drawn rows in order
        k32, v32, rows_of = k32_new, v32_new, []
    for r, (kind, src) in enumerate(rows_of):
        if kind == "new":
            k32[r] = k32_new[j]
            v32[r] = v32_new[j]
            j += 1
        else:
            k32[r] = k32[src]
            v32[r] = v32[src]
    src_dtype = spec.src_dtype
    k_src = _round_bits(k32, src_dtype)
    v_src = _round_bits(v32, src_dtype)
    case = Case(spec, ctx, free_order, prefix_group, prefix_lens, q,
                np.asarray(seq_ids, np.int32), np.asarray(positions, np.int32),
                k_src, v_src, token_index)
    if spec.kv_dtype == "e4m3":
        for which, bits in (("k", k_src), ("v", v_src)):
            amax = np.float32(np.abs(bits_to_f32(bits, src_dtype)).max()) if T else np.float32(1)
            sc = np.float32(amax / np.float32(448.0))
            inv = np.float32(np.float32(1.0) / sc)
            setattr(case, f"{which}_scale", float(sc))
            setattr(case, f"{which}_inv_scale", float(inv))
    return case


def poison_bits(dtype: str) -> int:
    """A NaN storage pattern for unused cache slots."""
    return {"f16": 0x7E00, "bf16": 0x7FC0, "e4m3": 0x7F}[dtype]


def empty_cache(spec: Spec, poison: bool = True) -> np.ndarray:
    """A [NB, Hkv, B, d] cache pool of storage bits, NaN-filled when `poison`."""
    shape = (spec.num_blocks, spec.num_kv_heads, spec.block_size, spec.head_dim)
    dt = np.uint8 if spec.kv_dtype == "e4m3" else np.uint16
    return np.full(shape, poison_bits(spec.kv_dtype) if poison else 0, dt)


def kv_bytes(spec: Spec, context_lens) -> int:
    """Algorithmic K+V bytes one decode pass reads: sum_s n_s * Hkv * d * 2 * e."""
    return int(np.sum(np.asarray(context_lens, np.int64))) * spec.num_kv_heads * spec.head_dim \
        * 2 * DTYPE_BYTES[spec.kv_dtype]


# ----------------------------------------------------------------- device-side inputs
def device_pool(spec: Spec, seed: int, device="cuda"):
    """Full-size pools drawn directly on the device with torch's seeded generator.

    Returns (q, k_cache, v_cache, k_scale, v_scale) as torch tensors; every slot of
    every block holds N(0,1) data (e4m3: scaled by amax/448), so any table is valid.
    """
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    S, Hq, Hkv, d, B, NB = (spec.num_seqs, spec.num_heads, spec.num_kv_heads, spec.head_dim,
                            spec.block_size, spec.num_blocks)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    q = torch.randn((S, Hq, d), generator=g, device=device, dtype=torch.float32).to(tdt[spec.q_dtype])
    caches, scales = [], []
    for _ in range(2):
        x = torch.randn((NB, Hkv, B, d), generator=g, device=device, dtype=torch.float32)
        if spec.kv_dtype == "e4m3":
            x = x.to(tdt[spec.src_dtype]).float()
            sc = (x.abs().max() / 448.0).item()
            inv = float(np.float32(1.0) / np.float32(sc))
            c = (x * inv).to(torch.float8_e4m3fn).view(torch.uint8)
            scales.append(float(np.float32(sc)))
        else:
            c = x.to(tdt[spec.kv_dtype])
            scales.append(1.0)
        del x
        caches.append(c)
    return q, caches[0], caches[1], scales[0], scales[1]


def draw_lengths(spec: Spec, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Context lengths and free-list order for `spec` (same draws as `generate`)."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(spec.ctx_lo, spec.ctx_hi + 1, size=spec.num_seqs).astype(np.int32) \
        + spec.prompt_len
    free_order = rng.permutation(spec.num_blocks).astype(np.int32)
    return ctx.astype(np.int32), free_order


def prefix_groups(spec: Spec):
    if not spec.group_size:
        return None, None
    S = spec.num_seqs
    pg = (np.arange(S) // spec.group_size).astype(np.int32)
    pl = np.full(S // spec.group_size, spec.prompt_len, np.int32)
    return pg, pl
