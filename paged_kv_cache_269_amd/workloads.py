"""Seeded synthetic inputs for paged decode attention.

This module is the only code that both the HIP path's tests/benchmark and the
float64 oracle consume.  It draws lengths, block permutations and N(0,1) data,
lays them out in the pool the way an engine's block allocator would, and does
none of the attention arithmetic.

Recipe (numpy ``SeedSequence(seed)`` spawned into independent streams, drawn
in this order: lengths, block permutation, q, K pool, V pool, new-token K,
new-token V):

* Context length L_s counts every cached token including the one being decoded;
  that newest token is written by reshape_and_cache at logical position L_s-1.
* Pages hold 16 tokens ("vLLM 2026 推理引擎全解" (chenxutan.com), §2.1); a
  sequence needs ceil(L_s/16) of them, the allocation rule of the vLLM manual
  (doramagic.ai), KVCacheManager cache-block management.
* Physical ids come from one seeded permutation of the pool; sequences take
  consecutive ids of it in order, so physical pages are scattered (§2.1's
  example of non-contiguous pages).  A shared prefix takes the first ids and
  every sequence's table points at them (§2.3 of the same page).
* Pool size: ceil(1.2 x pages needed), shared pages counted once; the tiny
  workload uses a fixed 32-page pool.
* Values: float32 N(0,1) rounded to nearest-even into the element type.
  bfloat16 arrays are held as uint16 bit patterns.
* Multi-token queries (generate_query_spans): q rows for the last n_s tokens
  of each context, N(0,1) from their own seed; the cache already holds those
  tokens' K/V.
* Poison (parity runs): every slot no sequence owns -- the tail of a last
  page, pages nobody uses and the slot the new token is about to fill -- is
  NaN, so a read of it shows up in the output.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

BLOCK_SIZE = 16
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NP_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}

# The five decode workloads (one layer each).  ``lens`` gives fixed lengths;
# otherwise ``len_dist`` draws them.  ``len_cap`` sizes the block-table rows.
# ``partition_size`` is the launch configuration the benchmark times: 0 (one
# pass per sequence) where that measured fastest, 512-token partitions with
# the log-sum-exp reduce for the long-context workload, whose definition
# fixes them.  ``cascade`` marks the workload whose batch shares prompt pages:
# it is decoded through the cascade entry point, which attends each run's
# shared pages once.
CONFIGS: Dict[str, dict] = {
    "tiny": dict(dtype="f32", num_seqs=4, num_q_heads=4, num_kv_heads=4, head_dim=64,
                 len_dist="fixed", lens=[1, 17, 33, 50], pool_blocks=32,
                 partition_size=512, seed=1),
    "llama7b": dict(dtype="f16", num_seqs=64, num_q_heads=32, num_kv_heads=32, head_dim=128,
                    len_dist="uniform", len_lo=512, len_hi=2048,
                    partition_size=0, seed=2),
    "gqa": dict(dtype="bf16", num_seqs=128, num_q_heads=64, num_kv_heads=8, head_dim=128,
                len_dist="lognormal", len_median=2048, len_sigma=0.5, len_cap=8192,
                partition_size=0, seed=3),
    "shared_prefix": dict(dtype="bf16", num_seqs=256, num_q_heads=32, num_kv_heads=32,
                          head_dim=128, len_dist="uniform", len_lo=64, len_hi=512,
                          shared_prefix_blocks=64, partition_size=0, cascade=True, seed=4),
    "long_context": dict(dtype="bf16", num_seqs=8, num_q_heads=64, num_kv_heads=8,
                         head_dim=128, len_dist="uniform", len_lo=32768, len_hi=131072,
                         partition_size=512, seed=5),
}
CONFIG_ORDER = ["tiny", "llama7b", "gqa", "shared_prefix", "long_context"]


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    partition_size: int
    shared_prefix_blocks: int
    context_lens: np.ndarray   # [B] int32, includes the new token
    block_tables: np.ndarray   # [B, M] int32
    slot_mapping: np.ndarray   # [T] int64 (T = B, one new token per sequence)
    q: np.ndarray              # [B, Hq, D]
    key: np.ndarray            # [T, Hkv, D] new tokens' K
    value: np.ndarray          # [T, Hkv, D] new tokens' V
    k_cache: np.ndarray        # [N, Hkv, 16, D] pool before the write
    v_cache: np.ndarray
    params: dict

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def _round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage type, round-to-nearest-even (inputs are finite)."""
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16)
    u = x.view(np.uint32)
    return ((u + (0x7FFF + ((u >> 16) & 1))) >> 16).astype(np.uint16)


def _normal(ss: np.random.SeedSequence, shape, dtype: str) -> np.ndarray:
    x = np.random.default_rng(ss).standard_normal(int(np.prod(shape)), dtype=np.float32)
    return _round_to_dtype(x, dtype).reshape(shape)


def _normal_pool(ss: np.random.SeedSequence, shape, dtype: str,
                 chunk: int = 1 << 22, threads: Optional[int] = None) -> np.ndarray:
    """Large N(0,1) array filled in fixed chunks, each from its own spawned
    stream, so the bytes do not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, NP_STORAGE[dtype])
    nchunks = max(1, (n + chunk - 1) // chunk)
    kids = ss.spawn(nchunks)

    def fill(i):
        lo, hi = i * chunk, min(n, (i + 1) * chunk)
        x = np.random.default_rng(kids[i]).standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = _round_to_dtype(x, dtype)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nchunks == 1 or threads <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _nan_fill(a: np.ndarray, dtype: str, index) -> None:
    if dtype == "f32":
        a[index] = np.nan
    else:  # a quiet-NaN bit pattern (f16 pools are float16, bf16 pools uint16 bits)
        a.view(np.uint16)[index] = _NAN_BITS[dtype]


def _draw_lengths(rng: np.random.Generator, p: dict) -> np.ndarray:
    B = p["num_seqs"]
    dist = p["len_dist"]
    if dist == "fixed":
        lens = np.asarray(p["lens"], np.int64)
        if lens.shape[0] != B:
            raise ValueError("fixed lens must have num_seqs entries")
    elif dist == "uniform":
        lens = rng.integers(p["len_lo"], p["len_hi"], size=B, endpoint=True)
    elif dist == "lognormal":
        x = rng.normal(math.log(p["len_median"]), p["len_sigma"], size=B)
        lens = np.clip(np.rint(np.exp(x)), 1, p["len_cap"]).astype(np.int64)
    else:
        raise ValueError(f"unknown length distribution {dist!r}")
    return lens.astype(np.int64) + _bs(p) * p.get("shared_prefix_blocks", 0)


def _bs(p: dict) -> int:
    return int(p.get("block_size", BLOCK_SIZE))


def _len_cap(p: dict) -> int:
    prefix = _bs(p) * p.get("shared_prefix_blocks", 0)
    if p["len_dist"] == "fixed":
        return int(max(p["lens"])) + prefix
    if p["len_dist"] == "uniform":
        return int(p["len_hi"]) + prefix
    return int(p["len_cap"]) + prefix


def config_params(name: str, **overrides) -> dict:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; have {sorted(CONFIGS)}")
    p = dict(CONFIGS[name])
    p.update({k: v for k, v in overrides.items() if v is not None})
    if "lens" in overrides and overrides["lens"] is not None:
        p["len_dist"] = "fixed"
        p["num_seqs"] = len(overrides["lens"])
    return p


def generate(name: str, poison: bool = True, threads: Optional[int] = None,
             **overrides) -> Workload:
    """Build one seeded workload.  Overrides (num_seqs, lens, len_lo, len_hi,
    num_q_heads, num_kv_heads, head_dim, dtype, seed, pool_blocks, scale,
    partition_size, shared_prefix_blocks, ...) give the smaller parity cases."""
    p = config_params(name, **overrides)
    dtype = p["dtype"]
    B, Hq, Hkv, D = p["num_seqs"], p["num_q_heads"], p["num_kv_heads"], p["head_dim"]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    shared = int(p.get("shared_prefix_blocks", 0))
    bs = int(p.get("block_size", BLOCK_SIZE))
    root = np.random.SeedSequence(p["seed"])
    s_len, s_perm, s_q, s_k, s_v, s_nk, s_nv = root.spawn(7)

    lens = _draw_lengths(np.random.default_rng(s_len), p)
    if shared and np.any(lens <= bs * shared):
        raise ValueError("shared-prefix sequences need a private suffix")
    pages = (lens + bs - 1) // bs
    private_pages = pages - shared
    needed = int(shared + private_pages.sum())
    if "pool_blocks" in p:
        N = int(p["pool_blocks"])
        if N < needed:
            raise ValueError("pool too small for the drawn lengths")
    else:
        N = int(math.ceil(1.2 * needed))
    M = max(1, (_len_cap(p) + bs - 1) // bs)
    if int(pages.max(initial=0)) > M:
        raise ValueError("a drawn length exceeds the block-table row")

    perm = np.random.default_rng(s_perm).permutation(N).astype(np.int32)
    guard = int(perm[needed]) if needed < N else 0
    tables = np.full((B, M), guard, np.int32)
    cursor = shared
    for s in range(B):
        tables[s, :shared] = perm[:shared]
        n = int(private_pages[s])
        tables[s, shared:shared + n] = perm[cursor:cursor + n]
        cursor += n

    # newest token of each sequence sits at logical position L-1; an empty
    # sequence writes nothing (slot -1)
    last = np.maximum(lens - 1, 0)
    slots = (tables[np.arange(B), last // bs].astype(np.int64) * bs
             + last % bs).astype(np.int64)
    slots[lens == 0] = -1

    q = _normal(s_q, (B, Hq, D), dtype)
    k_cache = _normal_pool(s_k, (N, Hkv, bs, D), dtype, threads=threads)
    v_cache = _normal_pool(s_v, (N, Hkv, bs, D), dtype, threads=threads)
    key = _normal(s_nk, (B, Hkv, D), dtype)
    value = _normal(s_nv, (B, Hkv, D), dtype)

    if poison:
        used = np.zeros(N, bool)
        used[perm[:needed]] = True
        for cache in (k_cache, v_cache):
            _nan_fill(cache, dtype, ~used)
            for s in range(B):
                tail = int(lens[s] % bs)
                if tail:
                    _nan_fill(cache, dtype, (tables[s, pages[s] - 1], slice(None), slice(tail, None)))
            w_ = slots[slots >= 0]
            _nan_fill(cache, dtype, (w_ // bs, slice(None), w_ % bs))

    scale = float(p.get("scale", 1.0 / math.sqrt(D)))
    return Workload(name=name, dtype=dtype, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, block_size=bs, num_blocks=N, max_blocks_per_seq=M,
                    scale=scale, partition_size=int(p.get("partition_size", 512)),
                    shared_prefix_blocks=shared, context_lens=lens.astype(np.int32),
                    block_tables=tables, slot_mapping=slots, q=q, key=key, value=value,
                    k_cache=k_cache, v_cache=v_cache, params=p)


# ---------------------------------------------------------------------------
# several new query tokens per sequence (chunked prefill, drafted tokens)

@dataclasses.dataclass
class QuerySpans:
    q: np.ndarray            # [T, Hq, D] query rows, token-major
    query_start: np.ndarray  # [B + 1] int32
    query_lens: np.ndarray   # [B] int32
    max_query_len: int

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])


def generate_query_spans(w: Workload, query_lens, seed: int = 0) -> QuerySpans:
    """Query rows for the last n_s tokens of every context of ``w`` (their K/V
    are the pool's own, in place once the workload's KV write has run).
    ``query_lens``: one int for every sequence (capped at its length) or one
    per sequence, taken as given; q ~ N(0, 1) rounded into the workload's
    element type, drawn from SeedSequence(seed)."""
    B = w.num_seqs
    if np.ndim(query_lens) == 0:
        n = np.minimum(int(query_lens), w.context_lens).astype(np.int64)
    else:
        n = np.asarray(query_lens, np.int64)
        if n.shape != (B,) or (n < 0).any():
            raise ValueError("one non-negative query length per sequence")
    qs = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    q = _normal(np.random.SeedSequence(seed), (int(qs[-1]), w.num_q_heads, w.head_dim), w.dtype)
    return QuerySpans(q=q, query_start=qs, query_lens=n.astype(np.int32),
                      max_query_len=max(1, int(n.max(initial=0))))


def multi_query_flops(w: Workload, spans: QuerySpans) -> int:
    """Score and output products of a multi-query pass: query token i of a
    span sees p + 1 = L - n + i + 1 tokens; per query head and seen token a
    D-long dot product and a D-long multiply-add, 2 flops each."""
    seen = 0
    for L, n in zip(w.context_lens.astype(np.int64), spans.query_lens.astype(np.int64)):
        p1 = np.maximum(L - n + np.arange(n) + 1, 0)
        seen += int(p1.sum())
    return 4 * seen * w.num_q_heads * w.head_dim


# ---------------------------------------------------------------------------
# byte accounting (measurement, not part of the computed result)

def kv_bytes_per_token(num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one token in one layer: 2 * H * D * dtype_size, the per-token
    factor of the KV-size formula on "vLLM 2026 推理引擎全解" §1.1 and the
    vLLM tutorial (mjmagnets.cn) §2."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def kv_cache_bytes(context_len: int, num_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return context_len * kv_bytes_per_token(num_kv_heads, head_dim, elem_bytes)


def algorithmic_bytes(w: Workload, unique: bool = True) -> Dict[str, int]:
    """Bytes one decode step must move at minimum: K and V of every context
    token (shared-prefix pages once when ``unique``), q in and out, the table
    entries actually used and the lengths.  Partial results, page padding and
    re-reads are overhead and are not counted."""
    e = w.elem_bytes
    per_tok = kv_bytes_per_token(w.num_kv_heads, w.head_dim, e)
    lens = w.context_lens.astype(np.int64)
    total_tokens = int(lens.sum())
    if unique and w.shared_prefix_blocks:
        prefix = w.block_size * w.shared_prefix_blocks
        kv_tokens = prefix + int((lens - prefix).sum())
    else:
        kv_tokens = total_tokens
    kv = kv_tokens * per_tok
    qo = 2 * w.num_seqs * w.num_q_heads * w.head_dim * e
    pages = int(((lens + w.block_size - 1) // w.block_size).sum())
    meta = 4 * pages + 4 * w.num_seqs
    return dict(kv=kv, q_out=qo, meta=meta, total=kv + qo + meta,
                logical_kv=total_tokens * per_tok)


def reshape_bytes(w: Workload) -> int:
    """Bytes the KV write moves on its own: read the new K/V rows, write
    them, read the slots."""
    rows = 2 * w.slot_mapping.shape[0] * w.num_kv_heads * w.head_dim * w.elem_bytes
    return 2 * rows + 8 * w.slot_mapping.shape[0]


def step_bytes(w: Workload) -> int:
    """Algorithmic bytes of one decode step (KV write + decode): those of
    algorithmic_bytes -- whose K/V of every context token already include
    each new token's row, read once -- plus the new rows written and the
    slots read.  An implementation that writes the rows and then reads them
    back from the cache moves more; the re-read is overhead."""
    rows = 2 * w.slot_mapping.shape[0] * w.num_kv_heads * w.head_dim * w.elem_bytes
    return algorithmic_bytes(w, unique=True)["total"] + rows + 8 * w.slot_mapping.shape[0]


# ---------------------------------------------------------------------------
# synthetic split-K partials (inputs for testing the merge on its own)

@dataclasses.dataclass
class Partials:
    context_lens: np.ndarray  # [B] int32
    max_logits: np.ndarray    # [B, Hq, P] float32
    exp_sums: np.ndarray      # [B, Hq, P] float32
    tmp_out: np.ndarray       # [B, Hq, P, D] float32
    num_parts: np.ndarray     # [B] int32 = ceil(L / partition_size)
    partition_size: int


def generate_partials(seed: int, num_seqs: int, num_q_heads: int, head_dim: int,
                      partition_size: int, lens: Optional[List[int]] = None,
                      len_hi: int = 4096, poison: bool = True) -> Partials:
    """Random but well-formed partials: max logit ~ N(0, 4), sum of weights in
    [1, partition tokens], normalised output ~ N(0, 1).  Slots past a
    sequence's partition count are NaN when ``poison``."""
    ss = np.random.SeedSequence(seed)
    s_len, s_m, s_l, s_o = ss.spawn(4)
    if lens is None:
        lens_a = np.random.default_rng(s_len).integers(1, len_hi, size=num_seqs, endpoint=True)
    else:
        lens_a = np.asarray(lens, np.int64)
        num_seqs = lens_a.shape[0]
    nparts = (lens_a + partition_size - 1) // partition_size
    P = max(1, int(nparts.max(initial=0)))
    m = (np.random.default_rng(s_m).standard_normal((num_seqs, num_q_heads, P), np.float32) * 4)
    tokens = np.minimum(partition_size, np.maximum(
        1, lens_a[:, None] - partition_size * np.arange(P)[None, :])).astype(np.float32)
    u = np.random.default_rng(s_l).random((num_seqs, num_q_heads, P), dtype=np.float32)
    l = (1.0 + u * (tokens[:, None, :] - 1.0)).astype(np.float32)
    o = np.random.default_rng(s_o).standard_normal((num_seqs, num_q_heads, P, head_dim),
                                                   np.float32)
    if poison:
        dead = np.arange(P)[None, :] >= nparts[:, None]   # [B, P]
        m[dead[:, None, :].repeat(num_q_heads, 1)] = np.nan
        l[dead[:, None, :].repeat(num_q_heads, 1)] = np.nan
        o[dead[:, None, :].repeat(num_q_heads, 1)] = np.nan
    return Partials(context_lens=lens_a.astype(np.int32), max_logits=m, exp_sums=l,
                    tmp_out=o, num_parts=nparts.astype(np.int32),
                    partition_size=partition_size)


def to_device(w: Workload, device="cuda") -> Dict[str, "object"]:
    """Upload a workload into torch tensors (device memory plumbing only)."""
    import torch

    def t(a, is_data=True):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if is_data and w.dtype == "bf16":
            x = x.view(torch.bfloat16)
        return x.to(device)

    return dict(q=t(w.q), key=t(w.key), value=t(w.value), k_cache=t(w.k_cache),
                v_cache=t(w.v_cache), block_tables=t(w.block_tables, False),
                context_lens=t(w.context_lens, False), slot_mapping=t(w.slot_mapping, False))


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
