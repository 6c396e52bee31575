"""The entry points at the limits their declarations state, against the oracle.

* 65535 sequences (the largest num_seqs: sequences are a grid dimension),
  past the 256 sequences up to which decode items take the longest-first
  order: the vector path (MHA) and the matrix-core path (8 query heads per KV
  head, bf16 and f16) and the one-call step, every output row.
* One context cut into 2500 partitions (16-token partitions of 40000
  tokens): the workgroup-per-row reduce sweeps its weights in chunks of 512.
* 65535 query tokens in one multi-query call (the largest num_query_tokens),
  120 rows per KV head (wide items), bf16 and f16, every row.
* The reduce alone with 1100 partitions a row.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_269_amd import workloads as W

from parity import Run, check_close, oracle_all, tensor_to_np, to_f64

pytestmark = pytest.mark.gpu

MAX_GRID = 65535


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def tiny_lens(n, hi, seed):
    return np.random.default_rng(seed).integers(0, hi + 1, n).tolist()


def pool_for(lens):
    """A pool 1.2x the blocks the lengths need."""
    return int(1.2 * sum((L + 15) // 16 for L in lens)) + 4


@pytest.mark.parametrize("dtype,G", [("f16", 1), ("bf16", 8), ("f16", 8)])
def test_decode_max_sequences(cuda, dtype, G):
    import paged_kv_cache_269_amd as pa
    announce("decode, sequences", MAX_GRID, dtype, "G", G)
    lens = tiny_lens(MAX_GRID, 40, 3)
    w = W.generate("tiny", dtype=dtype, num_seqs=MAX_GRID, num_kv_heads=2, num_q_heads=2 * G,
                   head_dim=64, lens=lens, pool_blocks=pool_for(lens), seed=31)
    run = Run(w, cuda)
    d = run.dev
    # one-call step first (KV write inside the decode launch) ...
    out_fused = torch.full_like(d["q"], float("nan"))
    pa.reshape_and_decode(out_fused, d["q"], d["key"], d["value"], d["k_cache"], d["v_cache"],
                          d["slot_mapping"], d["block_tables"], d["context_lens"], w.scale,
                          w.max_context_len)
    # ... then decode alone on the written pool
    out = run.decode(partition_size=0)
    run.oracle_reshape()
    ref = oracle_all(w)
    got = to_f64(tensor_to_np(out, w.dtype), w.dtype)
    check_close(got, ref, w.dtype, f"decode {MAX_GRID} sequences")
    got_fused = to_f64(tensor_to_np(out_fused, w.dtype), w.dtype)
    check_close(got_fused, ref, w.dtype, f"one-call step {MAX_GRID} sequences")
    # the written pool is the oracle's, bit for bit (NaN poison included)
    for dev_pool, host_pool in ((d["k_cache"], w.k_cache), (d["v_cache"], w.v_cache)):
        assert np.array_equal(tensor_to_np(dev_pool, w.dtype).view(np.uint16),
                              host_pool.view(np.uint16))


def test_decode_thousands_of_partitions(cuda):
    announce("decode, 2500 partitions")
    w = W.generate("long_context", dtype="bf16", num_seqs=2, num_kv_heads=2, num_q_heads=4,
                   head_dim=128, lens=[40000, 17], seed=32)
    run = Run(w, cuda)
    run.reshape()
    run.oracle_reshape()
    got = to_f64(tensor_to_np(run.decode(partition_size=16), w.dtype), w.dtype)
    check_close(got, oracle_all(w), w.dtype, "16-token partitions of 40000 tokens")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_multi_query_max_tokens(cuda, dtype):
    import paged_kv_cache_269_amd as pa
    nseq, n = MAX_GRID // 15, 15          # 4369 sequences x 15 tokens = 65535
    announce("multi-query, query tokens", nseq * n, dtype)
    lens = (np.random.default_rng(4).integers(n, 60, nseq)).tolist()
    w = W.generate("tiny", dtype=dtype, num_seqs=nseq, num_kv_heads=2, num_q_heads=16,
                   head_dim=64, lens=lens, pool_blocks=pool_for(lens), seed=33)
    run = Run(w, cuda)
    run.reshape()
    run.oracle_reshape()
    spans = W.generate_query_spans(w, n, seed=34)
    assert spans.q.shape[0] == MAX_GRID
    d = run.dev
    q = torch.from_numpy(spans.q)
    q = (q.view(torch.bfloat16) if dtype == "bf16" else q).to(cuda)
    qs = torch.from_numpy(spans.query_start).to(cuda)
    out = torch.full_like(q, float("nan"))
    pa.paged_attention_multi_query(out, q, d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], qs, w.scale, w.max_context_len,
                                   spans.max_query_len)
    torch.cuda.synchronize()
    got = to_f64(tensor_to_np(out, dtype), dtype)
    ref = oracle.multi_query(spans.q, w.k_cache, w.v_cache, w.block_tables, w.context_lens,
                             spans.query_start, w.scale, w.dtype)
    check_close(got, ref, dtype, f"multi-query {MAX_GRID} tokens {dtype}")


def test_reduce_over_a_thousand_partitions(cuda):
    import paged_kv_cache_269_amd as pa
    part = 16
    announce("reduce, 1100 partitions")
    p = W.generate_partials(seed=35, num_seqs=3, num_q_heads=4, head_dim=128,
                            partition_size=part, lens=[1100 * part, 513 * part + 3, 5])
    B, Hq, P = p.max_logits.shape
    R = B * Hq
    ref = oracle.lse_merge(np.nan_to_num(p.max_logits.reshape(R, P)),
                           np.nan_to_num(p.exp_sums.reshape(R, P)),
                           np.nan_to_num(p.tmp_out.reshape(R, P, 128)),
                           np.repeat(p.num_parts, Hq)).reshape(B, Hq, 128)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(cuda)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.bfloat16, device=cuda)
    pa.paged_attention_reduce(out, t(p.max_logits), t(p.exp_sums), t(p.tmp_out),
                              t(p.context_lens), part)
    torch.cuda.synchronize()
    check_close(to_f64(tensor_to_np(out, "bf16"), "bf16"), ref, "bf16", "reduce 1100 partitions")
