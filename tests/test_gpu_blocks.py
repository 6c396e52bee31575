"""Block copy (copy-on-write) and swap through the C ABI against the host
reference, bit-exact over the whole pool; and a multi-step decode with forked
requests whose copy-on-write copies run on the device, checked against the
oracle at every step."""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import copy_blocks as ref_copy_blocks
from paged_kv_cache_269_amd import workloads as W

from parity import check_close, tensor_to_np, to_f64

pytestmark = pytest.mark.gpu

BS = 16


def announce(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rand_pool(rng, shape, dtype):
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    return W._round_to_dtype(x, dtype).reshape(shape)


def to_dev(a, dtype, cuda):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.to(cuda)


def bits(t, dtype):
    return tensor_to_np(t, dtype).view(np.uint32 if dtype == "f32" else np.uint16)


@pytest.mark.parametrize("dtype,Hkv,D", [("bf16", 8, 128), ("f16", 2, 64), ("f32", 4, 128)])
def test_copy_blocks_bit_exact(cuda, dtype, Hkv, D):
    import paged_kv_cache_269_amd as pa
    announce("copy", dtype, Hkv, D)
    N = 300
    rng = np.random.default_rng(3)
    kh = rand_pool(rng, (N, Hkv, BS, D), dtype)
    vh = rand_pool(rng, (N, Hkv, BS, D), dtype)
    kd, vd = to_dev(kh, dtype, cuda), to_dev(vh, dtype, cuda)
    perm = rng.permutation(N)
    src, dst = perm[:70], perm[70:140]
    pairs = np.stack([src, dst], 1).astype(np.int32)
    pairs[5, 0] = pairs[3, 0]                      # one source copied twice
    assert pa.validate_copy_host(pairs, N) == 0
    bad = np.array([[N + 3, int(perm[200])], [int(perm[201]), -1]], np.int32)   # skipped
    pa.copy_blocks(kd, vd, torch.from_numpy(np.concatenate([pairs, bad])).to(cuda))
    torch.cuda.synchronize()
    ref_copy_blocks(kh, vh, pairs)
    view = np.uint32 if dtype == "f32" else np.uint16
    assert np.array_equal(bits(kd, dtype), kh.view(view))
    assert np.array_equal(bits(vd, dtype), vh.view(view))
    pa.copy_blocks(kd, vd, torch.zeros((0, 2), dtype=torch.int32, device=cuda))   # no-op


def test_swap_out_and_in(cuda):
    import paged_kv_cache_269_amd as pa
    dtype, Hkv, D, N, NH = "bf16", 8, 128, 200, 64
    rng = np.random.default_rng(4)
    kh = rand_pool(rng, (N, Hkv, BS, D), dtype)
    kd = to_dev(kh, dtype, cuda)
    host = torch.zeros((NH, Hkv, BS, D), dtype=torch.bfloat16).pin_memory()
    out_pairs = np.array([[10, 0], [11, 1], [12, 2], [40, 7], [3, 8], [4, 9]], np.int64)
    pa.swap_blocks(kd, host, out_pairs)                 # device -> host, runs of consecutive pairs
    torch.cuda.synchronize()
    hb = host.view(torch.uint16).numpy()
    for s, d in out_pairs:
        assert np.array_equal(hb[d], kh[s])
    in_pairs = np.array([[0, 150], [1, 151], [7, 20], [9, 199]], np.int64)
    pa.swap_blocks(host, kd, in_pairs)                  # host -> device
    torch.cuda.synchronize()
    got = bits(kd, dtype)
    for s, d in in_pairs:
        assert np.array_equal(got[d], hb[s])
    untouched = np.setdiff1d(np.arange(N), in_pairs[:, 1])
    assert np.array_equal(got[untouched], kh[untouched])


def test_swap_mapped_out_and_in(cuda):
    """The one-kernel swap through pinned host memory's device mapping:
    scattered device blocks out to a pinned host cache (pairs in pinned host
    memory) and back in (pairs on the device), bit-exact; pairs naming a
    block outside either cache are skipped; pageable host memory is refused
    before anything runs."""
    import paged_kv_cache_269_amd as pa
    from paged_kv_cache_269_amd import PagedAttnError
    dtype, Hkv, D, N, NH = "bf16", 8, 128, 300, 96
    rng = np.random.default_rng(6)
    kh = rand_pool(rng, (N, Hkv, BS, D), dtype)
    kd = to_dev(kh, dtype, cuda)
    host = torch.zeros((NH, Hkv, BS, D), dtype=torch.bfloat16).pin_memory()
    src = rng.permutation(N)[:40]
    dst = rng.permutation(NH)[:40]
    out_pairs = np.stack([src, dst], 1).astype(np.int64)
    bad = np.array([[N, 0], [0, NH], [-1, 5]], np.int64)          # skipped
    pairs_h = torch.from_numpy(np.concatenate([out_pairs, bad])).pin_memory()
    pa.swap_blocks_mapped(kd, host, pairs_h)                       # device -> pinned host
    torch.cuda.synchronize()
    hb = host.view(torch.uint16).numpy()
    for s_, d_ in out_pairs:
        assert np.array_equal(hb[d_], kh[s_])
    untouched_h = np.setdiff1d(np.arange(NH), dst)
    assert not hb[untouched_h].any()
    in_pairs = np.stack([dst[:20], rng.permutation(N)[:20]], 1).astype(np.int64)
    pa.swap_blocks_mapped(host, kd, torch.from_numpy(in_pairs).to(cuda))   # pinned host -> device
    torch.cuda.synchronize()
    got = bits(kd, dtype)
    for s_, d_ in in_pairs:
        assert np.array_equal(got[d_], hb[s_])
    untouched = np.setdiff1d(np.arange(N), in_pairs[:, 1])
    assert np.array_equal(got[untouched], kh[untouched])
    pageable = torch.zeros((NH, Hkv, BS, D), dtype=torch.bfloat16)
    with pytest.raises(PagedAttnError):
        pa.swap_blocks_mapped(kd, pageable, pairs_h)
    with pytest.raises(PagedAttnError):
        pa.swap_blocks_mapped(kd, host, torch.from_numpy(out_pairs))  # pageable pairs


def test_multistep_with_forks_and_copy_on_write(cuda):
    import paged_kv_cache_269_amd as pa
    dtype, Hq, Hkv, D, N, M = "bf16", 16, 2, 128, 64, 12
    rng = np.random.default_rng(9)
    bm = pa.BlockManager(N, BS)
    kh = np.zeros((N, Hkv, BS, D), np.uint16)
    vh = np.zeros_like(kh)
    W._nan_fill(kh, dtype, slice(None))
    W._nan_fill(vh, dtype, slice(None))
    kd, vd = to_dev(kh, dtype, cuda), to_dev(vh, dtype, cuda)

    def write(slots):
        k = rand_pool(rng, (len(slots), Hkv, D), dtype)
        v = rand_pool(rng, (len(slots), Hkv, D), dtype)
        sl = np.asarray(slots, np.int64)
        pa.reshape_and_cache(to_dev(k, dtype, cuda), to_dev(v, dtype, cuda), kd, vd,
                             torch.from_numpy(sl).to(cuda))
        oracle.reshape_and_cache(k, v, kh, vh, sl, dtype)

    bm.allocate(0, 0)
    write([bm.append(0)[0] for _ in range(40)])   # prompt: 2.5 blocks
    bm.fork(0, 1)                                  # parallel samples of one prompt
    bm.fork(0, 2)
    live = [0, 1, 2]
    ncopies = 0
    scale = 1.0 / np.sqrt(D)
    for step in range(25):
        if step == 9:
            bm.fork(1, 3)                           # a sample forks again, mid-block
            live.append(3)
        slots, copies = bm.append_batch(live)
        if len(copies):
            ncopies += len(copies)
            assert pa.validate_copy_host(copies, N) == 0
            pa.copy_blocks(kd, vd, torch.from_numpy(np.ascontiguousarray(copies)).to(cuda))
            ref_copy_blocks(kh, vh, copies)
        write(slots.tolist())
        bt, cl = bm.block_tables(live, M, pad=0)
        q = rand_pool(rng, (len(live), Hq, D), dtype)
        out = torch.empty((len(live), Hq, D), dtype=torch.bfloat16, device=cuda)
        pa.paged_attention_decode(out, to_dev(q, dtype, cuda), kd, vd, torch.from_numpy(bt).to(cuda),
                                  torch.from_numpy(cl).to(cuda), scale, int(cl.max()),
                                  partition_size=0)
        torch.cuda.synchronize()
        B = len(live)
        ref, _, _ = oracle.decode_rows(q, kh, vh, bt, cl, scale, dtype,
                                       np.repeat(np.arange(B), Hq), np.tile(np.arange(Hq), B))
        check_close(to_f64(tensor_to_np(out, dtype), dtype), ref.reshape(B, Hq, D), dtype,
                    f"fork step {step}")
    assert ncopies >= 3                              # every fork of a partial block copied once
    announce("copies", ncopies)
    bm.close()
