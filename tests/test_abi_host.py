"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
HEADERS = [os.path.join(INCLUDE, f) for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h")]

OK, NULL, SHAPE, UNSUP, WS, RANGE = 0, 1, 2, 3, 4, 5
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_symbols():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol(hiplib):
    lib = hiplib.load_library()
    names = declared_symbols()
    assert names, "no declarations found"
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(hiplib.EXPORTS) == names


def test_version_and_status_strings(hiplib):
    assert "gfx950" in hiplib.version()
    for code in range(0, 9):
        assert hiplib.status_string(code) and hiplib.status_string(code) != "unknown status"
    assert hiplib.status_string(99) == "unknown status"


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, B=2, Hq=8, Hkv=2, D=128, bs=16,
             M=4, N=10, scale=0.1, dtype=1, part=512, maxlen=64, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.pa_paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"],
                                         a["B"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["M"],
                                         a["N"], a["scale"], a["dtype"], a["part"], a["maxlen"],
                                         a["ws"], a["wsb"], a["stream"])


def test_decode_argument_checks(hiplib):
    lib = hiplib.load_library()
    assert _decode(lib, out=None) == NULL
    assert _decode(lib, bt=None) == NULL
    assert _decode(lib, D=96) == UNSUP
    assert _decode(lib, bs=24) == UNSUP     # 8, 16 and 32 are the block sizes taken
    assert _decode(lib, bs=64) == UNSUP
    assert _decode(lib, dtype=7) == UNSUP
    assert _decode(lib, part=100) == UNSUP
    assert _decode(lib, part=-16) == UNSUP
    assert _decode(lib, Hq=6, Hkv=4) == SHAPE
    assert _decode(lib, Hkv=0) == SHAPE
    assert _decode(lib, B=-1) == SHAPE
    assert _decode(lib, B=70000) == SHAPE
    assert _decode(lib, maxlen=-1) == SHAPE
    assert _decode(lib, N=0) == SHAPE
    # 1024 tokens in 512-token partitions need partials space
    assert _decode(lib, maxlen=1024, M=64) == WS
    need = lib.pa_decode_workspace_bytes(2, 8, 128, 1024, 512)
    assert _decode(lib, maxlen=1024, M=64, ws=FAKE, wsb=need - 1) == WS
    # zero sequences: nothing to do, no pointer is looked at
    assert _decode(lib, B=0, out=None) == OK


def _fused(lib, **kw):
    a = dict(out=FAKE, q=FAKE, key=FAKE, value=FAKE, k=FAKE, v=FAKE, slots=FAKE, bt=FAKE,
             cl=FAKE, B=2, Hq=8, Hkv=2, D=128, bs=16, M=4, N=10, scale=0.1, dtype=1, part=512,
             maxlen=64, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.pa_reshape_and_decode(a["out"], a["q"], a["key"], a["value"], a["k"], a["v"],
                                     a["slots"], a["bt"], a["cl"], a["B"], a["Hq"], a["Hkv"],
                                     a["D"], a["bs"], a["M"], a["N"], a["scale"], a["dtype"],
                                     a["part"], a["maxlen"], a["ws"], a["wsb"], a["stream"])


def test_fused_write_decode_argument_checks(hiplib):
    """pa_reshape_and_decode: the decode checks, plus the new tokens' rows
    and slots; all refused before any launch."""
    lib = hiplib.load_library()
    assert _fused(lib, key=None) == NULL
    assert _fused(lib, value=None) == NULL
    assert _fused(lib, slots=None) == NULL
    assert _fused(lib, out=None) == NULL
    assert _fused(lib, D=96) == UNSUP
    assert _fused(lib, bs=24) == UNSUP
    assert _fused(lib, part=100) == UNSUP
    assert _fused(lib, Hq=6, Hkv=4) == SHAPE
    assert _fused(lib, N=0) == SHAPE
    assert _fused(lib, maxlen=1024, M=64) == WS
    assert _fused(lib, B=0, key=None, slots=None) == OK


def _fused_cascade(lib, **kw):
    a = dict(out=FAKE, q=FAKE, key=FAKE, value=FAKE, k=FAKE, v=FAKE, slots=FAKE, bt=FAKE,
             cl=FAKE, B=2, Hq=8, Hkv=2, D=128, bs=16, M=4, N=10, scale=0.1, dtype=1,
             maxlen=64, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.pa_reshape_and_decode_cascade(a["out"], a["q"], a["key"], a["value"], a["k"],
                                             a["v"], a["slots"], a["bt"], a["cl"], a["B"],
                                             a["Hq"], a["Hkv"], a["D"], a["bs"], a["M"], a["N"],
                                             a["scale"], a["dtype"], a["maxlen"], a["ws"],
                                             a["wsb"], a["stream"])


def test_fused_cascade_argument_checks(hiplib):
    """pa_reshape_and_decode_cascade: the cascade checks, plus the new
    tokens' rows and slots; all refused before any launch."""
    lib = hiplib.load_library()
    f = lib.pa_cascade_workspace_bytes
    assert _fused_cascade(lib, key=None) == NULL
    assert _fused_cascade(lib, value=None) == NULL
    assert _fused_cascade(lib, slots=None) == NULL
    assert _fused_cascade(lib, out=None) == NULL
    assert _fused_cascade(lib, D=96) == UNSUP
    assert _fused_cascade(lib, bs=24) == UNSUP
    assert _fused_cascade(lib, Hq=6, Hkv=4) == SHAPE
    assert _fused_cascade(lib, ws=None, wsb=0) == WS
    assert _fused_cascade(lib, wsb=f(2, 8, 128) - 1) == WS
    assert _fused_cascade(lib, B=0, key=None, slots=None, ws=None, wsb=0) == OK


def test_workspace_bytes(hiplib):
    lib = hiplib.load_library()
    f = lib.pa_decode_workspace_bytes
    assert f(4, 8, 128, 512, 512) == 0          # one partition: no partials
    assert f(4, 8, 128, 4096, 0) == 0           # single pass
    rows = 4 * 8 * 2
    exp = -(-rows * 128 * 4 // 256) * 256 + 2 * (-(-rows * 4 // 256) * 256)
    assert f(4, 8, 128, 513, 512) == exp
    assert f(-1, 8, 128, 513, 512) == 0



def _cascade(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, B=2, Hq=8, Hkv=2, D=128, bs=16,
             M=4, N=10, scale=0.1, dtype=1, maxlen=64, ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.pa_paged_attention_decode_cascade(a["out"], a["q"], a["k"], a["v"], a["bt"],
                                                 a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                                 a["bs"], a["M"], a["N"], a["scale"], a["dtype"],
                                                 a["maxlen"], a["ws"], a["wsb"], a["stream"])


def test_multi_query_partition_size(hiplib):
    """The suggested multi-query partition follows its stated rule (no device
    here: the library assumes 256 compute units, target 1024 items)."""
    f = hiplib.multi_query_partition_size
    target = 4 * 256

    def items(B, Hq, Hkv, n, L, part):
        rows = n * (Hq // Hkv)
        one = B * Hkv * -(-rows // 128)
        return one * (-(-L // part) if part else 1), one, rows

    cases = [(8, 64, 8, 16, 131072), (8, 64, 8, 4, 131072), (2, 32, 32, 8, 40000),
             (1, 64, 8, 64, 1 << 20), (4, 8, 8, 2, 20000), (16, 64, 8, 16, 65536)]
    for B, Hq, Hkv, n, L in cases:
        part = f(B, Hq, Hkv, n, L)
        tot, one, rows = items(B, Hq, Hkv, n, L, part)
        assert part > 0 and part < L, (B, Hq, Hkv, n, L, part)
        assert part & (part - 1) == 0 and part % 16 == 0
        assert part >= max(512, 16 * min(rows, 128))
        # the longest such partition that still makes `target` items, or the
        # shortest allowed one when none does
        assert tot >= target or part == max(512, 1 << (16 * min(rows, 128) - 1).bit_length())
        assert items(B, Hq, Hkv, n, L, 2 * part)[0] < target
    # enough items in one pass, or one partition covering the context: one pass
    assert f(128, 64, 8, 16, 8192) == 0
    assert f(64, 32, 32, 8, 2048) == 0
    assert f(2, 64, 8, 16, 1000) == 0
    # invalid arguments
    assert f(0, 64, 8, 16, 4096) == 0 and f(8, 64, 7, 16, 4096) == 0
    assert f(8, 64, 8, 0, 4096) == 0 and f(8, 64, 8, 16, 0) == 0


def test_cascade_argument_checks_and_workspace(hiplib):
    lib = hiplib.load_library()
    f = lib.pa_cascade_workspace_bytes
    rows = 5 * 8
    al = lambda x: -(-x // 256) * 256
    assert f(5, 8, 128) == al(5 * 4) + 2 * al(rows * 4) + al(rows * 128 * 4)
    assert f(-1, 8, 128) == 0 and f(5, 0, 128) == 0
    assert _cascade(lib, out=None) == NULL
    assert _cascade(lib, D=96) == UNSUP
    assert _cascade(lib, dtype=9) == UNSUP
    assert _cascade(lib, Hq=6, Hkv=4) == SHAPE
    assert _cascade(lib, ws=None, wsb=0) == WS
    need = f(2, 8, 128)
    assert _cascade(lib, wsb=need - 1) == WS
    assert _cascade(lib, B=0, out=None, ws=None, wsb=0) == OK


def _mq(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, cl=FAKE, qs=FAKE, B=2, T=8, Hq=8, Hkv=2,
             D=128, bs=16, M=4, N=10, scale=0.1, dtype=1, mq=4, part=512, maxlen=64, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return lib.pa_paged_attention_multi_query(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["qs"], a["B"], a["T"], a["Hq"],
        a["Hkv"], a["D"], a["bs"], a["M"], a["N"], a["scale"], a["dtype"], a["mq"], a["part"],
        a["maxlen"], a["ws"], a["wsb"], a["stream"])


def test_multi_query_argument_checks_and_workspace(hiplib):
    lib = hiplib.load_library()
    assert _mq(lib, qs=None) == NULL
    assert _mq(lib, out=None) == NULL
    assert _mq(lib, dtype=0) == UNSUP          # float32 is not taken here
    assert _mq(lib, D=96) == UNSUP
    assert _mq(lib, bs=24) == UNSUP
    assert _mq(lib, part=100) == UNSUP
    assert _mq(lib, Hq=6, Hkv=4) == SHAPE
    assert _mq(lib, T=70000) == SHAPE
    assert _mq(lib, B=-1) == SHAPE
    assert _mq(lib, mq=-1) == SHAPE
    assert _mq(lib, maxlen=1024, M=64) == WS   # partials for 2 partitions
    f = lib.pa_multi_query_workspace_bytes
    need = f(8, 8, 128, 1024, 512)
    al = lambda x: -(-x // 256) * 256
    rows = 8 * 8 * 2
    assert need == al(rows * 128 * 4) + 2 * al(rows * 4) + al(8 * 4)
    assert _mq(lib, maxlen=1024, M=64, ws=FAKE, wsb=need - 1) == WS
    assert f(8, 8, 128, 512, 512) == 0 and f(8, 8, 128, 4096, 0) == 0 and f(-1, 8, 128, 9, 16) == 0
    # nothing to do: no pointer is looked at
    assert _mq(lib, T=0, out=None) == OK and _mq(lib, B=0, qs=None) == OK


def test_swap_mapped_argument_checks(hiplib):
    """Only checks that fail before any runtime call (no GPU here)."""
    f = hiplib.load_library().pa_swap_blocks_mapped
    assert f(FAKE, FAKE, FAKE, -1, 4096, 8, 8, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 70000, 4096, 8, 8, None) == SHAPE
    assert f(FAKE, FAKE, FAKE, 2, 4100, 8, 8, None) == SHAPE      # not a multiple of 16
    assert f(FAKE, FAKE, FAKE, 2, 4096, 0, 8, None) == SHAPE
    assert f(None, FAKE, FAKE, 2, 4096, 8, 8, None) == NULL
    assert f(FAKE, FAKE, None, 2, 4096, 8, 8, None) == NULL
    assert f(FAKE, ctypes.c_void_p(0x1008), FAKE, 2, 4096, 8, 8, None) == UNSUP   # misaligned
    assert f(None, None, None, 0, 4096, 8, 8, None) == OK


def test_query_start_validator(hiplib):
    v = hiplib.validate_query_start_host
    assert v([0, 3, 3, 7], [5, 1, 9], 7, 4) == 0
    assert v([0, 3, 3, 7], None, 7, 4) == 0
    assert v([1, 3, 3, 7], None, 7, 4) == RANGE       # must start at 0
    assert v([0, 3, 3, 6], None, 7, 4) == RANGE       # must end at T
    assert v([0, 3, 2, 7], None, 7, 5) == RANGE       # decreasing
    assert v([0, 3, 3, 7], None, 7, 3) == RANGE       # a span longer than max_query_len
    assert v([0, 3, 3, 7], [2, 1, 9], 7, 4) == RANGE  # more new tokens than context
    assert v([0], None, 0, 1) == 0


def test_reshape_and_reduce_argument_checks(hiplib):
    lib = hiplib.load_library()
    r = lib.pa_reshape_and_cache
    assert r(None, FAKE, FAKE, FAKE, FAKE, 3, 2, 128, 16, 10, 2, None) == NULL
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 2, 80, 16, 10, 2, None) == UNSUP
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 2, 128, 12, 10, 2, None) == UNSUP
    assert r(FAKE, FAKE, FAKE, FAKE, FAKE, -3, 2, 128, 16, 10, 2, None) == SHAPE
    assert r(None, None, None, None, None, 0, 2, 128, 16, 10, 2, None) == OK
    d = lib.pa_paged_attention_reduce
    assert d(None, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 512, 3, 2, None) == NULL
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 128, 0, 3, 2, None) == UNSUP
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 4, 100, 512, 3, 2, None) == UNSUP
    assert d(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 128, 512, 3, 2, None) == SHAPE


@pytest.mark.parametrize("case", range(6))
def test_table_validator_agrees_with_oracle(hiplib, case):
    rng = np.random.default_rng(case)
    B, M, N = 5, 6, 20
    bt = rng.integers(0, N, size=(B, M)).astype(np.int32)
    cl = rng.integers(0, M * 16 + 1, size=B).astype(np.int32)
    if case == 1:
        bt[2, 0] = N            # used entry out of the pool
        cl[2] = max(cl[2], 1)
    if case == 2:
        cl[0] = M * 16 + 1      # does not fit the row
    if case == 3:
        cl[4] = -5
    if case == 4:
        bt[1, M - 1] = -7       # only bad if used
        cl[1] = (M - 1) * 16
    if case == 5:
        bt[3, :] = -1           # unused row of an empty sequence
        cl[3] = 0
    got = hiplib.validate_tables_host(bt, cl, N)
    try:
        oracle.check_tables(bt, cl, N)
        want = OK
    except oracle.OracleError:
        want = RANGE
    assert got == want
    assert got == (RANGE if case in (1, 2, 3) else OK)


def test_slot_validator(hiplib):
    assert hiplib.validate_slots_host(np.array([0, 17, -1, -1, 159]), 10) == OK
    assert hiplib.validate_slots_host(np.array([0, 17, 17]), 10) == RANGE
    assert hiplib.validate_slots_host(np.array([160]), 10) == RANGE
    assert hiplib.validate_slots_host(np.zeros(0, np.int64), 10) == OK


def test_step_validator(hiplib):
    """pa_validate_step_host: the one-call step's condition -- no context
    reads a slot written in the step, except the writer's own last position."""
    from paged_kv_cache_269_amd import workloads as W
    for name, over in (("tiny", {}), ("llama7b", dict(num_seqs=5, len_lo=1, len_hi=300)),
                       ("shared_prefix", dict(num_seqs=6, len_lo=20, len_hi=60,
                                              shared_prefix_blocks=4))):
        w = W.generate(name, **over)
        assert hiplib.validate_step_host(w.slot_mapping, w.block_tables, w.context_lens,
                                         w.num_blocks, w.block_size) == OK, name
    # hand-built: 3 sequences, 16-token blocks; 0 and 1 share block 7
    bt = np.array([[7, 2, 0], [7, 3, 0], [5, 0, 0]], np.int32)
    cl = np.array([20, 18, 16], np.int32)
    ok = np.array([2 * 16 + 3, 3 * 16 + 1, 5 * 16 + 15], np.int64)  # each one's last position
    assert hiplib.validate_step_host(ok, bt, cl, 10) == OK
    assert hiplib.validate_step_host(np.array([-1, -1, -1]), bt, cl, 10) == OK
    free = ok.copy(); free[2] = 9 * 16 + 4            # a block no context reads
    assert hiplib.validate_step_host(free, bt, cl, 10) == OK
    shared = ok.copy(); shared[0] = 7 * 16 + 5        # block 7 is read by sequence 1 as well
    assert hiplib.validate_step_host(shared, bt, cl, 10) == RANGE
    own = ok.copy(); own[1] = 3 * 16 + 0              # sequence 1 reads position 16 as context
    assert hiplib.validate_step_host(own, bt, cl, 10) == RANGE
    other = ok.copy(); other[2] = 2 * 16 + 1          # inside sequence 0's context
    assert hiplib.validate_step_host(other, bt, cl, 10) == RANGE
    dup = ok.copy(); dup[2] = dup[0]                  # two tokens, one slot
    assert hiplib.validate_step_host(dup, bt, cl, 10) == RANGE
    assert hiplib.validate_step_host(ok, bt, cl, 6) == RANGE  # block 7 outside the pool
    tail = ok.copy(); tail[1] = 3 * 16 + 5            # past sequence 1's end: nobody reads it
    assert hiplib.validate_step_host(tail, bt, cl, 10) == OK


def test_binding_refuses_host_tensors(hiplib):
    import torch
    x = torch.zeros(2, 4, 128, dtype=torch.float16)
    kc = torch.zeros(3, 4, 16, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        hiplib.reshape_and_cache(x, x, kc, kc, torch.zeros(2, dtype=torch.int64))
    # the one-call steps check shapes, then refuse host tensors, before any launch
    q = torch.zeros(2, 4, 128, dtype=torch.float16)
    bt = torch.zeros(2, 3, dtype=torch.int32)
    cl = torch.ones(2, dtype=torch.int32)
    sl = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        hiplib.reshape_and_decode(torch.empty_like(q), q, x, x, kc, kc, sl, bt, cl, 0.1, 16,
                                  partition_size=0)
    with pytest.raises(ValueError):
        hiplib.reshape_and_decode_cascade(torch.empty_like(q), q, x, x, kc, kc, sl, bt, cl, 0.1,
                                          16, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    with pytest.raises(ValueError):  # key rows must be [num_seqs, num_kv_heads, head_dim]
        hiplib.reshape_and_decode(torch.empty_like(q), q, x[:1], x[:1], kc, kc, sl, bt, cl, 0.1, 16,
                                  partition_size=0)


def _step_ok_brute(slots, bt, cl, num_blocks, bs):
    """Plain definition of pa_validate_step_host's condition, slot by slot."""
    B, M = bt.shape
    for s in range(B):
        L = int(cl[s])
        if L < 0 or (L + bs - 1) // bs > M:
            return False
        for j in range((L + bs - 1) // bs):
            if not 0 <= bt[s, j] < num_blocks:
                return False
    live = [int(x) for x in slots if x >= 0]
    if any(x >= num_blocks * bs for x in live) or len(set(live)) != len(live):
        return False
    for s in range(B):
        slot = int(slots[s])
        if slot < 0:
            continue
        for r in range(B):                       # every position every context reads
            for t in range(int(cl[r])):
                pos_slot = int(bt[r, t // bs]) * bs + t % bs
                if pos_slot == slot and not (r == s and t == int(cl[s]) - 1):
                    return False
    return True


def test_step_validator_matches_brute_force(hiplib):
    rng = np.random.default_rng(31)
    agree = {True: 0, False: 0}
    for _ in range(300):
        bs = int(rng.choice([8, 16, 32]))
        B, M, N = int(rng.integers(1, 5)), int(rng.integers(1, 4)), int(rng.integers(2, 9))
        bt = rng.integers(0, N, size=(B, M)).astype(np.int32)   # blocks may be shared
        cl = rng.integers(0, M * bs + 1, size=B).astype(np.int32)
        slots = np.full(B, -1, np.int64)
        for s in range(B):
            r = rng.random()
            if r < 0.5 and cl[s] > 0:            # its own last position
                t = int(cl[s]) - 1
                slots[s] = int(bt[s, t // bs]) * bs + t % bs
            elif r < 0.85:                       # anywhere in the pool
                slots[s] = int(rng.integers(0, N * bs))
        want = _step_ok_brute(slots, bt, cl, N, bs)
        got = hiplib.validate_step_host(slots, bt, cl, N, bs)
        assert (got == OK) == want, (bt, cl, slots, bs, got)
        agree[want] += 1
    assert agree[True] > 20 and agree[False] > 20   # both outcomes exercised


def test_library_binds_to_torchs_hip_runtime():
    """Loaded before torch is imported, the library still ends up on torch's
    copy of the HIP runtime (the one whose memory and streams it is given):
    one libamdhip64 in the process, not the system's beside torch's.  Checked
    in a fresh interpreter, which imports the package and loads the library
    first."""
    import ast
    import subprocess
    import sys
    code = ("import paged_kv_cache_269_amd as pa; pa.load_library(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') "
            "if 'libamdhip64' in l}))")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    runtimes = ast.literal_eval(r.stdout.strip().splitlines()[-1])
    assert len(runtimes) == 1, f"two HIP runtimes loaded: {runtimes}"
