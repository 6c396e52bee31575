"""Float64 CPU oracle for paged decode attention: Python side.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  It never imports the
HIP library or its binding, and the HIP path never imports it.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc and OpenMP); this
module only builds and loads that library and marshals numpy arrays into it.
Definitions followed (page titles and sections, see ``oracle.c``):
  * decode attention o_t = Attention(q_t, K_{1:t}, V_{1:t})
    -- "vLLM 2026 推理引擎全解" (chenxutan.com), §1.1;
  * 16-token pages, page table, shared pages -- same page, §2.1;
  * cache layout [num_pages, num_heads, page_size, head_dim] and the token
    address page_id * BLOCK_SIZE + page_offset -- same page, §2.2;
  * gather through the block table -- vLLM tutorial (mjmagnets.cn), §2.2;
  * several new query tokens per sequence, each attending causally to the
    context up to its own position -- the §1.1 definition for each of them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# The in-tree build; ORACLE_LIB may name another build of oracle.c (the
# sanitizer run of the CPU tests).
_LIB = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}

OK, ERR_ARG, ERR_RANGE, ERR_DUP, ERR_NOMEM = 0, 1, 2, 3, 4


class OracleError(RuntimeError):
    def __init__(self, fn: str, code: int):
        names = {ERR_ARG: "bad argument", ERR_RANGE: "value out of range",
                 ERR_DUP: "duplicate slot", ERR_NOMEM: "out of memory"}
        super().__init__(f"{fn}: {names.get(code, 'error')} (code {code})")
        self.code = code


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no HIP involved)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib: Optional[ctypes.CDLL] = None


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_reshape_and_cache.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i64, i32]
    lib.oracle_check_tables.argtypes = [P, P, i32, i32, i64, i32]
    lib.oracle_decode_rows.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                       i32, i64, f64, i32, P, P, P, P, i64, i32]
    lib.oracle_lse_merge.argtypes = [P, P, P, P, P, i64, i32, i32]
    lib.oracle_max_threads.argtypes = []
    for fn in (lib.oracle_reshape_and_cache, lib.oracle_check_tables,
               lib.oracle_decode_rows, lib.oracle_lse_merge, lib.oracle_max_threads):
        fn.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(fn: str, rc: int):
    if rc != OK:
        raise OracleError(fn, rc)


def _c(a, dtype=None) -> np.ndarray:
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, dtype: str) -> None:
    """Write each token's K/V row into its slot, in place on k_cache/v_cache.

    key/value [T, Hkv, D]; caches [N, Hkv, block_size, D] (numpy, same element
    type; bf16 held as uint16 bit patterns); slot_mapping [T] int64.
    """
    key, value, slots = _c(key), _c(value), _c(slot_mapping, np.int64)
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be C-contiguous (they are written in place)")
    N, Hkv, bs, D = k_cache.shape
    T = key.shape[0]
    rc = _load().oracle_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(slots), T, Hkv, D, bs, N, DTYPE_CODES[dtype])
    _check("oracle_reshape_and_cache", rc)


def check_tables(block_tables, context_lens, num_blocks: int, block_size: int = 16) -> None:
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    rc = _load().oracle_check_tables(_ptr(bt), _ptr(cl), cl.shape[0], bt.shape[1],
                                     int(num_blocks), block_size)
    _check("oracle_check_tables", rc)


def decode_rows(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
                rows_seq: Sequence[int], rows_head: Sequence[int],
                rows_t_begin: Optional[Sequence[int]] = None,
                rows_t_end: Optional[Sequence[int]] = None,
                num_threads: int = 0):
    """Decode attention for the listed (seq, head[, token range]) rows.

    Returns (out [R, D] float64, m [R], l [R]) where m is the max scaled score
    over the range and l = sum exp(z - m).  A token range end of -1 means the
    sequence's full context length.
    """
    q = _c(q)
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    k_cache, v_cache = _c(k_cache), _c(v_cache)
    B, Hq, D = q.shape
    N, Hkv, bs, D2 = k_cache.shape
    if D2 != D:
        raise ValueError("head_dim mismatch between q and the cache")
    rs = _c(rows_seq, np.int32)
    rh = _c(rows_head, np.int32)
    R = rs.shape[0]
    t0 = _c(np.zeros(R) if rows_t_begin is None else rows_t_begin, np.int32)
    t1 = _c(np.full(R, -1) if rows_t_end is None else rows_t_end, np.int32)
    out = np.zeros((R, D), np.float64)
    m = np.zeros(R, np.float64)
    l = np.zeros(R, np.float64)
    rc = _load().oracle_decode_rows(_ptr(out), _ptr(m), _ptr(l), _ptr(q), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(bt), _ptr(cl), B, Hq, Hkv, D, bs,
                                    bt.shape[1], N, float(scale), DTYPE_CODES[dtype],
                                    _ptr(rs), _ptr(rh), _ptr(t0), _ptr(t1), R, int(num_threads))
    _check("oracle_decode_rows", rc)
    return out, m, l


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str,
           num_threads: int = 0) -> np.ndarray:
    """Full decode: out [B, Hq, D] float64 over each sequence's whole context."""
    B, Hq, D = np.asarray(q).shape
    rs = np.repeat(np.arange(B, dtype=np.int32), Hq)
    rh = np.tile(np.arange(Hq, dtype=np.int32), B)
    out, _, _ = decode_rows(q, k_cache, v_cache, block_tables, context_lens, scale, dtype,
                            rs, rh, num_threads=num_threads)
    return out.reshape(B, Hq, D)


def lse_merge(m, l, o, num_parts) -> np.ndarray:
    """Merge per-part (max, sum, normalised output) triples into one row each.

    m, l [R, P]; o [R, P, D]; num_parts [R].  Inputs are upcast to float64
    (exact for float32 partials).
    """
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    np_ = _c(num_parts, np.int32)
    R, P, D = o.shape
    out = np.zeros((R, D), np.float64)
    rc = _load().oracle_lse_merge(_ptr(out), _ptr(m), _ptr(l), _ptr(o), _ptr(np_), R, P, D)
    _check("oracle_lse_merge", rc)
    return out


def multi_query(q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                dtype: str, rows_token: Optional[Sequence[int]] = None,
                rows_head: Optional[Sequence[int]] = None, num_threads: int = 0) -> np.ndarray:
    """Several new query tokens per sequence: out [T, Hq, D] float64.

    Sequence s owns query tokens query_start[s] .. query_start[s+1] - 1, the
    last n_s of its L_s context tokens; token i of that span sits at position
    p = L_s - n_s + i and attends to tokens 0 .. p.  That is the decode
    definition o_t = Attention(q_t, K_{1:t}, V_{1:t}) ("vLLM 2026 推理引擎全解"
    (chenxutan.com) §1.1) once for each of those t, so every row here is one
    decode row of oracle.c over the token range [0, p + 1); a token with
    p < 0 gets a zero row.  q [T, Hq, D].  With ``rows_token``/``rows_head``
    only those (token, head) rows are computed and [R, D] is returned.
    """
    q = _c(q)
    qs = _c(query_start, np.int64)
    bt, cl = _c(block_tables, np.int32), _c(context_lens, np.int32)
    T, Hq, D = q.shape
    B = qs.shape[0] - 1
    if qs[0] != 0 or qs[-1] != T or (np.diff(qs) < 0).any() or cl.shape[0] != B:
        raise ValueError("query_start must run from 0 to T without decreasing")
    n = np.diff(qs)
    seq_of = np.repeat(np.arange(B), n)                      # sequence of each query token
    pos = cl[seq_of].astype(np.int64) - n[seq_of] + (np.arange(T) - qs[seq_of])
    full = rows_token is None
    if full:
        rows_tok = np.repeat(np.arange(T, dtype=np.int32), Hq)
        rows_h = np.tile(np.arange(Hq, dtype=np.int32), T)
    else:
        rows_tok, rows_h = _c(rows_token, np.int32), _c(rows_head, np.int32)
    t_end = np.maximum(pos[rows_tok] + 1, 0).astype(np.int32)
    # one "sequence" per query token: its q row, its sequence's table and length
    out, _, _ = decode_rows(q, k_cache, v_cache, bt[seq_of], cl[seq_of], scale, dtype,
                            rows_tok, rows_h, np.zeros_like(t_end), t_end,
                            num_threads=num_threads)
    return out.reshape(T, Hq, D) if full else out
