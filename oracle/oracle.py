"""ctypes wrapper of the fp64 CPU oracle (pkv_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check of the
package entry file and by the CPU-baseline leg of the benchmark.  Nothing in the
product path may import it.

Parity status: every function here is pinned by tests that do not call the oracle
to produce their expectations (see the test files named test_oracle_*.py): the
pages' byte counts and worked address examples, brute-force attention over the
contiguous logical arrays, closed forms (n = 1, scale = 0, one dominant key, GQA
as repeated MHA heads), invariance under relabelling of physical blocks, the
merge identity, and prefix-sharing equivalence.  No function is parity-unpinned.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "libpkv_oracle.so")
# The mutation tests point this at a copy of the oracle built with a planted mistake.
_LIB_OVERRIDE = os.environ.get("PKV_ORACLE_LIB")

FP16, BF16 = 0, 1
DTYPES = {"fp16": FP16, "bf16": BF16}

_ERRORS = {
    -1: "bad argument",
    -10: "table entry outside the pool or past the table row",
    -11: "offset outside [0, block_size)",
    -12: "two writes target the same slot",
    -13: "out of memory",
}


class OracleError(RuntimeError):
    pass


def build(force: bool = False) -> str:
    """Compile pkv_oracle.c with gcc (no fast-math) into libpkv_oracle.so."""
    if _LIB_OVERRIDE:
        return _LIB_OVERRIDE
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(build())
        P = C.c_void_p
        i64 = C.c_int64
        L.oracle_fp16_to_double.argtypes = [C.c_uint16]
        L.oracle_fp16_to_double.restype = C.c_double
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_elem_offset.argtypes = [i64] * 7
        L.oracle_elem_offset.restype = i64
        L.oracle_locate.argtypes = [P, i64, i64, i64, i64, P, P]
        L.oracle_locate.restype = C.c_int
        L.oracle_append.argtypes = [P, P, P, P, P, P, P] + [i64] * 6
        L.oracle_append.restype = C.c_int
        L.oracle_append_tokens.argtypes = [P, P, P, P, P, P, P] + [i64] * 6
        L.oracle_append_tokens.restype = C.c_int
        L.oracle_locate_slotted.argtypes = [P, i64, i64, i64, i64, P, P]
        L.oracle_locate_slotted.restype = C.c_int
        L.oracle_append_slotted.argtypes = [P, P, P, P, P, P, P] + [i64] * 6
        L.oracle_append_slotted.restype = C.c_int
        L.oracle_attention_slotted.argtypes = [P, P, P, P, P, P] + [i64] * 7 + [C.c_double,
                                                                                C.c_int, C.c_int]
        L.oracle_attention_slotted.restype = C.c_int
        L.oracle_copy_blocks.argtypes = [P, P, P, P] + [i64] * 5
        L.oracle_copy_blocks.restype = C.c_int
        L.oracle_copy_slots.argtypes = [P, P, P] + [i64] * 5
        L.oracle_copy_slots.restype = C.c_int
        L.oracle_attention.argtypes = [P, P, P, P, P, P] + [i64] * 7 + [C.c_double, C.c_int,
                                                                          C.c_int]
        L.oracle_attention.restype = C.c_int
        L.oracle_partials.argtypes = [P, P, P, P, P, P, P] + [i64] * 7 + [
            C.c_double, C.c_int, i64, i64, C.c_int]
        L.oracle_partials.restype = C.c_int
        L.oracle_merge.argtypes = [P, P, P, P] + [i64] * 5
        L.oracle_merge.restype = C.c_int
        L.oracle_max_threads.argtypes = [C.c_int]
        L.oracle_max_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what}: {_ERRORS.get(rc, rc)}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------------------
def fp16_to_double(bits: int) -> float:
    return lib().oracle_fp16_to_double(bits)


def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def elem_offset(phys, h, off, d, num_kv_heads, block_size, head_dim) -> int:
    return lib().oracle_elem_offset(phys, h, off, d, num_kv_heads, block_size, head_dim)


def locate(table_row, block_size: int, num_blocks: int, t: int) -> Tuple[int, int]:
    row = _c(table_row, np.int32)
    phys, off = C.c_int64(), C.c_int64()
    rc = lib().oracle_locate(_p(row), row.shape[0], block_size, num_blocks, t,
                             C.byref(phys), C.byref(off))
    _check(rc, "locate")
    return phys.value, off.value


def max_threads(nthreads: int = 0) -> int:
    return lib().oracle_max_threads(nthreads)


def append(k_pool, v_pool, k_new, v_new, tables, lens, block_size, num_blocks):
    """In-place append of one token per sequence; returns slot ids (int64 [S])."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    S, Hkv, D = k_new.shape
    tables = _c(tables, np.int32)
    lens = _c(lens, np.int32)
    slots = np.empty(S, dtype=np.int64)
    rc = lib().oracle_append(_p(k_pool), _p(v_pool), _p(_c(k_new, np.uint16)),
                             _p(_c(v_new, np.uint16)), _p(tables), _p(lens), _p(slots),
                             S, Hkv, D, block_size, tables.shape[1], num_blocks)
    _check(rc, "append")
    return slots


def append_tokens(k_pool, v_pool, k_src, v_src, cu, start_pos, seg_tables, block_size,
                  num_blocks):
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    _, Hkv, D = k_src.shape
    seg_tables = _c(seg_tables, np.int32)
    rc = lib().oracle_append_tokens(_p(k_pool), _p(v_pool), _p(_c(k_src, np.uint16)),
                                    _p(_c(v_src, np.uint16)), _p(_c(cu, np.int64)),
                                    _p(_c(start_pos, np.int32)), _p(seg_tables),
                                    seg_tables.shape[0], Hkv, D, block_size,
                                    seg_tables.shape[1], num_blocks)
    _check(rc, "append_tokens")


def copy_blocks(k_pool, v_pool, src, dst):
    """Copy-on-write duplication: block dst[i] of both pools becomes a copy of
    block src[i] (pools [NB][Hkv][B][D] uint16, modified in place)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    NB, Hkv, B, D = k_pool.shape
    src, dst = _c(src, np.int32), _c(dst, np.int32)
    assert src.shape == dst.shape
    rc = lib().oracle_copy_blocks(_p(k_pool), _p(v_pool), _p(src), _p(dst), src.shape[0], Hkv,
                                  D, B, NB)
    _check(rc, "copy_blocks")


def copy_slots(k_pool, v_pool, copies):
    """Copy-on-write split of shared slots: for each row (src block, src offset,
    dst block, dst offset, length) of `copies` ([n][5] int32), the source rows go
    to the destination rows of both pools ([NB][Hkv][B][D] uint16, in place)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    NB, Hkv, B, D = k_pool.shape
    copies = _c(np.asarray(copies, np.int32).reshape(-1, 5), np.int32)
    rc = lib().oracle_copy_slots(_p(k_pool), _p(v_pool), _p(copies), copies.shape[0], Hkv, D,
                                 B, NB)
    _check(rc, "copy_slots")


def attention(q, k_pool, v_pool, tables, lens, num_kv_heads, block_size, num_blocks, scale,
              dtype: str, nthreads: int = 0) -> np.ndarray:
    S, Hq, D = q.shape
    tables = _c(tables, np.int32)
    out = np.empty((S, Hq, D), dtype=np.float64)
    rc = lib().oracle_attention(_p(out), _p(_c(q, np.uint16)), _p(k_pool), _p(v_pool),
                                _p(tables), _p(_c(lens, np.int32)), S, Hq, num_kv_heads, D,
                                block_size, tables.shape[1], num_blocks, float(scale),
                                DTYPES[dtype], nthreads)
    _check(rc, "attention")
    return out


def locate_slotted(segs, block_size: int, num_blocks: int, t: int):
    """(physical block, in-block offset) of logical token t of a sequence given as
    (block id, slot offset, length) segments."""
    segs = _c(segs, np.int32).reshape(-1, 3)
    phys, off = C.c_int64(), C.c_int64()
    rc = lib().oracle_locate_slotted(_p(segs), segs.shape[0], block_size, num_blocks, t,
                                     C.byref(phys), C.byref(off))
    _check(rc, "locate_slotted")
    return phys.value, off.value


def append_slotted(k_pool, v_pool, k_new, v_new, segs, num_segs, block_size, num_blocks):
    """In-place append of each sequence's new token at position n-1 of its segment
    list (n = sum of its segment lengths); returns slot ids (int64 [S], -1 for
    n = 0)."""
    assert k_pool.flags.c_contiguous and v_pool.flags.c_contiguous
    S, Hkv, D = k_new.shape
    segs = _c(segs, np.int32)
    slots = np.empty(S, dtype=np.int64)
    rc = lib().oracle_append_slotted(_p(k_pool), _p(v_pool), _p(_c(k_new, np.uint16)),
                                     _p(_c(v_new, np.uint16)), _p(segs),
                                     _p(_c(num_segs, np.int32)), _p(slots), S, segs.shape[1],
                                     Hkv, D, block_size, num_blocks)
    _check(rc, "append_slotted")
    return slots


def attention_slotted(q, k_pool, v_pool, segs, num_segs, num_kv_heads, block_size, num_blocks,
                      scale, dtype: str, nthreads: int = 0) -> np.ndarray:
    """Decode attention of sequences given as segment lists: segs [S][max_segs][3]
    (block id, slot offset, length), num_segs [S]."""
    S, Hq, D = q.shape
    segs = _c(segs, np.int32)
    out = np.empty((S, Hq, D), dtype=np.float64)
    rc = lib().oracle_attention_slotted(_p(out), _p(_c(q, np.uint16)), _p(k_pool), _p(v_pool),
                                        _p(segs), _p(_c(num_segs, np.int32)), S, Hq,
                                        num_kv_heads, D, block_size, segs.shape[1], num_blocks,
                                        float(scale), DTYPES[dtype], nthreads)
    _check(rc, "attention_slotted")
    return out


def partials(q, k_pool, v_pool, tables, lens, num_kv_heads, block_size, num_blocks, scale,
             dtype: str, partition_size: int, max_partitions: int, nthreads: int = 0):
    S, Hq, D = q.shape
    tables = _c(tables, np.int32)
    po = np.full((S, Hq, max_partitions, D), np.nan, dtype=np.float64)
    pl = np.full((S, Hq, max_partitions), np.nan, dtype=np.float64)
    rc = lib().oracle_partials(_p(po), _p(pl), _p(_c(q, np.uint16)), _p(k_pool), _p(v_pool),
                               _p(tables), _p(_c(lens, np.int32)), S, Hq, num_kv_heads, D,
                               block_size, tables.shape[1], num_blocks, float(scale),
                               DTYPES[dtype], partition_size, max_partitions, nthreads)
    _check(rc, "partials")
    return po, pl


def merge(part_o, part_lse, lens, partition_size: int) -> np.ndarray:
    S, Hq, MP, D = part_o.shape
    part_o = _c(part_o, np.float64)
    part_lse = _c(part_lse, np.float64)
    out = np.empty((S, Hq, D), dtype=np.float64)
    rc = lib().oracle_merge(_p(out), _p(part_o), _p(part_lse), _p(_c(lens, np.int32)), S, Hq,
                            D, partition_size, MP)
    _check(rc, "merge")
    return out


# ---------------------------------------------------------------------------
def new_pools(num_blocks, num_kv_heads, block_size, head_dim, fill_bits: int):
    shape = (num_blocks, num_kv_heads, block_size, head_dim)
    return (np.full(shape, fill_bits, dtype=np.uint16), np.full(shape, fill_bits, dtype=np.uint16))


def run_step(w, scale: Optional[float] = None, nthreads: int = 0, partition_size: int = 0,
             max_partitions: int = 0):
    """Whole decode step of one layer of a workload: pools filled with the NaN
    sentinel, history segments written, the new token appended, attention.

    Returns dict(k_pool, v_pool, slots, out[, part_o, part_lse, merged])."""
    c = w.cfg
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(c.head_dim)))
    kp, vp = new_pools(w.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, w.nan_bits)
    append_tokens(kp, vp, w.k_src, w.v_src, w.seg_cu, w.seg_start, w.seg_tables, c.block_size,
                  w.num_blocks)
    slots = append(kp, vp, w.k_new, w.v_new, w.tables, w.lengths, c.block_size, w.num_blocks)
    out = attention(w.q, kp, vp, w.tables, w.lengths, c.num_kv_heads, c.block_size,
                    w.num_blocks, scale, c.dtype, nthreads)
    res = dict(k_pool=kp, v_pool=vp, slots=slots, out=out)
    if partition_size:
        po, pl = partials(w.q, kp, vp, w.tables, w.lengths, c.num_kv_heads, c.block_size,
                          w.num_blocks, scale, c.dtype, partition_size, max_partitions, nthreads)
        res.update(part_o=po, part_lse=pl, merged=merge(po, pl, w.lengths, partition_size))
    return res
