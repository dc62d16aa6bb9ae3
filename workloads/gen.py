"""Seeded generator for paged-decode inputs.

Every random stream is drawn from ``numpy.random.default_rng(SeedSequence([cfg_id,
layer, stream, index]))`` so that each piece can be regenerated on its own and in
parallel without changing a single bit.  Lengths and block tables use layer 0 for
every layer: one block id covers a token's K/V in all layers (the page
"显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结" (blog.llmgo.top), §二.1,
"块大小" and "块表"), so all layers share the tables; only the K/V/Q values differ
per layer.

Values are drawn as float32 standard normals, multiplied by the config's scale (a
power of two, so exact) and rounded to fp16 or bf16 with round-to-nearest-even.
Positions that hold no token (the tail of each sequence's last block, blocks no
table points at) are left to the caller, who fills them with a NaN sentinel.

The history that exists before the step is described as *segments*: runs of
consecutive logical positions of one table row, with their K/V rows.  A segment is
an input description only; each side (oracle, HIP path) writes segments into its
own pool copy with its own code.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import List, Sequence, Tuple

import numpy as np

from .configs import Config

# stream ids of the seed namespace
S_LENGTHS, S_TABLES, S_Q, S_KHIST, S_VHIST, S_KNEW, S_VNEW = range(7)

# quiet-NaN bit patterns used to fill positions that hold no token
NAN_BITS = {"fp16": 0x7E00, "bf16": 0x7FC0}


def _rng(cfg_id: int, layer: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, layer, stream, index]))


# --------------------------------------------------------------------------
# rounding of float32 draws to 16-bit storage formats (IEEE 754 binary16 and
# bfloat16, both round-to-nearest-even)
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> binary16 bits, round to nearest even (numpy's cast is RNE)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r = r.copy()
        r[nan] = (u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040)
    return r


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp16/bf16 bit patterns to float64 (exact)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal_bits(rng: np.random.Generator, shape, scale: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return round_to_bits(x, dtype)


# --------------------------------------------------------------------------
# lengths and tables
# --------------------------------------------------------------------------
def draw_lengths(cfg: Config) -> np.ndarray:
    """Attended lengths n_s (the appended token included)."""
    rng = _rng(cfg.cfg_id, 0, S_LENGTHS)
    if cfg.length_kind == "fixed":
        n = np.array(cfg.fixed_lengths, dtype=np.int64)
    elif cfg.length_kind == "uniform":
        n = rng.integers(cfg.uniform_lo, cfg.uniform_hi + 1, size=cfg.num_seqs)
    elif cfg.length_kind == "lognormal":
        x = rng.lognormal(cfg.lognormal_mu, cfg.lognormal_sigma, size=cfg.num_seqs)
        n = np.clip(np.rint(x), cfg.clip_lo, cfg.clip_hi).astype(np.int64)
    elif cfg.length_kind == "prefix":
        b = rng.integers(cfg.uniform_lo, cfg.uniform_hi + 1, size=cfg.num_seqs)
        n = cfg.prefix_tokens + b
    else:
        raise ValueError(cfg.length_kind)
    assert n.shape == (cfg.num_seqs,)
    assert (n >= 0).all() and (n <= cfg.max_context).all()
    return n.astype(np.int32)


def pool_blocks_for(cfg: Config, lengths: np.ndarray) -> int:
    if cfg.pool_blocks is not None:
        return int(cfg.pool_blocks)
    # prefix config: shared prefix blocks + every private block, plus slack
    B = cfg.block_size
    pre = cfg.prefix_tokens // B
    priv = sum(cfg.blocks_for(int(n)) - pre for n in lengths)
    return int(math.ceil((pre + priv) * cfg.pool_slack))


def draw_tables(cfg: Config, lengths: np.ndarray, num_blocks: int) -> np.ndarray:
    """Block tables dealt from a seeded shuffled free list; padding is -1."""
    rng = _rng(cfg.cfg_id, 0, S_TABLES)
    S, W = cfg.num_seqs, cfg.max_blocks_per_seq
    free = rng.permutation(num_blocks).astype(np.int32)
    tables = np.full((S, W), -1, dtype=np.int32)
    pos = 0
    shared: List[int] = []
    if cfg.length_kind == "prefix":
        npre = cfg.prefix_tokens // cfg.block_size
        shared = list(free[:npre])
        pos = npre
    for s in range(S):
        need = cfg.blocks_for(int(lengths[s]))
        row = list(shared[:need])
        k = need - len(row)
        if pos + k > num_blocks:
            raise MemoryError("pool exhausted while dealing block tables")
        row += list(free[pos:pos + k])
        pos += k
        tables[s, :need] = row
    return tables


# --------------------------------------------------------------------------
# workload
# --------------------------------------------------------------------------
@dataclass
class Workload:
    cfg: Config
    layer: int
    lengths: np.ndarray      # int32 [S]
    tables: np.ndarray       # int32 [S, W]
    num_blocks: int
    q: np.ndarray            # uint16 [S, Hq, D]
    k_new: np.ndarray        # uint16 [S, Hkv, D]
    v_new: np.ndarray        # uint16 [S, Hkv, D]
    seg_tables: np.ndarray   # int32 [nseg, W]
    seg_start: np.ndarray    # int32 [nseg] first logical position of the segment
    seg_cu: np.ndarray       # int64 [nseg+1] row offsets into k_src/v_src
    k_src: np.ndarray        # uint16 [T, Hkv, D]
    v_src: np.ndarray        # uint16 [T, Hkv, D]
    seq_segments: List[Tuple[int, ...]]  # history segments of each sequence, in order

    @property
    def dtype(self) -> str:
        return self.cfg.dtype

    @property
    def nan_bits(self) -> int:
        return NAN_BITS[self.cfg.dtype]

    def pool_shape(self) -> Tuple[int, int, int, int]:
        c = self.cfg
        return (self.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)

    def logical_kv(self, s: int) -> Tuple[np.ndarray, np.ndarray]:
        """Contiguous K, V of sequence s for positions 0..n-1 ([n, Hkv, D] bits)."""
        ks, vs = [], []
        for g in self.seq_segments[s]:
            a, b = int(self.seg_cu[g]), int(self.seg_cu[g + 1])
            ks.append(self.k_src[a:b])
            vs.append(self.v_src[a:b])
        if int(self.lengths[s]) > 0:
            ks.append(self.k_new[s:s + 1])
            vs.append(self.v_new[s:s + 1])
        shp = (0, self.cfg.num_kv_heads, self.cfg.head_dim)
        K = np.concatenate(ks) if ks else np.zeros(shp, np.uint16)
        V = np.concatenate(vs) if vs else np.zeros(shp, np.uint16)
        assert K.shape[0] == int(self.lengths[s])
        return K, V

    def total_history_tokens(self) -> int:
        return int(self.seg_cu[-1])


def _segments(cfg: Config, lengths: np.ndarray, tables: np.ndarray):
    """History segments: (table row, start position, token count)."""
    segs = []
    seq_segs: List[Tuple[int, ...]] = []
    if cfg.length_kind == "prefix":
        P = cfg.prefix_tokens
        segs.append((0, 0, P))
        for s in range(cfg.num_seqs):
            segs.append((s, P, int(lengths[s]) - 1 - P))
            seq_segs.append((0, 1 + s))
    else:
        for s in range(cfg.num_seqs):
            segs.append((s, 0, max(int(lengths[s]) - 1, 0)))
            seq_segs.append((s,))
    return segs, seq_segs


def _fill_parallel(jobs, threads: int):
    if threads <= 1 or len(jobs) <= 1:
        for j in jobs:
            j()
        return
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda f: f(), jobs))


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_workload(cfg: Config, layer: int = 0, lengths: Sequence[int] | None = None,
                  threads: int | None = None) -> Workload:
    """Build the seeded inputs of one layer of one decode step.

    ``lengths`` overrides the config's drawn lengths (used for small edge-case
    tests); tables are then dealt for those lengths.
    """
    if lengths is None:
        n = draw_lengths(cfg)
    else:
        n = np.asarray(lengths, dtype=np.int32)
        assert n.shape == (cfg.num_seqs,)
    NB = pool_blocks_for(cfg, n)
    tables = draw_tables(cfg, n, NB)
    S, Hq, Hkv, D = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    sc, dt = cfg.value_scale, cfg.dtype

    q = _normal_bits(_rng(cfg.cfg_id, layer, S_Q), (S, Hq, D), sc, dt)
    k_new = _normal_bits(_rng(cfg.cfg_id, layer, S_KNEW), (S, Hkv, D), sc, dt)
    v_new = _normal_bits(_rng(cfg.cfg_id, layer, S_VNEW), (S, Hkv, D), sc, dt)

    segs, seq_segs = _segments(cfg, n, tables)
    counts = np.array([c for (_, _, c) in segs], dtype=np.int64)
    cu = np.zeros(len(segs) + 1, dtype=np.int64)
    np.cumsum(counts, out=cu[1:])
    T = int(cu[-1])
    k_src = np.empty((T, Hkv, D), dtype=np.uint16)
    v_src = np.empty((T, Hkv, D), dtype=np.uint16)

    def job(i, stream, dst):
        def run():
            a, b = int(cu[i]), int(cu[i + 1])
            if b > a:
                dst[a:b] = _normal_bits(_rng(cfg.cfg_id, layer, stream, i), (b - a, Hkv, D), sc, dt)
        return run

    jobs = [job(i, S_KHIST, k_src) for i in range(len(segs))]
    jobs += [job(i, S_VHIST, v_src) for i in range(len(segs))]
    _fill_parallel(jobs, default_threads() if threads is None else threads)

    seg_tables = np.ascontiguousarray(tables[[r for (r, _, _) in segs]])
    seg_start = np.array([st for (_, st, _) in segs], dtype=np.int32)
    return Workload(cfg=cfg, layer=layer, lengths=n, tables=tables, num_blocks=NB,
                    q=q, k_new=k_new, v_new=v_new, seg_tables=seg_tables,
                    seg_start=seg_start, seg_cu=cu, k_src=k_src, v_src=v_src,
                    seq_segments=seq_segs)
