"""Seeded radix-tree batch for slotted-segment decode.

A tree of prompt nodes is laid out in a block pool by the slot-packing rule of the
mhpq.cn page on Radix-Tree fragmentation (sections "核心设计原则" and "物理内存管理器
核心逻辑实现"): a node shorter than a block is packed into the first partly filled
block with enough free slots, at the block's first free offset, else at offset 0
of the next block taken from the free list; a node of a block or more takes whole
blocks of its own.  Every sequence of the batch walks root -> level-1 node ->
level-2 node -> its own leaf, so nodes are shared by many sequences and short
ones share blocks with unrelated nodes.  Each sequence is described by the
(block_id, slot_offset, length) segments of the nodes on its path.

Like the rest of this package this draws inputs only: node lengths, the block
free list, K/V rows and queries.  The segment triples are the allocator's
output, not an address computation of the method; each side writes the node
rows into its own pool copy with its own code (one run per segment).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .configs import Config
from .gen import NAN_BITS, f32_to_bf16_bits, f32_to_f16_bits

# tree shape of the batch
ROOT_TOKENS = 512          # shared system prompt (whole blocks)
LEVEL1 = (16, 5, 40)       # nodes, min and max tokens
LEVEL2 = (64, 3, 15)
LEAF = (5, 128)            # private tail of each sequence

# stream ids (disjoint from the decode generator's)
S_LENS, S_FREE, S_NODE_K, S_NODE_V, S_Q, S_NEW_K, S_NEW_V = range(20, 27)

Segment = Tuple[int, int, int]


def _rng(cfg_id: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, 0, stream, index]))


def _bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_f16_bits(x) if dtype == "fp16" else f32_to_bf16_bits(x)


@dataclass
class SlottedWorkload:
    cfg: Config
    num_blocks: int
    node_segments: List[List[Segment]]
    node_k: List[np.ndarray]        # per node [len][Hkv][D] bits
    node_v: List[np.ndarray]
    paths: List[List[int]]          # node ids per sequence, root first
    q: np.ndarray                   # [S][Hq][D] bits
    segments: np.ndarray            # int32 [S][max_segments][3]
    num_segments: np.ndarray        # int32 [S]
    nan_bits: int
    k_new: np.ndarray = None        # [S][Hkv][D] bits: the step's new rows, which an
    v_new: np.ndarray = None        # append writes to the last row of each leaf

    def logical_kv(self, s: int):
        p = self.paths[s]
        return (np.concatenate([self.node_k[i] for i in p]),
                np.concatenate([self.node_v[i] for i in p]))

    def lengths(self) -> np.ndarray:
        return np.array([sum(len(self.node_k[i]) for i in p) for p in self.paths], np.int64)

    def unique_tokens(self) -> int:
        return sum(len(k) for k in self.node_k)

    def runs(self):
        """One run per segment (rows, start offset, one-entry table): the rows of
        the segment go to positions offset .. offset+length-1 of that block."""
        rows_k, rows_v, starts, tables, cu = [], [], [], [], [0]
        for segs, k, v in zip(self.node_segments, self.node_k, self.node_v):
            r = 0
            for blk, off, ln in segs:
                rows_k.append(k[r:r + ln])
                rows_v.append(v[r:r + ln])
                starts.append(off)
                tables.append([blk])
                cu.append(cu[-1] + ln)
                r += ln
        return (np.concatenate(rows_k), np.concatenate(rows_v), np.array(cu, np.int64),
                np.array(starts, np.int32), np.array(tables, np.int32))

    def pool_shape(self):
        c = self.cfg
        return (self.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)


def pack(node_lens, block_size: int, free_list: List[int]) -> List[List[Segment]]:
    """Lay out nodes (lengths >= 1) by the page's slot-packing rule: a node shorter
    than a block goes into the first slotted block, in the order the blocks were
    opened, that still has room for it, at that block's first free row; with no
    such block, the next block of the free list is opened for it (offset 0).  A
    node of a block or more takes whole blocks of its own from the free list.

    Kept as two arrays over the opened slotted blocks (block id, rows in use), so
    the first fit is a vectorised search over `used + n <= block_size`; a full
    block never fits again."""
    B = block_size
    take = iter(free_list)  # blocks come from the head of the free list
    ids = np.zeros(0, np.int64)    # slotted blocks in the order they were opened
    used = np.zeros(0, np.int64)   # rows in use in each of them
    out: List[List[Segment]] = []
    for n in node_lens:
        n = int(n)
        assert n >= 1, "nodes hold at least one token"
        if n >= B:
            blocks = [next(take) for _ in range(-(-n // B))]
            out.append([(int(b), 0, min(B, n - i * B)) for i, b in enumerate(blocks)])
            continue
        fit = np.flatnonzero(used + n <= B)
        if fit.size:
            j = int(fit[0])
            out.append([(int(ids[j]), int(used[j]), n)])
            used[j] += n
        else:
            b = next(take)
            ids = np.append(ids, b)
            used = np.append(used, n)
            out.append([(int(b), 0, n)])
    return out


def make_slotted_workload(cfg: Config, num_seqs: int = None, seed_id: int = None) -> SlottedWorkload:
    c = cfg
    S = num_seqs or c.num_seqs
    cid = c.cfg_id if seed_id is None else seed_id
    B, Hkv, Hq, D = c.block_size, c.num_kv_heads, c.num_q_heads, c.head_dim
    lr = _rng(cid, S_LENS)
    n1, lo1, hi1 = LEVEL1
    n2, lo2, hi2 = LEVEL2
    n1, n2 = min(n1, S), min(n2, S)
    lens = ([ROOT_TOKENS] + [int(x) for x in lr.integers(lo1, hi1 + 1, size=n1)] +
            [int(x) for x in lr.integers(lo2, hi2 + 1, size=n2)] +
            [int(x) for x in lr.integers(LEAF[0], LEAF[1] + 1, size=S)])
    need = sum(-(-n // B) for n in lens)
    num_blocks = int(math.ceil(need * 1.15)) + 1
    free = [int(x) for x in _rng(cid, S_FREE).permutation(num_blocks)]
    node_segs = pack(lens, B, free)
    scale = c.value_scale
    node_k = [_bits(_rng(cid, S_NODE_K, i).standard_normal((n, Hkv, D), dtype=np.float32) * scale,
                    c.dtype) for i, n in enumerate(lens)]
    node_v = [_bits(_rng(cid, S_NODE_V, i).standard_normal((n, Hkv, D), dtype=np.float32) * scale,
                    c.dtype) for i, n in enumerate(lens)]
    paths = [[0, 1 + s % n1, 1 + n1 + s % n2, 1 + n1 + n2 + s] for s in range(S)]
    max_segs = max(sum(len(node_segs[i]) for i in p) for p in paths)
    segments = np.zeros((S, max_segs, 3), np.int32)
    num_segments = np.zeros(S, np.int32)
    for s, p in enumerate(paths):
        flat = [x for i in p for x in node_segs[i]]
        segments[s, :len(flat)] = flat
        num_segments[s] = len(flat)
    q = _bits(_rng(cid, S_Q).standard_normal((S, Hq, D), dtype=np.float32) * scale, c.dtype)
    k_new = _bits(_rng(cid, S_NEW_K).standard_normal((S, Hkv, D), dtype=np.float32) * scale,
                  c.dtype)
    v_new = _bits(_rng(cid, S_NEW_V).standard_normal((S, Hkv, D), dtype=np.float32) * scale,
                  c.dtype)
    return SlottedWorkload(cfg=c, num_blocks=num_blocks, node_segments=node_segs, node_k=node_k,
                           node_v=node_v, paths=paths, q=q, segments=segments,
                           num_segments=num_segments, nan_bits=NAN_BITS[c.dtype], k_new=k_new,
                           v_new=v_new)
