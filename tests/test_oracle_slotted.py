"""Pins of the oracle's slotted-segment walk and attention: the page's slot
example (tests/golden/slotted_blocks.json), brute force over logical arrays, and
the reduction to an ordinary block table.  No expectation comes from the oracle."""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute
from workloads.slotted import make_slotted_workload, pack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(1.0 / math.sqrt(128)))


def golden():
    with open(os.path.join(GOLDEN, "slotted_blocks.json")) as f:
        return json.load(f)


def pack_nodes(node_lens, B, rng=None):
    """The page's slotted allocation (workloads.slotted.pack) on the free list
    [0, 1, 2, ...]; returns per-node segment lists and the blocks used."""
    segs = [[list(x) for x in node] for node in pack(node_lens, B, list(range(10 ** 5)))]
    used = max(s[0] for node in segs for s in node) + 1
    return segs, used


def test_golden_allocation_follows_the_page_policy():
    g = golden()
    names = ["A", "B", "C", "D", "E"]
    lens = [sum(s[2] for s in g["allocations"][k]) for k in names]
    segs, _ = pack_nodes(lens, g["block_size"])
    for k, sg in zip(names, segs):
        assert sg == g["allocations"][k]


@pytest.mark.parametrize("path", ["A,B", "A,C,D", "A,E"])
def test_golden_walk(oracle_lib, path):
    g = golden()
    case = g["paths"][path]
    segs = [s for k in path.split(",") for s in g["allocations"][k]]
    assert segs == case["segments"]
    assert sum(s[2] for s in segs) == case["length"]
    for t, phys, off in case["token_to_slot"]:
        assert oracle_lib.locate_slotted(segs, g["block_size"], g["pool_blocks"], t) == (phys, off)
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.locate_slotted(segs, g["block_size"], g["pool_blocks"], case["length"])


def test_walk_rejects_bad_segments(oracle_lib):
    O = oracle_lib
    with pytest.raises(O.OracleError):
        O.locate_slotted([[0, 12, 5]], 16, 4, 0)     # slot runs past the block
    with pytest.raises(O.OracleError):
        O.locate_slotted([[0, -1, 5]], 16, 4, 0)     # negative offset
    with pytest.raises(O.OracleError):
        O.locate_slotted([[9, 0, 5]], 16, 4, 2)      # block outside the pool
    assert O.locate_slotted([[3, 4, 0], [2, 1, 3]], 16, 4, 0) == (2, 1)  # empty segment skipped


def _random_slotted(seed, S, Hq, Hkv, B, dtype="fp16", shared_frac=0.5):
    """Sequences whose paths reuse each other's nodes (a tiny radix tree): every
    sequence walks a shared root node, some shared mid nodes and a private tail."""
    rng = np.random.default_rng(seed)
    node_lens = [int(x) for x in rng.integers(1, 2 * B + 5, size=3 * S + 2)]
    segs, NB = pack_nodes(node_lens, B, rng)
    node_k = [rng.standard_normal((L, Hkv, 128)).astype(np.float16).view(np.uint16)
              for L in node_lens]
    node_v = [rng.standard_normal((L, Hkv, 128)).astype(np.float16).view(np.uint16)
              for L in node_lens]
    kp = np.full((NB, Hkv, B, 128), 0x7E00, np.uint16)
    vp = kp.copy()
    for sg, k, v in zip(segs, node_k, node_v):
        r = 0
        for blk, off, ln in sg:
            kp[blk, :, off:off + ln] = k[r:r + ln].transpose(1, 0, 2)
            vp[blk, :, off:off + ln] = v[r:r + ln].transpose(1, 0, 2)
            r += ln
    paths = []
    for s in range(S):
        mids = [1 + int(x) for x in rng.choice(len(node_lens) - 2, size=rng.integers(0, 4),
                                               replace=False)]
        paths.append([0] + mids + [len(node_lens) - 1 - (s % 2)])
    max_segs = max(sum(len(segs[i]) for i in p) for p in paths)
    table = np.zeros((S, max_segs, 3), np.int32)
    nsegs = np.zeros(S, np.int32)
    logical = []
    for s, p in enumerate(paths):
        flat = [x for i in p for x in segs[i]]
        table[s, :len(flat)] = flat
        nsegs[s] = len(flat)
        logical.append((np.concatenate([node_k[i] for i in p]),
                        np.concatenate([node_v[i] for i in p])))
    q = rng.standard_normal((S, Hq, 128)).astype(np.float16).view(np.uint16)
    return dict(kp=kp, vp=vp, table=table, nsegs=nsegs, logical=logical, q=q, NB=NB)


@pytest.mark.parametrize("seed,B,Hq,Hkv", [(1, 16, 12, 2), (2, 16, 4, 4), (3, 4, 8, 2),
                                           (4, 32, 16, 1)])
def test_slotted_attention_matches_brute_force(oracle_lib, seed, B, Hq, Hkv):
    c = _random_slotted(seed, 5, Hq, Hkv, B)
    out = oracle_lib.attention_slotted(c["q"], c["kp"], c["vp"], c["table"], c["nsegs"], Hkv, B,
                                       c["NB"], SCALE, "fp16")
    G = Hq // Hkv
    q = brute.widen(c["q"], "fp16")
    for s, (Kb, Vb) in enumerate(c["logical"]):
        K, V = brute.widen(Kb, "fp16"), brute.widen(Vb, "fp16")
        for h in range(Hq):
            ref = brute.attention_one(q[s, h], K[:, h // G], V[:, h // G], SCALE)
            assert np.allclose(out[s, h], ref, rtol=0, atol=1e-12)


def test_block_table_as_segments_is_bitwise_the_same(oracle_lib):
    """A block table is the special case of whole-block segments plus a partly
    filled last one: same tokens in the same order, so the same bits."""
    from workloads import get_config, make_workload
    w = make_workload(get_config("c1a"))
    c = w.cfg
    r = oracle_lib.run_step(w, SCALE)
    S, B = c.num_seqs, c.block_size
    nb = -(-w.lengths // B)
    table = np.zeros((S, int(nb.max()), 3), np.int32)
    for s in range(S):
        for j in range(nb[s]):
            table[s, j] = (w.tables[s, j], 0, min(B, w.lengths[s] - j * B))
    out = oracle_lib.attention_slotted(w.q, r["k_pool"], r["v_pool"], table, nb.astype(np.int32),
                                       c.num_kv_heads, B, w.num_blocks, SCALE, c.dtype)
    assert np.array_equal(out, r["out"])


def test_empty_sequence_gives_zeros(oracle_lib):
    kp = np.zeros((2, 1, 16, 128), np.uint16)
    q = np.ones((1, 1, 128), np.uint16)
    out = oracle_lib.attention_slotted(q, kp, kp, np.zeros((1, 1, 3), np.int32),
                                       np.zeros(1, np.int32), 1, 16, 2, SCALE, "fp16")
    assert (out == 0).all()


def test_radix_batch_layout(oracle_lib):
    """The seeded radix-tree batch: segments stay inside their blocks, no two
    nodes share a slot, and the oracle over the pools equals brute force over
    the logical arrays of a few sequences."""
    from workloads import get_config
    cfg = get_config("c5")
    w = make_slotted_workload(cfg, num_seqs=24)
    B = cfg.block_size
    owner = {}
    for n, segs in enumerate(w.node_segments):
        assert sum(x[2] for x in segs) == len(w.node_k[n])
        for blk, off, ln in segs:
            assert 0 <= blk < w.num_blocks and off >= 0 and off + ln <= B
            for r in range(off, off + ln):
                assert owner.setdefault((blk, r), n) == n
    kr, vr, cu, st, tb = w.runs()
    kp, vp = oracle_lib.new_pools(w.num_blocks, cfg.num_kv_heads, B, cfg.head_dim, w.nan_bits)
    oracle_lib.append_tokens(kp, vp, kr, vr, cu, st, tb, B, w.num_blocks)
    out = oracle_lib.attention_slotted(w.q, kp, vp, w.segments, w.num_segments, cfg.num_kv_heads,
                                       B, w.num_blocks, SCALE, cfg.dtype)
    G = cfg.num_q_heads // cfg.num_kv_heads
    q = brute.widen(w.q, cfg.dtype)
    for s in (0, 7, 23):
        Kb, Vb = w.logical_kv(s)
        K, V = brute.widen(Kb, cfg.dtype), brute.widen(Vb, cfg.dtype)
        for h in range(0, cfg.num_q_heads, 5):
            ref = brute.attention_one(q[s, h], K[:, h // G], V[:, h // G], SCALE)
            assert np.allclose(out[s, h], ref, rtol=0, atol=1e-12)
