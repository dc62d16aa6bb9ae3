"""Pins of the oracle's slot copy (the copy-on-write split of a node held in a
shared slot) against the page's slot example (tests/golden/slot_cow.json),
row-for-row moves written out with numpy slicing, and brute-force attention over
each path's logical arrays after the split and the append.  No expectation here
comes from the oracle."""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(1.0 / math.sqrt(128)))


def _marked_pools(NB, Hkv, B, D, seed):
    """Pools whose every element holds distinct random bits (finite fp16)."""
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((NB, Hkv, B, D)) * 0.5).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((NB, Hkv, B, D)) * 0.5).astype(np.float16).view(np.uint16)
    return np.ascontiguousarray(k), np.ascontiguousarray(v)


def _golden():
    return json.load(open(os.path.join(GOLDEN, "slot_cow.json")))


def test_page_example_moves_exactly_the_node_rows(oracle_lib):
    g = _golden()
    B, NB, c = g["block_size"], g["pool_blocks"], g["copy"]
    for Hkv in (1, 2, 8):
        kp, vp = _marked_pools(NB, Hkv, B, 128, seed=Hkv)
        want_k, want_v = kp.copy(), vp.copy()
        n = c["length"]
        want_k[c["dst_block"], :, c["dst_offset"]:c["dst_offset"] + n] = \
            kp[c["src_block"], :, c["src_offset"]:c["src_offset"] + n]
        want_v[c["dst_block"], :, c["dst_offset"]:c["dst_offset"] + n] = \
            vp[c["src_block"], :, c["src_offset"]:c["src_offset"] + n]
        oracle_lib.copy_slots(kp, vp, [[c["src_block"], c["src_offset"], c["dst_block"],
                                        c["dst_offset"], n]])
        assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)
        # exactly the rows the fixture names differ from the pools before the copy
        rw = g["rows_written"]
        k0, v0 = _marked_pools(NB, Hkv, B, 128, seed=Hkv)
        for pool, before in ((kp, k0), (vp, v0)):
            rows = {(int(b), int(r)) for b, h, r in np.argwhere((pool != before).any(axis=3))}
            assert rows == {(rw["block"], r) for r in range(rw["first"], rw["first"] + rw["count"])}


def test_split_then_append_then_attend(oracle_lib):
    """The page's split inside a decode step: nodes packed as in slotted_blocks.json;
    path X = A,B keeps reading B's old slot, path Y = A,B appends a token, so B is
    split into block 4 first and Y's token lands at (4, 8).  Each path's attention
    equals brute force over its own logical rows, and block 0 never changes."""
    O = oracle_lib
    g = _golden()
    B, NB = g["block_size"], g["pool_blocks"]
    Hkv, Hq, D = 2, 4, 128
    rng = np.random.default_rng(7)

    def draw(*shape):
        return (rng.standard_normal(shape) * 0.5).astype(np.float16).view(np.uint16)

    nodes = {name: sum(s[2] for s in segs) for name, segs in g["before"].items()}
    rows = {name: (draw(n, Hkv, D), draw(n, Hkv, D)) for name, n in nodes.items()}
    kp = np.full((NB, Hkv, B, D), 0x7E00, np.uint16)
    vp = kp.copy()
    for name, segs in g["before"].items():
        r = 0
        for blk, off, ln in segs:
            O.append_tokens(kp, vp, rows[name][0][r:r + ln], rows[name][1][r:r + ln],
                            np.array([0, ln], np.int64), np.array([off], np.int32),
                            np.array([[blk]], np.int32), B, NB)
            r += ln
    block0_k, block0_v = kp[0].copy(), vp[0].copy()
    c = g["copy"]
    O.copy_slots(kp, vp, [[c["src_block"], c["src_offset"], c["dst_block"], c["dst_offset"],
                           c["length"]]])
    new_k, new_v = draw(1, Hkv, D), draw(1, Hkv, D)
    a = g["append"]
    O.append_tokens(kp, vp, new_k, new_v, np.array([0, 1], np.int64),
                    np.array([a["offset"]], np.int32), np.array([[a["block"]]], np.int32), B, NB)
    assert np.array_equal(kp[0], block0_k) and np.array_equal(vp[0], block0_v)
    b_after = g["after"]["B"][0]
    segs = np.zeros((2, 2, 3), np.int32)
    segs[0] = [g["before"]["A"][0], g["before"]["B"][0]]                  # X
    segs[1] = [g["before"]["A"][0], [b_after[0], b_after[1], b_after[2] + 1]]  # Y, grown
    nseg = np.array([2, 2], np.int32)
    q = draw(2, Hq, D)
    out = O.attention_slotted(q, kp, vp, segs, nseg, Hkv, B, NB, SCALE, "fp16")
    lx = (np.concatenate([rows["A"][0], rows["B"][0]]), np.concatenate([rows["A"][1], rows["B"][1]]))
    ly = (np.concatenate([rows["A"][0], rows["B"][0], new_k]),
          np.concatenate([rows["A"][1], rows["B"][1], new_v]))
    G = Hq // Hkv
    qd = brute.widen(q, "fp16")
    for s, (lk, lv) in enumerate((lx, ly)):
        K, V = brute.widen(lk, "fp16"), brute.widen(lv, "fp16")
        for h in range(Hq):
            ref = brute.attention_one(qd[s, h], K[:, h // G], V[:, h // G], SCALE)
            assert np.abs(out[s, h] - ref).max() <= 1e-12


def test_any_destination_offset_and_several_copies(oracle_lib):
    """Several copies in one call, to non-zero destination offsets and within one
    block, against the same moves written with numpy slicing."""
    NB, Hkv, B = 6, 3, 32
    kp, vp = _marked_pools(NB, Hkv, B, 128, seed=11)
    copies = [[1, 3, 4, 10, 7], [1, 3, 5, 0, 7], [2, 0, 2, 20, 12], [0, 31, 3, 0, 1],
              [5, 16, 0, 0, 0]]
    want_k, want_v = kp.copy(), vp.copy()
    for sb, so, db, do, n in copies:
        want_k[db, :, do:do + n] = kp[sb, :, so:so + n]
        want_v[db, :, do:do + n] = vp[sb, :, so:so + n]
    oracle_lib.copy_slots(kp, vp, copies)
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)


@pytest.mark.parametrize("copies", [
    [[0, 0, 1, 0, 8], [1, 4, 2, 0, 4]],     # a destination read by another copy
    [[0, 0, 1, 0, 8], [2, 0, 1, 7, 4]],     # two destinations overlap
    [[0, 0, 0, 4, 8]],                      # source and destination overlap in one block
    [[0, 10, 1, 0, 8]],                     # source rows past the block
    [[0, 0, 1, 9, 8]],                      # destination rows past the block
    [[0, 0, 16, 0, 4]],                     # destination block outside the pool
    [[0, -1, 1, 0, 4]],
])
def test_order_dependent_or_out_of_range_copies_are_rejected(oracle_lib, copies):
    kp, vp = _marked_pools(16, 1, 16, 128, seed=3)
    kp = kp[:16]
    with pytest.raises(Exception):
        oracle_lib.copy_slots(np.ascontiguousarray(kp), np.ascontiguousarray(vp), copies)
