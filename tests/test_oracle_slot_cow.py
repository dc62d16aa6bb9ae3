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


# ---------------------------------------------------------------------------
# the append of a decode step's token to a slotted sequence
# ---------------------------------------------------------------------------
def test_slotted_append_of_the_page_example(oracle_lib):
    """After the split, path Y = A, B lists B as (4, 0, 9): the token counted by its
    grown length lands at the fixture's append slot (4, 8), in every head, K and
    V.  A sequence with no segments (n = 0) gets slot -1 and writes nothing.
    Nothing else in the pool changes."""
    g = _golden()
    B, NB, a = g["block_size"], g["pool_blocks"], g["append"]
    Hkv, D = 2, 128
    kp, vp = _marked_pools(NB, Hkv, B, D, seed=21)
    k0, v0 = kp.copy(), vp.copy()
    rng = np.random.default_rng(22)
    kn = (rng.standard_normal((2, Hkv, D)) * 0.5).astype(np.float16).view(np.uint16)
    vn = (rng.standard_normal((2, Hkv, D)) * 0.5).astype(np.float16).view(np.uint16)
    b_after = g["after"]["B"][0]
    segs = np.zeros((2, 2, 3), np.int32)
    segs[1] = [g["before"]["A"][0], [b_after[0], b_after[1], b_after[2] + 1]]
    nseg = np.array([0, 2], np.int32)
    slots = oracle_lib.append_slotted(kp, vp, kn, vn, segs, nseg, B, NB)
    assert slots.tolist() == [-1, a["block"] * B + a["offset"]]
    want_k, want_v = k0.copy(), v0.copy()
    want_k[a["block"], :, a["offset"]] = kn[1]
    want_v[a["block"], :, a["offset"]] = vn[1]
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)


def test_slotted_append_then_attention_is_brute_force(oracle_lib):
    """Random node lists, each sequence's last segment a private slot: after the
    append, attention over the segments equals brute force over each sequence's
    logical rows with the new row last; zero-length segments and empty
    sequences included."""
    rng = np.random.default_rng(5)
    B, Hkv, Hq, D, NB = 16, 2, 6, 128, 40
    S, MS = 6, 5
    kp, vp = _marked_pools(NB, Hkv, B, D, seed=8)
    free = list(rng.permutation(NB))
    segs = np.zeros((S, MS, 3), np.int32)
    nseg = np.zeros(S, np.int32)
    for s in range(S):
        ns = int(rng.integers(0, MS + 1)) if s else 0
        for i in range(ns):
            blk = int(free.pop())
            off = int(rng.integers(0, B))
            ln = int(rng.integers(0, B - off + 1)) if i < ns - 1 else int(rng.integers(1, B - off + 1))
            segs[s, i] = (blk, off, ln)
        nseg[s] = ns
    logical = []
    for s in range(S):
        rows = [(kp[b, :, o:o + ln].transpose(1, 0, 2), vp[b, :, o:o + ln].transpose(1, 0, 2))
                for b, o, ln in segs[s, :nseg[s]]]
        logical.append(rows)
    kn = (rng.standard_normal((S, Hkv, D)) * 0.5).astype(np.float16).view(np.uint16)
    vn = (rng.standard_normal((S, Hkv, D)) * 0.5).astype(np.float16).view(np.uint16)
    slots = oracle_lib.append_slotted(kp, vp, kn, vn, segs, nseg, B, NB)
    q = (rng.standard_normal((S, Hq, D)) * 0.5).astype(np.float16).view(np.uint16)
    out = oracle_lib.attention_slotted(q, kp, vp, segs, nseg, Hkv, B, NB, SCALE, "fp16")
    G = Hq // Hkv
    qd = brute.widen(q, "fp16")
    for s in range(S):
        n = int(segs[s, :nseg[s], 2].sum())
        if n == 0:
            assert slots[s] == -1
            assert np.all(out[s] == 0.0)
            continue
        lk = np.concatenate([r[0] for r in logical[s]]) if logical[s] else np.zeros((0, Hkv, D), np.uint16)
        lv = np.concatenate([r[1] for r in logical[s]]) if logical[s] else np.zeros((0, Hkv, D), np.uint16)
        # the last logical row is the new token's
        lk = np.concatenate([lk[:n - 1], kn[s:s + 1]])
        lv = np.concatenate([lv[:n - 1], vn[s:s + 1]])
        b, o, ln = [x for x in segs[s, :nseg[s]] if x[2] > 0][-1]
        assert slots[s] == b * B + o + ln - 1
        K, V = brute.widen(lk, "fp16"), brute.widen(lv, "fp16")
        for h in range(Hq):
            ref = brute.attention_one(qd[s, h], K[:, h // G], V[:, h // G], SCALE)
            assert np.abs(out[s, h] - ref).max() <= 1e-12


def test_slotted_append_rejects_two_writes_to_one_slot(oracle_lib):
    B, Hkv, D, NB = 16, 1, 128, 4
    kp, vp = _marked_pools(NB, Hkv, B, D, seed=9)
    segs = np.array([[[2, 0, 5]], [[2, 0, 5]]], np.int32)   # both end on (2, 4)
    kn = np.zeros((2, Hkv, D), np.uint16)
    with pytest.raises(Exception):
        oracle_lib.append_slotted(kp, vp, kn, kn, segs, np.array([1, 1], np.int32), B, NB)
