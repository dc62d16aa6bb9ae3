"""Pins of the oracle's block copy (copy-on-write) against the page's fork
example (tests/golden/cow_fork.json) and brute force over each branch's logical
arrays.  No expectation here comes from the oracle."""
import json
import math
import os

import numpy as np
import pytest

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(1.0 / math.sqrt(128)))
SENTINEL = 0x7E00


def _fork(oracle_lib, case, B, NB, Hkv=2, Hq=4, D=128, seed=0):
    """Run the page's fork: write the prompt through the shared table, apply the
    case's copies, append one token per branch, and attend for each branch."""
    O = oracle_lib
    rng = np.random.default_rng(seed)
    T = case["prompt_tokens"]

    def draw(*shape):
        return (rng.standard_normal(shape) * 0.5).astype(np.float16).view(np.uint16)

    prompt_k, prompt_v = draw(T, Hkv, D), draw(T, Hkv, D)
    new = {b: (draw(1, Hkv, D), draw(1, Hkv, D)) for b in "AB"}
    q = draw(2, Hq, D)
    kp = np.full((NB, Hkv, B, D), SENTINEL, np.uint16)
    vp = kp.copy()
    O.append_tokens(kp, vp, prompt_k, prompt_v, np.array([0, T], np.int64),
                    np.array([0], np.int32), np.array([case["prompt_table"]], np.int32), B, NB)
    before_k, before_v = kp.copy(), vp.copy()
    if case["copies"]:
        src, dst = zip(*case["copies"])
        O.copy_blocks(kp, vp, np.array(src, np.int32), np.array(dst, np.int32))
    W = max(len(t) for t in case["tables_after"].values())
    tables = np.full((2, W), -1, np.int32)
    for i, b in enumerate("AB"):
        tables[i, :len(case["tables_after"][b])] = case["tables_after"][b]
    lens = np.array([T + 1, T + 1], np.int32)
    # one branch at a time, as the block manager orders them (A's copy first)
    for i, b in enumerate("AB"):
        slots = O.append(kp, vp, new[b][0], new[b][1], tables[i:i + 1], lens[i:i + 1], B, NB)
        w = case["writes"][b]
        assert slots[0] == w["phys"] * B + w["offset"]
    out = O.attention(q, kp, vp, tables, lens, Hkv, B, NB, SCALE, "fp16")
    logical = {b: (np.concatenate([prompt_k, new[b][0]]), np.concatenate([prompt_v, new[b][1]]))
               for b in "AB"}
    return dict(kp=kp, vp=vp, before_k=before_k, before_v=before_v, out=out, q=q,
                logical=logical, prompt=(prompt_k, prompt_v), new=new)


@pytest.mark.parametrize("name", ["fresh_blocks", "copy_on_write"])
def test_fork_matches_each_branch_logical_sequence(oracle_lib, name):
    g = json.load(open(os.path.join(GOLDEN, "cow_fork.json")))
    B, NB = g["block_size"], g["pool_blocks"]
    r = _fork(oracle_lib, g["cases"][name], B, NB)
    G = r["q"].shape[1] // r["logical"]["A"][0].shape[1]
    for i, b in enumerate("AB"):
        K, V = (brute.widen(x, "fp16") for x in r["logical"][b])
        q = brute.widen(r["q"][i], "fp16")
        for h in range(q.shape[0]):
            ref = brute.attention_one(q[h], K[:, h // G], V[:, h // G], SCALE)
            assert np.allclose(r["out"][i, h], ref, rtol=0, atol=1e-12)


def test_copy_on_write_block_contents(oracle_lib):
    """#45 holds the prompt's tokens 16..19 (copied), A's new token at offset 4 and
    the copied sentinel rows after it; #11 keeps the prompt rows plus B's token."""
    g = json.load(open(os.path.join(GOLDEN, "cow_fork.json")))
    B, NB = g["block_size"], g["pool_blocks"]
    r = _fork(oracle_lib, g["cases"]["copy_on_write"], B, NB)
    pk, pv = r["prompt"]
    kp, vp = r["kp"], r["vp"]
    for pool, prompt, j in ((kp, pk, 0), (vp, pv, 1)):
        assert (pool[45, :, :4, :] == prompt[16:20].transpose(1, 0, 2)).all()
        assert (pool[11, :, :4, :] == prompt[16:20].transpose(1, 0, 2)).all()
        assert (pool[10] == prompt[:16].transpose(1, 0, 2)).all()
        assert (pool[45, :, 4, :] == r["new"]["A"][j][0]).all()
        assert (pool[11, :, 4, :] == r["new"]["B"][j][0]).all()
        assert (pool[45, :, 5:, :] == SENTINEL).all() and (pool[11, :, 5:, :] == SENTINEL).all()
    untouched = np.ones(NB, bool)
    untouched[[11, 45]] = False
    assert (kp[untouched] == r["before_k"][untouched]).all()
    assert (vp[untouched] == r["before_v"][untouched]).all()


def test_copy_duplicates_whole_blocks_and_nothing_else(oracle_lib):
    rng = np.random.default_rng(5)
    NB, Hkv, B, D = 40, 3, 16, 8
    kp = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    vp = rng.integers(0, 1 << 16, size=(NB, Hkv, B, D), dtype=np.uint16)
    k0, v0 = kp.copy(), vp.copy()
    src = np.array([3, 3, 17, 39, 0], np.int32)      # a source may fork into several copies
    dst = np.array([5, 6, 1, 38, 20], np.int32)
    oracle_lib.copy_blocks(kp, vp, src, dst)
    for s_, d_ in zip(src, dst):
        assert (kp[d_] == k0[s_]).all() and (vp[d_] == v0[s_]).all()
    keep = np.setdiff1d(np.arange(NB), dst)
    assert (kp[keep] == k0[keep]).all() and (vp[keep] == v0[keep]).all()
    assert not np.shares_memory(kp, k0)


@pytest.mark.parametrize("src,dst", [
    ([1, 2], [2, 3]),     # a destination that is also a source: order-dependent
    ([1, 2], [3, 3]),     # two copies into one block
    ([1], [40]),          # outside the pool
    ([-1], [3]),
])
def test_copy_rejects_ambiguous_or_out_of_range(oracle_lib, src, dst):
    kp = np.zeros((40, 1, 16, 8), np.uint16)
    vp = kp.copy()
    with pytest.raises(oracle_lib.OracleError):
        oracle_lib.copy_blocks(kp, vp, np.array(src, np.int32), np.array(dst, np.int32))


def test_empty_copy_list_is_a_no_op(oracle_lib):
    kp = np.arange(2 * 16 * 8, dtype=np.uint16).reshape(2, 1, 16, 8)
    vp = kp.copy()
    oracle_lib.copy_blocks(kp, vp, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert (kp == vp).all() and kp[1, 0, 0, 0] == 128
