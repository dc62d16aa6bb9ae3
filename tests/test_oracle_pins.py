"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these expectations is produced by the oracle itself: they are the pages'
printed numbers and worked examples (tests/golden/*.json), textbook decodings,
brute force over the contiguous logical arrays, closed forms and invariants.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

from workloads import get_config, make_workload
from workloads.gen import NAN_BITS
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SCALE = float(np.float32(1.0 / math.sqrt(128)))


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def tiny_cfg(block_size=16, lengths=(5, 16, 37, 64), hq=12, hkv=2, dtype="fp16", pool=None,
             width=None, key="tiny"):
    base = get_config("c1a")
    W = width or max(1, -(-max(lengths) // block_size))
    NB = pool or (sum(-(-n // block_size) for n in lengths) + 3)
    return dataclasses.replace(base, key=key, num_seqs=len(lengths), num_q_heads=hq,
                               num_kv_heads=hkv, block_size=block_size, dtype=dtype,
                               max_blocks_per_seq=W, fixed_lengths=tuple(lengths),
                               pool_blocks=NB)


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def _val(v):
    return {"inf": math.inf, "-inf": -math.inf, "nan": math.nan}.get(v, v) if isinstance(v, str) else v


def test_storage_format_decoding(oracle_lib):
    g = golden("storage_formats.json")
    for hexbits, v in g["fp16"]:
        got = oracle_lib.fp16_to_double(int(hexbits, 16))
        exp = _val(v)
        if math.isnan(exp):
            assert math.isnan(got)
        else:
            assert got == exp and math.copysign(1, got) == math.copysign(1, exp), hexbits
    for hexbits, v in g["bf16"]:
        got = oracle_lib.bf16_to_double(int(hexbits, 16))
        exp = _val(v)
        assert (math.isnan(got) and math.isnan(exp)) or got == exp, hexbits


# ---------------------------------------------------------------------------
# byte accounting of the layout
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", golden("kv_bytes.json")["cases"])
def test_kv_bytes(oracle_lib, case):
    O = oracle_lib
    Hkv, D, e, L = case["num_kv_heads"], case["head_dim"], case["elem_bytes"], case["layers"]
    B = case.get("block_size", 16)
    # element offsets one token occupies in one pool: all heads, all dims
    offs = {O.elem_offset(5, h, 3, d, Hkv, B, D) for h in range(Hkv) for d in range(D)}
    per_token_layer = 2 * len(offs) * e  # K pool + V pool
    if "bytes_per_token_per_layer" in case:
        assert per_token_layer == case["bytes_per_token_per_layer"]
        assert per_token_layer * L == case["bytes_per_token_all_layers"]
    # one physical block is one contiguous slab of the pool
    start = O.elem_offset(7, 0, 0, 0, Hkv, B, D)
    nxt = O.elem_offset(8, 0, 0, 0, Hkv, B, D)
    slab = {O.elem_offset(7, h, t, d, Hkv, B, D) for h in range(Hkv) for t in range(B)
            for d in range(0, D, 17)}
    assert min(slab) == start and max(slab) < nxt
    if "block_bytes_all_layers" in case:
        assert 2 * (nxt - start) * e * L == case["block_bytes_all_layers"]


# ---------------------------------------------------------------------------
# the address walk and the append, against the worked example
# ---------------------------------------------------------------------------
def test_worked_address_walk(oracle_lib):
    g = golden("address_walk.json")
    B, NB = g["block_size"], g["pool_blocks"]
    for t, phys, off in g["token_to_block"]:
        assert oracle_lib.locate(g["table"], B, NB, t) == (phys, off)
    assert -(-g["prompt_tokens"] // B) == g["prompt_blocks"]
    # the last block of the 38-token prompt holds tokens 32..37
    last = [oracle_lib.locate(g["table"], B, NB, t) for t in range(g["prompt_tokens"])]
    assert sum(1 for p, _ in last if p == g["table"][-1]) == g["prompt_last_block_fill"]


@pytest.mark.parametrize("which", ["decode_write", "new_block_write"])
def test_worked_append(oracle_lib, which):
    g = golden("address_walk.json")
    case = g[which]
    B, NB, Hkv, D = g["block_size"], g["pool_blocks"], 2, 128
    W = len(case["table"])
    kp = np.full((NB, Hkv, B, D), 0x7E00, np.uint16)
    vp = kp.copy()
    rng = np.random.default_rng(3)
    kn = rng.integers(0, 0x7C00, size=(1, Hkv, D), dtype=np.uint16)
    vn = rng.integers(0, 0x7C00, size=(1, Hkv, D), dtype=np.uint16)
    before_k, before_v = kp.copy(), vp.copy()
    slots = oracle_lib.append(kp, vp, kn, vn, np.array([case["table"]], np.int32),
                              np.array([case["attended_len"]], np.int32), B, NB)
    assert slots[0] == case["slot"] == case["phys"] * B + case["offset"]
    # the new rows sit at [phys][h][offset][:] of the [NB][Hkv][B][D] pools ...
    assert (kp[case["phys"], :, case["offset"], :] == kn[0]).all()
    assert (vp[case["phys"], :, case["offset"], :] == vn[0]).all()
    # ... and nothing else moved
    mask = np.ones(kp.shape, bool)
    mask[case["phys"], :, case["offset"], :] = False
    assert (kp[mask] == before_k[mask]).all() and (vp[mask] == before_v[mask]).all()
    del W


def test_locate_rejects_out_of_range(oracle_lib):
    O = oracle_lib
    with pytest.raises(O.OracleError):
        O.locate([7, 3, 12], 16, 26, 48)        # past the table row
    with pytest.raises(O.OracleError):
        O.locate([7, -1, 12], 16, 26, 20)       # padding entry
    with pytest.raises(O.OracleError):
        O.locate([7, 3, 30], 16, 26, 40)        # entry outside the pool
    with pytest.raises(O.OracleError):
        O.locate([7, 3, 12], 16, 26, -1)        # negative position


def test_append_rejects_duplicate_slots(oracle_lib):
    O = oracle_lib
    kp = np.zeros((4, 1, 16, 8), np.uint16)
    vp = kp.copy()
    new = np.ones((2, 1, 8), np.uint16)
    tables = np.array([[2, 3], [1, 3]], np.int32)
    with pytest.raises(O.OracleError):
        O.append(kp, vp, new, new, tables, np.array([20, 20], np.int32), 16, 4)


def test_append_skips_empty_sequences(oracle_lib):
    O = oracle_lib
    kp = np.zeros((4, 1, 16, 8), np.uint16)
    vp = kp.copy()
    new = np.ones((2, 1, 8), np.uint16)
    tables = np.array([[-1, -1], [1, 3]], np.int32)
    slots = O.append(kp, vp, new, new, tables, np.array([0, 17], np.int32), 16, 4)
    assert list(slots) == [-1, 3 * 16 + 0]
    assert kp.sum() == 8 and vp.sum() == 8


def test_history_lands_in_walked_slots(oracle_lib):
    """After writing a workload's history and new tokens, every logical token's
    rows sit at [table[t // B]][h][t % B] of the pools, every other slot still
    holds the sentinel."""
    O = oracle_lib
    w = make_workload(get_config("c1b"))
    c = w.cfg
    r = O.run_step(w, SCALE)
    kp, vp = r["k_pool"], r["v_pool"]
    touched = np.zeros(kp.shape[:1] + kp.shape[2:3], bool)  # [NB, B]
    for s in range(c.num_seqs):
        K, V = w.logical_kv(s)
        for t in range(int(w.lengths[s])):
            phys, off = w.tables[s, t // c.block_size], t % c.block_size
            assert (kp[phys, :, off] == K[t]).all() and (vp[phys, :, off] == V[t]).all()
            touched[phys, off] = True
    assert (kp.transpose(0, 2, 1, 3)[~touched] == NAN_BITS["fp16"]).all()
    assert (vp.transpose(0, 2, 1, 3)[~touched] == NAN_BITS["fp16"]).all()


# ---------------------------------------------------------------------------
# attention: brute force on tiny inputs
# ---------------------------------------------------------------------------
def _random_tiny_cases():
    rng = np.random.default_rng(1234)
    cases = []
    for B in (1, 2, 16):
        for trial in range(3):
            S = int(rng.integers(1, 5))
            lens = tuple(int(x) for x in rng.integers(1, 71, size=S))
            hkv = int(rng.choice([1, 2, 3]))
            G = int(rng.choice([1, 2, 4]))
            dt = "bf16" if trial == 2 else "fp16"
            cases.append((B, lens, hkv * G, hkv, dt))
    return cases


@pytest.mark.parametrize("key", ["c1a", "c1b"])
def test_brute_force_matches_oracle_c1(oracle_lib, key):
    w = make_workload(get_config(key))
    r = oracle_lib.run_step(w, SCALE)
    b = brute.attention(w, SCALE)
    assert np.abs(r["out"] - b).max() <= 1e-12


@pytest.mark.parametrize("B,lens,hq,hkv,dt", _random_tiny_cases())
def test_brute_force_matches_oracle_random(oracle_lib, B, lens, hq, hkv, dt):
    cfg = tiny_cfg(block_size=B, lengths=lens, hq=hq, hkv=hkv, dtype=dt, key=f"rnd{B}")
    w = make_workload(cfg, lengths=lens)
    r = oracle_lib.run_step(w, SCALE)
    b = brute.attention(w, SCALE)
    assert np.abs(r["out"] - b).max() <= 1e-12


# ---------------------------------------------------------------------------
# invariants and closed forms
# ---------------------------------------------------------------------------
def _relabel(kp, vp, tables, seed):
    rng = np.random.default_rng(seed)
    NB = kp.shape[0]
    pi = rng.permutation(NB)
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[pi] = kp
    vp2[pi] = vp
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    return kp2, vp2, t2


@pytest.mark.parametrize("key", ["c1a", "c1b"])
def test_permutation_invariance(oracle_lib, key):
    O = oracle_lib
    w = make_workload(get_config(key))
    c = w.cfg
    r = O.run_step(w, SCALE)
    for seed in range(3):
        kp2, vp2, t2 = _relabel(r["k_pool"], r["v_pool"], w.tables, seed)
        out2 = O.attention(w.q, kp2, vp2, t2, w.lengths, c.num_kv_heads, c.block_size,
                           w.num_blocks, SCALE, c.dtype)
        assert np.array_equal(out2, r["out"])


def test_single_token_returns_its_value(oracle_lib):
    cfg = tiny_cfg(lengths=(1, 1, 1, 1))
    w = make_workload(cfg, lengths=(1, 1, 1, 1))
    out = oracle_lib.run_step(w, SCALE)["out"]
    v = brute.widen(w.v_new, "fp16")
    G = cfg.num_q_heads // cfg.num_kv_heads
    for h in range(cfg.num_q_heads):
        assert np.array_equal(out[:, h], v[:, h // G])


@pytest.mark.parametrize("key", ["c1a", "c1b"])
def test_zero_scale_is_mean_of_exactly_n_values(oracle_lib, key):
    w = make_workload(get_config(key))
    c = w.cfg
    out = oracle_lib.run_step(w, 0.0)["out"]
    G = c.group
    for s in range(c.num_seqs):
        _, V = w.logical_kv(s)
        V = brute.widen(V, c.dtype)
        n = int(w.lengths[s])
        for h in range(c.num_q_heads):
            col = V[:, h // G, :]
            exp = np.array([math.fsum(col[:, d]) / n for d in range(c.head_dim)])
            assert np.abs(out[s, h] - exp).max() <= 1e-13


def test_dominant_key_selects_its_value(oracle_lib):
    cfg = tiny_cfg(lengths=(40, 23), hq=2, hkv=2)
    w = make_workload(cfg, lengths=(40, 23))
    c = w.cfg
    # make the key at logical position 17 of each sequence 8x that sequence's query
    # of head h (same KV head index since G = 1); 8x is exact in fp16
    target = 17
    for s in range(c.num_seqs):
        a = int(w.seg_cu[s]) + target
        for h in range(c.num_kv_heads):
            q = w.q[s, h].view(np.float16).astype(np.float32) * 8
            w.k_src[a, h] = q.astype(np.float16).view(np.uint16)
    out = oracle_lib.run_step(w, SCALE)["out"]
    for s in range(c.num_seqs):
        _, V = w.logical_kv(s)
        V = brute.widen(V, c.dtype)
        for h in range(c.num_q_heads):
            assert np.abs(out[s, h] - V[target, h]).max() <= 1e-12


def test_gqa_equals_mha_with_repeated_heads(oracle_lib):
    O = oracle_lib
    w = make_workload(get_config("c1a"))
    c = w.cfg
    r = O.run_step(w, SCALE)
    kp2 = np.ascontiguousarray(np.repeat(r["k_pool"], c.group, axis=1))
    vp2 = np.ascontiguousarray(np.repeat(r["v_pool"], c.group, axis=1))
    out2 = O.attention(w.q, kp2, vp2, w.tables, w.lengths, c.num_q_heads, c.block_size,
                       w.num_blocks, SCALE, c.dtype)
    assert np.array_equal(out2, r["out"])


def test_prefix_sharing_equals_private_copies(oracle_lib):
    """Sequences that share prefix blocks give the same output as the same data
    with the prefix blocks duplicated privately per sequence."""
    O = oracle_lib
    base = get_config("c5")
    cfg = dataclasses.replace(base, key="c5tiny", num_seqs=5, prefix_tokens=32,
                              max_blocks_per_seq=12)
    w = make_workload(cfg)
    c = w.cfg
    r = O.run_step(w, SCALE)
    npre = c.prefix_tokens // c.block_size
    shared = w.tables[0, :npre]
    assert (w.tables[:, :npre] == shared).all()
    NB2 = w.num_blocks + c.num_seqs * npre
    kp2 = np.full((NB2,) + r["k_pool"].shape[1:], NAN_BITS["fp16"], np.uint16)
    vp2 = kp2.copy()
    kp2[:w.num_blocks] = r["k_pool"]
    vp2[:w.num_blocks] = r["v_pool"]
    t2 = w.tables.copy()
    nxt = w.num_blocks
    for s in range(c.num_seqs):
        for j in range(npre):
            kp2[nxt] = r["k_pool"][shared[j]]
            vp2[nxt] = r["v_pool"][shared[j]]
            t2[s, j] = nxt
            nxt += 1
    out2 = O.attention(w.q, kp2, vp2, t2, w.lengths, c.num_kv_heads, c.block_size, NB2, SCALE,
                       c.dtype)
    assert np.array_equal(out2, r["out"])


# ---------------------------------------------------------------------------
# partitions and the log-sum-exp merge
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ["c1a", "c1b"])
@pytest.mark.parametrize("mult", [1, 2, 3, 4])
def test_partials_merge_equals_direct(oracle_lib, key, mult):
    O = oracle_lib
    w = make_workload(get_config(key))
    c = w.cfg
    P = mult * c.block_size
    MP = -(-c.max_context // P)
    r = O.run_step(w, SCALE, partition_size=P, max_partitions=MP)
    assert np.abs(r["merged"] - r["out"]).max() <= 1e-12


def test_partials_match_brute_force_per_range(oracle_lib):
    """Each partition's output and log-sum-exp equal brute force over that token
    range of the logical arrays."""
    O = oracle_lib
    w = make_workload(get_config("c1b"))
    c = w.cfg
    P, MP = 16, 5
    r = O.run_step(w, SCALE, partition_size=P, max_partitions=MP)
    q = brute.widen(w.q, c.dtype)
    for s in range(c.num_seqs):
        K, V = (brute.widen(x, c.dtype) for x in w.logical_kv(s))
        n = int(w.lengths[s])
        for h in range(c.num_q_heads):
            g = h // c.group
            for p in range(-(-n // P)):
                a, b = p * P, min(n, (p + 1) * P)
                z = SCALE * (K[a:b, g] @ q[s, h])
                lse = z.max() + math.log(math.fsum(np.exp(z - z.max())))
                assert abs(r["part_lse"][s, h, p] - lse) <= 1e-12
                o = brute.attention_one(q[s, h], K[a:b, g], V[a:b, g], SCALE)
                assert np.abs(r["part_o"][s, h, p] - o).max() <= 1e-12
            assert np.isnan(r["part_lse"][s, h, -(-n // P):]).all()  # untouched


def test_merge_of_equal_lse_is_mean(oracle_lib):
    rng = np.random.default_rng(7)
    S, H, MP, D, P = 2, 3, 4, 8, 16
    po = rng.standard_normal((S, H, MP, D))
    pl = np.full((S, H, MP), 1.75)
    lens = np.array([64, 33], np.int32)  # 4 and 3 partitions
    out = oracle_lib.merge(po, pl, lens, P)
    assert np.abs(out[0] - po[0].mean(axis=1)).max() <= 1e-15
    assert np.abs(out[1] - po[1, :, :3].mean(axis=1)).max() <= 1e-15


def test_merge_weights_follow_lse(oracle_lib):
    # two partitions whose lse differ by ln 3 weigh 3:1
    po = np.zeros((1, 1, 2, 2))
    po[0, 0, 0] = [1.0, 0.0]
    po[0, 0, 1] = [0.0, 1.0]
    pl = np.array([[[math.log(3.0) + 0.5, 0.5]]])
    out = oracle_lib.merge(po, pl, np.array([20], np.int32), 16)
    assert np.abs(out[0, 0] - [0.75, 0.25]).max() <= 1e-15


def test_empty_sequence_gives_zeros(oracle_lib):
    O = oracle_lib
    kp = np.full((4, 1, 16, 8), 0x7E00, np.uint16)
    out = O.attention(np.ones((1, 1, 8), np.uint16), kp, kp.copy(),
                      np.full((1, 2), -1, np.int32), np.array([0], np.int32), 1, 16, 4, SCALE,
                      "fp16")
    assert (out == 0).all()
    m = O.merge(np.full((1, 1, 2, 8), np.nan), np.full((1, 1, 2), np.nan),
                np.array([0], np.int32), 16)
    assert (m == 0).all()
