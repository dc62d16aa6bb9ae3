"""GPU parity of paged_attention_decode_slotted (slotted segment lists) with the
fp64 oracle, through the C ABI: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|.  Pools
are built on each side by its own code from the same runs; positions no segment
covers hold the NaN sentinel, so a read outside a sequence's slots would show."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import get_config, make_workload  # noqa: E402
from workloads.gen import NAN_BITS  # noqa: E402
from workloads.slotted import make_slotted_workload, pack  # noqa: E402
from oracle import oracle as O  # noqa: E402
from gpu_harness import bits_of, i32, i64, scale_for, to_dev, tol_ok, widen_out  # noqa: E402
import paged_kv_cache_09_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")
TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _pools_both(runs, NB, Hkv, B, dtype):
    kr, vr, cu, st, tb = runs
    kp, vp = O.new_pools(NB, Hkv, B, 128, NAN_BITS[dtype])
    O.append_tokens(kp, vp, kr, vr, cu, st, tb, B, NB)
    gk = torch.empty((NB, Hkv, B, 128), dtype=TDT[dtype], device=DEV)
    sentinel = int(np.array([NAN_BITS[dtype]], np.uint16).view(np.int16)[0])
    gk.view(torch.int16).fill_(sentinel)
    gv = gk.clone()
    pkv.paged_kv_append_tokens(gk, gv, to_dev(kr, dtype, DEV), to_dev(vr, dtype, DEV),
                               i64(cu, DEV), i32(st, DEV), i32(tb, DEV))
    return kp, vp, gk, gv


@pytest.fixture(params=["tiles", "per_sequence"])
def mode(request, monkeypatch):
    """Both kernels: tiles of sequences (PKV_SLOTTED_TILES=1: taken whenever a
    tile's sub-tile list fits in LDS) and one work-group per sequence
    (PKV_SLOTTED_TILES=0)."""
    monkeypatch.setenv("PKV_SLOTTED_TILES", "1" if request.param == "tiles" else "0")
    return request.param


def tile_list_fits(Hq, Hkv, B, max_segments):
    """The header's rule for the tiled kernel: 2 * floor(16 / G) sequences per
    tile, each with up to max_segments * ceil(B / 16) sub-tiles, within 1,024."""
    return 2 * (16 // (Hq // Hkv)) * max_segments * (-(-B // 16)) <= 1024


def _gpu_split(q, gk, gv, segs, nsegs, dtype, scale, P, B):
    """paged_attention_decode_slotted_split with a NaN-filled workspace; returns the
    widened output and the arrival counters."""
    S, Hq, _ = q.shape
    Hkv = gk.shape[1]
    mp = -(-segs.shape[1] * B // P)
    out = torch.empty((S, Hq, 128), dtype=TDT[dtype], device=DEV)
    out.view(torch.int16).fill_(0x5555)
    po = torch.full((S, Hq, mp, 128), float("nan"), dtype=torch.float32, device=DEV)
    pl = torch.full((S, Hq, mp), float("nan"), dtype=torch.float32, device=DEV)
    ctr = torch.zeros((S, Hkv), dtype=torch.int32, device=DEV)
    pkv.paged_attention_decode_slotted_split(out, to_dev(q, dtype, DEV), gk, gv, i32(segs, DEV),
                                             i32(nsegs, DEV), P, po, pl, ctr, scale=scale)
    torch.cuda.synchronize()
    return widen_out(out), ctr


def _gpu(q, gk, gv, segs, nsegs, dtype, scale):
    S, Hq, _ = q.shape
    out = torch.empty((S, Hq, 128), dtype=TDT[dtype], device=DEV)
    out.view(torch.int16).fill_(0x5555)
    pkv.paged_attention_decode_slotted(out, to_dev(q, dtype, DEV), gk, gv, i32(segs, DEV),
                                       i32(nsegs, DEV), scale=scale)
    torch.cuda.synchronize()
    return widen_out(out)


def test_radix_batch_matches_oracle(mode):
    cfg = get_config("c5")
    w = make_slotted_workload(cfg)
    print(f"[gpu] slotted radix batch ({mode}) S={len(w.paths)} NB={w.num_blocks} "
          f"max_segments={w.segments.shape[1]}", flush=True)
    kp, vp, gk, gv = _pools_both(w.runs(), w.num_blocks, cfg.num_kv_heads, cfg.block_size,
                                 cfg.dtype)
    scale = scale_for(128)
    ref = O.attention_slotted(w.q, kp, vp, w.segments, w.num_segments, cfg.num_kv_heads,
                              cfg.block_size, w.num_blocks, scale, cfg.dtype)
    got = _gpu(w.q, gk, gv, w.segments, w.num_segments, cfg.dtype, scale)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)


def _tree_order(w):
    """The radix batch with its sequences sorted by node path (depth-first order):
    a tile's consecutive sequences share the root, a level-1 node and, in runs of
    four, level-2 nodes."""
    import dataclasses
    perm = sorted(range(len(w.paths)), key=lambda t: w.paths[t])
    return dataclasses.replace(w, paths=[w.paths[t] for t in perm], q=w.q[perm],
                               segments=w.segments[perm], num_segments=w.num_segments[perm],
                               k_new=w.k_new[perm], v_new=w.v_new[perm])


def test_radix_batch_tree_order_matches_oracle(mode):
    """The radix batch in tree order: runs of members within a tile share nodes
    below the common path, read once per run by the tiled kernel."""
    cfg = get_config("c5")
    w = _tree_order(make_slotted_workload(cfg))
    print(f"[gpu] slotted radix batch in tree order ({mode})", flush=True)
    kp, vp, gk, gv = _pools_both(w.runs(), w.num_blocks, cfg.num_kv_heads, cfg.block_size,
                                 cfg.dtype)
    scale = scale_for(128)
    ref = O.attention_slotted(w.q, kp, vp, w.segments, w.num_segments, cfg.num_kv_heads,
                              cfg.block_size, w.num_blocks, scale, cfg.dtype)
    got = _gpu(w.q, gk, gv, w.segments, w.num_segments, cfg.dtype, scale)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)
    slots = _check_append(w.q, kp, vp, gk, gv, w.k_new, w.v_new, w.segments, w.num_segments,
                          cfg.num_kv_heads, cfg.block_size, w.num_blocks, cfg.dtype)
    assert (slots >= 0).all()


def _tree_case(seed, S, Hq, Hkv, B, dtype, fanout, depth, node_len_hi):
    """A random tree of prompt nodes (each internal node has 1..fanout children,
    some nodes empty) whose leaves, listed depth-first, are the sequences: runs of
    consecutive sequences share nodes at every depth, cut where the tree
    branches.  Paths are truncated at random for some sequences, and a few
    sequences repeat their neighbour's path with their own leaf."""
    rng = np.random.default_rng(seed)
    lens, paths = [], []

    def node(n):
        lens.append(n)
        return len(lens) - 1

    def grow(prefix, d):
        if len(paths) >= S:
            return
        if d == depth:
            paths.append(prefix + [node(int(rng.integers(1, node_len_hi + 1)))])
            return
        for _ in range(int(rng.integers(1, fanout + 1))):
            ln = int(rng.integers(0, node_len_hi + 1)) if rng.random() < 0.9 else 0
            grow(prefix + [node(ln)], d + 1)

    root = node(int(rng.integers(1, 4 * node_len_hi)))
    while len(paths) < S:
        grow([root], 1)
    for t in range(S):
        if rng.random() < 0.1:  # a shorter path: the leaf hangs higher up
            cut = int(rng.integers(1, len(paths[t])))
            paths[t] = paths[t][:cut] + [paths[t][-1]]
    free = [int(x) for x in rng.permutation(20 * len(lens) + 16)]
    node_segs = pack([max(n, 1) for n in lens], B, free)
    node_segs = [[(sg[0][0], sg[0][1], 0)] if lens[i] == 0 else sg for i, sg in enumerate(node_segs)]
    NB = max(x[0] for sg in node_segs for x in sg) + 1

    def draw(*sh):
        x = rng.standard_normal(sh).astype(np.float32)
        if dtype == "fp16":
            return x.astype(np.float16).view(np.uint16)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    node_k = [draw(n, Hkv, 128) for n in lens]
    node_v = [draw(n, Hkv, 128) for n in lens]
    MS = max(sum(len(node_segs[i]) for i in p) for p in paths)
    segs = np.zeros((S, MS, 3), np.int32)
    nsegs = np.zeros(S, np.int32)
    for t, p in enumerate(paths):
        flat = [x for i in p for x in node_segs[i]]
        segs[t, :len(flat)] = flat
        nsegs[t] = len(flat)
    rk, rv, st, tb, cu = [], [], [], [], [0]
    for sg, k, v in zip(node_segs, node_k, node_v):
        r = 0
        for blk, off, ln in sg:
            rk.append(k[r:r + ln]); rv.append(v[r:r + ln])
            st.append(off); tb.append([blk]); cu.append(cu[-1] + ln)
            r += ln
    runs = (np.concatenate(rk), np.concatenate(rv), np.array(cu, np.int64),
            np.array(st, np.int32), np.array(tb, np.int32))
    return dict(NB=NB, segs=segs, nsegs=nsegs, runs=runs, q=draw(S, Hq, 128))


TREE_CASES = [
    # (seed, S, Hq, Hkv, B, dtype, fanout, depth, max node length)
    (41, 40, 32, 8, 16, "fp16", 3, 3, 20),    # G 4: 8 per tile
    (42, 70, 16, 16, 16, "bf16", 4, 3, 12),   # G 1: 32 per tile, runs across the halves
    (43, 30, 12, 2, 16, "fp16", 2, 4, 10),    # G 6: 4 per tile
    (44, 50, 24, 8, 32, "bf16", 3, 3, 40),    # G 3, blocks of 32
    (45, 20, 32, 2, 64, "fp16", 2, 2, 90),    # G 16: 2 per tile
]


@pytest.mark.parametrize("case", TREE_CASES, ids=[f"seed{c[0]}" for c in TREE_CASES])
def test_random_trees_in_tree_order(case, mode):
    seed, S, Hq, Hkv, B, dtype, fan, depth, hi = case
    c = _tree_case(seed, S, Hq, Hkv, B, dtype, fan, depth, hi)
    print(f"[gpu] slotted tree ({mode}) seed={seed} S={S} Hq={Hq} Hkv={Hkv} B={B} {dtype} "
          f"max_segments={c['segs'].shape[1]}", flush=True)
    assert mode != "tiles" or tile_list_fits(Hq, Hkv, B, c["segs"].shape[1])
    kp, vp, gk, gv = _pools_both(c["runs"], c["NB"], Hkv, B, dtype)
    scale = scale_for(128)
    ref = O.attention_slotted(c["q"], kp, vp, c["segs"], c["nsegs"], Hkv, B, c["NB"], scale,
                              dtype)
    got = _gpu(c["q"], gk, gv, c["segs"], c["nsegs"], dtype, scale)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)


def _node_case(seed, S, Hq, Hkv, B, dtype, node_len_hi, nodes_per_path, trunks=False,
               leaves=False):
    """Random tree-less node sets: every sequence walks its own random list of
    nodes (shared ones included), some paths empty, some nodes of length 0.
    With trunks, runs of consecutive sequences first walk a common random list
    of nodes (cut short for some), as the paths of a radix tree do.  With
    leaves, every sequence but the empty one also ends in a private node of its
    own (every third one followed by a zero-length node), whose last row is the
    sequence's position n-1, and the case holds new K/V rows for the append."""
    rng = np.random.default_rng(seed)
    lrng = np.random.default_rng(seed + 1000)  # leaves and new rows: the rest is unchanged
    nn = max(3 * S + 8, 2 * nodes_per_path)
    lens = [int(x) for x in rng.integers(0, node_len_hi + 1, size=nn)]
    free = [int(x) for x in rng.permutation(10 * nn + 16)]
    if leaves:
        lens += [int(x) for x in lrng.integers(1, node_len_hi + 2, size=S)]
        free += list(range(10 * nn + 16, 10 * nn + 16 + S * (node_len_hi // B + 2)))
    node_segs = pack([max(n, 1) for n in lens], B, free)
    # zero-length nodes keep a (block, offset, 0) segment
    node_segs = [[(segs[0][0], segs[0][1], 0)] if lens[i] == 0 else segs
                 for i, segs in enumerate(node_segs)]
    NB = max(x[0] for segs in node_segs for x in segs) + 1

    def draw(*sh, gen=rng):
        x = gen.standard_normal(sh).astype(np.float32)
        if dtype == "fp16":
            return x.astype(np.float16).view(np.uint16)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    node_k = [draw(n, Hkv, 128) for n in lens[:nn]]
    node_v = [draw(n, Hkv, 128) for n in lens[:nn]]
    paths = [[int(x) for x in rng.choice(nn, size=rng.integers(0, nodes_per_path + 1),
                                         replace=False)] for _ in range(S)]
    if trunks:
        s = 0
        while s < S:
            run = int(rng.integers(8, 80))
            trunk = [int(x) for x in rng.choice(nn, size=rng.integers(0, nodes_per_path + 1),
                                                replace=False)]
            for t in range(s, min(S, s + run)):
                cut = len(trunk) if rng.random() < 0.97 else int(rng.integers(0, len(trunk) + 1))
                own = [x for x in paths[t] if x not in trunk[:cut]][:int(rng.integers(0, 4))]
                paths[t] = trunk[:cut] + own
            s += run
    paths[-1 if trunks else 0] = []
    extra = {}
    if leaves:
        node_k += [draw(n, Hkv, 128, gen=lrng) for n in lens[nn:]]
        node_v += [draw(n, Hkv, 128, gen=lrng) for n in lens[nn:]]
        zero = [i for i in range(nn) if lens[i] == 0]
        for t in range(S):
            if t != (S - 1 if trunks else 0):
                paths[t] = paths[t] + [nn + t] + (zero[:1] if t % 3 == 0 else [])
        extra = dict(k_new=draw(S, Hkv, 128, gen=lrng), v_new=draw(S, Hkv, 128, gen=lrng))
    MS = max(1, max(sum(len(node_segs[i]) for i in p) for p in paths))
    segs = np.zeros((S, MS, 3), np.int32)
    nsegs = np.zeros(S, np.int32)
    for s, p in enumerate(paths):
        flat = [x for i in p for x in node_segs[i]]
        if flat:
            segs[s, :len(flat)] = flat
        nsegs[s] = len(flat)
    rk, rv, st, tb, cu = [], [], [], [], [0]
    for segs_i, k, v in zip(node_segs, node_k, node_v):
        r = 0
        for blk, off, ln in segs_i:
            rk.append(k[r:r + ln]); rv.append(v[r:r + ln])
            st.append(off); tb.append([blk]); cu.append(cu[-1] + ln)
            r += ln
    runs = (np.concatenate(rk), np.concatenate(rv), np.array(cu, np.int64),
            np.array(st, np.int32), np.array(tb, np.int32))
    return dict(NB=NB, segs=segs, nsegs=nsegs, runs=runs, q=draw(S, Hq, 128), **extra)


NODE_CASES = [
    # (seed, S, Hq, Hkv, B, dtype, max node length, max nodes per path)
    (1, 6, 12, 2, 16, "fp16", 20, 6),        # G 6
    (2, 5, 32, 8, 16, "bf16", 40, 8),        # G 4
    (3, 4, 16, 16, 32, "fp16", 70, 5),       # G 1 on the matrix-core path
    (4, 3, 32, 2, 64, "bf16", 150, 4),       # G 16
    (5, 4, 12, 4, 128, "fp16", 300, 3),      # G 3
    (6, 3, 16, 8, 256, "bf16", 250, 4),      # G 2, the largest block (a full tile list)
    (7, 3, 12, 2, 16, "fp16", 3, 150),       # ~150 short segments: three rounds of 64
]


# runs of sequences sharing leading nodes: the tiles' common sub-tiles
TRUNK_CASES = [
    # (seed, S, Hq, Hkv, B, dtype, max node length, max nodes per path)
    (11, 37, 32, 8, 16, "fp16", 40, 10),     # G 4: 8 per tile, a partial last tile
    (12, 45, 16, 16, 16, "bf16", 30, 5),     # G 1: 32 per tile, then a partial tile
    (13, 9, 12, 2, 16, "fp16", 33, 8),       # G 6: 4 per tile (12 of 16 columns per half)
    (14, 7, 32, 2, 64, "bf16", 150, 4),      # G 16: 2 per tile
    (15, 19, 24, 8, 16, "fp16", 17, 40),     # G 3, many short segments
    (22, 70, 8, 8, 16, "fp16", 30, 6),       # G 1: two full tiles of 32 with common nodes
    (23, 40, 16, 8, 16, "bf16", 25, 8),      # G 2: 16 per tile
    (33, 7, 32, 2, 256, "fp16", 600, 3),     # G 16 at the largest block: 16 sub-tiles a segment
]


@pytest.mark.parametrize("case", NODE_CASES + TRUNK_CASES,
                         ids=[f"seed{c[0]}" for c in NODE_CASES + TRUNK_CASES])
def test_random_node_lists(case, mode):
    seed, S, Hq, Hkv, B, dtype, hi, per = case
    c = _node_case(seed, S, Hq, Hkv, B, dtype, hi, per, trunks=seed >= 11)
    print(f"[gpu] slotted ({mode}) seed={seed} S={S} Hq={Hq} Hkv={Hkv} B={B} {dtype} "
          f"max_segments={c['segs'].shape[1]}", flush=True)
    # every case labelled "tiles" really runs the tiled kernel
    assert mode != "tiles" or tile_list_fits(Hq, Hkv, B, c["segs"].shape[1])
    kp, vp, gk, gv = _pools_both(c["runs"], c["NB"], Hkv, B, dtype)
    scale = scale_for(128)
    ref = O.attention_slotted(c["q"], kp, vp, c["segs"], c["nsegs"], Hkv, B, c["NB"], scale,
                              dtype)
    got = _gpu(c["q"], gk, gv, c["segs"], c["nsegs"], dtype, scale)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)
    assert (got[-1 if seed >= 11 else 0] == 0).all()  # the empty sequence
    # split mode (per-sequence kernel, partitions of 32 positions merged in the
    # launch): segments straddle partition boundaries
    got2, ctr = _gpu_split(c["q"], gk, gv, c["segs"], c["nsegs"], dtype, scale, 32, B)
    ok, err, nbad = tol_ok(got2, ref)
    assert ok, ("split", err, nbad)
    assert not bool(ctr.any())


def test_segment_counts_are_clamped_to_the_row(mode):
    """Without the debug check, a count above max_segments reads no further than
    the sequence's own row (as if it were max_segments), and a negative count
    reads nothing."""
    seed, S, Hq, Hkv, B, dtype, hi, per = TRUNK_CASES[0]
    c = _node_case(seed, S, Hq, Hkv, B, dtype, hi, per, trunks=True)
    MS = c["segs"].shape[1]
    print(f"[gpu] slotted ({mode}) clamped counts S={S} max_segments={MS}", flush=True)
    kp, vp, gk, gv = _pools_both(c["runs"], c["NB"], Hkv, B, dtype)
    scale = scale_for(128)
    over = c["nsegs"].copy()
    over[1::3] = MS + 1000
    over[2::5] = -7
    clamped = np.clip(over, 0, MS).astype(np.int32)
    got = _gpu(c["q"], gk, gv, c["segs"], over, dtype, scale)
    ref = _gpu(c["q"], gk, gv, c["segs"], clamped, dtype, scale)
    assert (got == ref).all()
    assert (got[2::5] == 0).all()


_table_cache = {}


def _tables_as_segments(key):
    """A workload's block tables written as whole-block segments (plus the partly
    filled last block), with the oracle's result (computed once per module)."""
    if key not in _table_cache:
        w = make_workload(get_config(key))
        c = w.cfg
        r = O.run_step(w, scale_for(c.head_dim))
        B = c.block_size
        nb = -(-w.lengths.astype(np.int64) // B)
        segs = np.zeros((c.num_seqs, int(nb.max()), 3), np.int32)
        for s in range(c.num_seqs):
            for j in range(nb[s]):
                segs[s, j] = (w.tables[s, j], 0, min(B, int(w.lengths[s]) - j * B))
        _table_cache[key] = (w, r, segs, nb.astype(np.int32))
    return _table_cache[key]


# c4's tile list (8 sequences x 128 segments x 8 sub-tiles) does not fit: one
# work-group per sequence only
@pytest.mark.parametrize("key,mode", [("c1a", "tiles"), ("c1a", "per_sequence"),
                                      ("c2", "tiles"), ("c2", "per_sequence"),
                                      ("c4", "per_sequence")], indirect=["mode"])
def test_block_tables_as_segments(key, mode):
    """A block table as segments gives the oracle's ordinary attention."""
    w, r, segs, nsegs = _tables_as_segments(key)
    c = w.cfg
    print(f"[gpu] slotted from tables {key} ({mode})", flush=True)
    assert mode != "tiles" or tile_list_fits(c.num_q_heads, c.num_kv_heads, c.block_size,
                                             segs.shape[1])
    gk, gv = to_dev(r["k_pool"], c.dtype, DEV), to_dev(r["v_pool"], c.dtype, DEV)
    got = _gpu(w.q, gk, gv, segs, nsegs, c.dtype, scale_for(c.head_dim))
    ok, err, nbad = tol_ok(got, r["out"])
    assert ok, (err, nbad)


@pytest.mark.parametrize("key,P", [("c1a", 32), ("c2", 256), ("c2", 512), ("c4", 1024),
                                   ("c4", 2048)])
def test_block_tables_as_segments_split(key, P):
    """Split mode on block tables written as segments: the oracle's attention, the
    counters back at zero, and a second call on them giving the same bits."""
    w, r, segs, nsegs = _tables_as_segments(key)
    c = w.cfg
    print(f"[gpu] slotted split from tables {key} P={P}", flush=True)
    gk, gv = to_dev(r["k_pool"], c.dtype, DEV), to_dev(r["v_pool"], c.dtype, DEV)
    got, ctr = _gpu_split(w.q, gk, gv, segs, nsegs, c.dtype, scale_for(c.head_dim), P,
                          c.block_size)
    ok, err, nbad = tol_ok(got, r["out"])
    assert ok, (err, nbad)
    assert not bool(ctr.any())
    got2, _ = _gpu_split(w.q, gk, gv, segs, nsegs, c.dtype, scale_for(c.head_dim), P,
                         c.block_size)
    assert np.array_equal(got, got2)


def _gpu_append(q, gk, gv, k_new, v_new, segs, nsegs, dtype, scale):
    """paged_attention_append_decode_slotted on the device pools (written in
    place); returns the widened output and the slot ids."""
    S, Hq, _ = q.shape
    out = torch.empty((S, Hq, 128), dtype=TDT[dtype], device=DEV)
    out.view(torch.int16).fill_(0x5555)
    slots = torch.full((S,), -2, dtype=torch.int64, device=DEV)
    pkv.paged_attention_append_decode_slotted(
        out, to_dev(q, dtype, DEV), gk, gv, to_dev(k_new, dtype, DEV), to_dev(v_new, dtype, DEV),
        i32(segs, DEV), i32(nsegs, DEV), slot_out=slots, scale=scale)
    torch.cuda.synchronize()
    return widen_out(out), slots.cpu().numpy()


def _check_append(q, kp, vp, gk, gv, k_new, v_new, segs, nsegs, Hkv, B, NB, dtype):
    """The fused call against the oracle's append followed by its attention: the
    pools bit for bit, the slot ids exactly, the output within the tolerance;
    then a plain slotted decode over the written pools gives the same output bit
    for bit (the rows were in place before any wave read them)."""
    scale = scale_for(128)
    ref_slots = O.append_slotted(kp, vp, k_new, v_new, segs, nsegs, B, NB)
    ref = O.attention_slotted(q, kp, vp, segs, nsegs, Hkv, B, NB, scale, dtype)
    got, slots = _gpu_append(q, gk, gv, k_new, v_new, segs, nsegs, dtype, scale)
    assert np.array_equal(slots, ref_slots)
    assert np.array_equal(bits_of(gk), kp) and np.array_equal(bits_of(gv), vp)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)
    assert np.array_equal(_gpu(q, gk, gv, segs, nsegs, dtype, scale), got)
    return slots


def test_append_radix_batch_matches_oracle(mode):
    """The radix-tree batch with each sequence's new token written to the last
    row of its private leaf (the lengths count it) and attended in one launch."""
    cfg = get_config("c5")
    w = make_slotted_workload(cfg)
    S, Hkv = len(w.paths), cfg.num_kv_heads
    print(f"[gpu] slotted append radix batch ({mode}) S={S} NB={w.num_blocks}", flush=True)
    kp, vp, gk, gv = _pools_both(w.runs(), w.num_blocks, Hkv, cfg.block_size, cfg.dtype)
    slots = _check_append(w.q, kp, vp, gk, gv, w.k_new, w.v_new, w.segments, w.num_segments,
                          Hkv, cfg.block_size, w.num_blocks, cfg.dtype)
    assert (slots >= 0).all() and len(set(slots.tolist())) == S


APPEND_CASES = [NODE_CASES[i] for i in (0, 2, 3, 4, 6)] + [TRUNK_CASES[i] for i in (0, 1, 5, 7)]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[f"seed{c[0]}" for c in APPEND_CASES])
def test_append_random_node_lists(case, mode):
    """Random node lists, each ending in a private leaf (some followed by an empty
    segment, one sequence empty: slot -1, nothing written)."""
    seed, S, Hq, Hkv, B, dtype, hi, per = case
    c = _node_case(seed, S, Hq, Hkv, B, dtype, hi, per, trunks=seed >= 11, leaves=True)
    print(f"[gpu] slotted append ({mode}) seed={seed} S={S} Hq={Hq} Hkv={Hkv} B={B} {dtype} "
          f"max_segments={c['segs'].shape[1]}", flush=True)
    assert mode != "tiles" or tile_list_fits(Hq, Hkv, B, c["segs"].shape[1])
    kp, vp, gk, gv = _pools_both(c["runs"], c["NB"], Hkv, B, dtype)
    slots = _check_append(c["q"], kp, vp, gk, gv, c["k_new"], c["v_new"], c["segs"],
                          c["nsegs"], Hkv, B, c["NB"], dtype)
    assert slots[-1 if seed >= 11 else 0] == -1


def test_long_leaves_split():
    """A radix batch at the long-context shapes (32 query / 8 KV heads, blocks of
    128, bf16) whose sequences share a 512-token root and short slotted nodes and
    then own leaves of 16,000-20,000 tokens: split decode at 2,048 positions per
    partition against the oracle."""
    rng = np.random.default_rng(31)
    S, Hq, Hkv, B, dt = 8, 32, 8, 128, "bf16"
    lens = [512] + [int(x) for x in rng.integers(3, 40, size=4)] + \
        [int(x) for x in rng.integers(16000, 20001, size=S)]
    need = sum(-(-n // B) for n in lens)
    NB = need + 9
    free = [int(x) for x in rng.permutation(NB)]
    node_segs = pack(lens, B, free)

    def draw(*sh):
        x = rng.standard_normal(sh).astype(np.float32)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    node_k = [draw(n, Hkv, 128) for n in lens]
    node_v = [draw(n, Hkv, 128) for n in lens]
    paths = [[0, 1 + s % 4, 5 + s] for s in range(S)]
    MS = max(sum(len(node_segs[i]) for i in p) for p in paths)
    segs = np.zeros((S, MS, 3), np.int32)
    nsegs = np.zeros(S, np.int32)
    for s, p in enumerate(paths):
        flat = [x for i in p for x in node_segs[i]]
        segs[s, :len(flat)] = flat
        nsegs[s] = len(flat)
    rk, rv, st, tb, cu = [], [], [], [], [0]
    for segs_i, k, v in zip(node_segs, node_k, node_v):
        r = 0
        for blk, off, ln in segs_i:
            rk.append(k[r:r + ln]); rv.append(v[r:r + ln])
            st.append(off); tb.append([blk]); cu.append(cu[-1] + ln)
            r += ln
    runs = (np.concatenate(rk), np.concatenate(rv), np.array(cu, np.int64),
            np.array(st, np.int32), np.array(tb, np.int32))
    print(f"[gpu] slotted split, long leaves: S={S} NB={NB} max_segments={MS}", flush=True)
    kp, vp, gk, gv = _pools_both(runs, NB, Hkv, B, dt)
    q = draw(S, Hq, 128)
    scale = scale_for(128)
    ref = O.attention_slotted(q, kp, vp, segs, nsegs, Hkv, B, NB, scale, dt)
    got, ctr = _gpu_split(q, gk, gv, segs, nsegs, dt, scale, 2048, B)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)
    assert not bool(ctr.any())


def test_slotted_debug_check_rejects_bad_segments(monkeypatch):
    gk = torch.zeros((8, 2, 16, 128), dtype=torch.float16, device=DEV)
    q = np.zeros((2, 4, 128), np.uint16)
    monkeypatch.setenv("PKV_DEBUG_CHECK", "1")
    bad = [
        [[[0, 12, 5]], [[1, 0, 3]]],    # slot runs past its block
        [[[9, 0, 5]], [[1, 0, 3]]],     # block outside the pool
        [[[0, 0, -1]], [[1, 0, 3]]],    # negative length
    ]
    for segs in bad:
        with pytest.raises(pkv.PagedKVError) as ei:
            _gpu(q, gk, gk, np.array(segs, np.int32), np.array([1, 1], np.int32), "fp16", 0.1)
        assert ei.value.status == -5
    with pytest.raises(pkv.PagedKVError) as ei:  # more segments than the row holds
        _gpu(q, gk, gk, np.array([[[0, 0, 1]], [[1, 0, 3]]], np.int32),
             np.array([2, 1], np.int32), "fp16", 0.1)
    assert ei.value.status == -5


def test_append_debug_check_rejects_bad_segments_and_writes_nothing(monkeypatch):
    """The fused slotted append validates the segments before any kernel runs:
    a rejected call leaves the pools and the slot ids untouched."""
    gk = torch.zeros((8, 2, 16, 128), dtype=torch.float16, device=DEV)
    gv = torch.zeros_like(gk)
    q = np.zeros((2, 4, 128), np.uint16)
    new = np.full((2, 2, 128), 0x3C00, np.uint16)  # 1.0 in fp16
    monkeypatch.setenv("PKV_DEBUG_CHECK", "1")
    print("[gpu] slotted append debug rejections", flush=True)
    for segs, ns in (([[[0, 12, 5]], [[1, 0, 3]]], [1, 1]),   # slot past its block
                     ([[[9, 0, 5]], [[1, 0, 3]]], [1, 1]),    # block outside the pool
                     ([[[0, 0, 1]], [[1, 0, 3]]], [2, 1])):   # count above the row
        slots = torch.full((2,), -7, dtype=torch.int64, device=DEV)
        out = torch.empty((2, 4, 128), dtype=torch.float16, device=DEV)
        with pytest.raises(pkv.PagedKVError) as ei:
            pkv.paged_attention_append_decode_slotted(
                out, to_dev(q, "fp16", DEV), gk, gv, to_dev(new, "fp16", DEV),
                to_dev(new, "fp16", DEV), i32(np.array(segs, np.int32), DEV),
                i32(np.array(ns, np.int32), DEV), slot_out=slots, scale=0.1)
        assert ei.value.status == -5
        torch.cuda.synchronize()
        assert not bool(gk.any()) and not bool(gv.any())
        assert (slots.cpu().numpy() == -7).all()


def test_append_single_row_segments_and_block_edges(mode):
    """Segments of one row, and new rows landing on a block's first and last row
    (offsets 0 and B - 1) at every block size, against the oracle."""
    for B in (16, 32, 64, 128, 256):
        Hq, Hkv, S = 8, 2, 6
        rng = np.random.default_rng(500 + B)
        # sequence t: a shared one-row segment, then a private segment ending at
        # offset B-1 (t even) or a one-row segment at offset 0 of its own block
        NB = 2 * S + 2
        segs = np.zeros((S, 2, 3), np.int32)
        for t in range(S):
            segs[t, 0] = (0, 0, 1)
            segs[t, 1] = (1 + t, 3, B - 3) if t % 2 == 0 else (1 + t, 0, 1)
        nsegs = np.full(S, 2, np.int32)
        kr = (rng.standard_normal((1 + S * B, Hkv, 128)).astype(np.float16)).view(np.uint16)
        vr = (rng.standard_normal((1 + S * B, Hkv, 128)).astype(np.float16)).view(np.uint16)
        runs_k, runs_v, cu, st, tb = [kr[:1]], [vr[:1]], [0, 1], [0], [[0]]
        r = 1
        for t in range(S):
            off, ln = int(segs[t, 1, 1]), int(segs[t, 1, 2])
            runs_k.append(kr[r:r + ln]); runs_v.append(vr[r:r + ln])
            cu.append(cu[-1] + ln); st.append(off); tb.append([1 + t]); r += ln
        runs = (np.concatenate(runs_k), np.concatenate(runs_v), np.array(cu, np.int64),
                np.array(st, np.int32), np.array(tb, np.int32))
        print(f"[gpu] slotted append edges ({mode}) B={B}", flush=True)
        kp, vp, gk, gv = _pools_both(runs, NB, Hkv, B, "fp16")
        q = (rng.standard_normal((S, Hq, 128)).astype(np.float16)).view(np.uint16)
        kn = (rng.standard_normal((S, Hkv, 128)).astype(np.float16)).view(np.uint16)
        vn = (rng.standard_normal((S, Hkv, 128)).astype(np.float16)).view(np.uint16)
        slots = _check_append(q, kp, vp, gk, gv, kn, vn, segs, nsegs, Hkv, B, NB, "fp16")
        want = [(1 + t) * B + (B - 1 if t % 2 == 0 else 0) for t in range(S)]
        assert slots.tolist() == want


_big_cache = {}


def _big_radix():
    """A 1,024-sequence radix batch in tree order (1,024 tiles of the tiled
    kernel across 8 KV heads), with the oracle's append over the whole batch and
    its attention on 128 sampled sequences (computed once per module)."""
    if "w" not in _big_cache:
        cfg = get_config("c5")
        w = _tree_order(make_slotted_workload(cfg, num_seqs=1024))
        kp, vp = O.new_pools(w.num_blocks, cfg.num_kv_heads, cfg.block_size, 128,
                             NAN_BITS[cfg.dtype])
        kr, vr, cu, st, tb = w.runs()
        O.append_tokens(kp, vp, kr, vr, cu, st, tb, cfg.block_size, w.num_blocks)
        kp0, vp0 = kp.copy(), vp.copy()
        slots = O.append_slotted(kp, vp, w.k_new, w.v_new, w.segments, w.num_segments,
                                 cfg.block_size, w.num_blocks)
        sample = np.random.default_rng(77).choice(1024, size=128, replace=False)
        ref = O.attention_slotted(w.q[sample], kp, vp, w.segments[sample],
                                  w.num_segments[sample], cfg.num_kv_heads, cfg.block_size,
                                  w.num_blocks, scale_for(128), cfg.dtype)
        _big_cache.update(w=w, cfg=cfg, pools0=(kp0, vp0), pools=(kp, vp), slots=slots,
                          sample=sample, ref=ref)
    return _big_cache


def test_append_large_radix_batch(mode):
    """1,024 sequences in tree order, fused append: pools and slot ids bit for bit
    over the whole batch, outputs of 128 sampled sequences against the oracle."""
    c = _big_radix()
    w, cfg = c["w"], c["cfg"]
    print(f"[gpu] slotted append large radix batch ({mode}) S=1024 NB={w.num_blocks}",
          flush=True)
    assert mode != "tiles" or tile_list_fits(cfg.num_q_heads, cfg.num_kv_heads, cfg.block_size,
                                             w.segments.shape[1])
    gk = to_dev(c["pools0"][0], cfg.dtype, DEV)
    gv = to_dev(c["pools0"][1], cfg.dtype, DEV)
    got, slots = _gpu_append(w.q, gk, gv, w.k_new, w.v_new, w.segments, w.num_segments,
                             cfg.dtype, scale_for(128))
    assert np.array_equal(slots, c["slots"])
    assert np.array_equal(bits_of(gk), c["pools"][0]) and np.array_equal(bits_of(gv), c["pools"][1])
    ok, err, nbad = tol_ok(got[c["sample"]], c["ref"])
    assert ok, (err, nbad)


def _gpu_split_append(q, gk, gv, k_new, v_new, segs, nsegs, dtype, scale, P, B):
    """paged_attention_append_decode_slotted_split (pools written in place); returns
    the widened output, the slot ids and the arrival counters."""
    S, Hq, _ = q.shape
    Hkv = gk.shape[1]
    mp = -(-segs.shape[1] * B // P)
    out = torch.empty((S, Hq, 128), dtype=TDT[dtype], device=DEV)
    out.view(torch.int16).fill_(0x5555)
    po = torch.full((S, Hq, mp, 128), float("nan"), dtype=torch.float32, device=DEV)
    pl = torch.full((S, Hq, mp), float("nan"), dtype=torch.float32, device=DEV)
    ctr = torch.zeros((S, Hkv), dtype=torch.int32, device=DEV)
    slots = torch.full((S,), -2, dtype=torch.int64, device=DEV)
    pkv.paged_attention_append_decode_slotted_split(
        out, to_dev(q, dtype, DEV), gk, gv, to_dev(k_new, dtype, DEV), to_dev(v_new, dtype, DEV),
        i32(segs, DEV), i32(nsegs, DEV), P, po, pl, ctr, slot_out=slots, scale=scale)
    torch.cuda.synchronize()
    return widen_out(out), slots.cpu().numpy(), ctr


@pytest.mark.parametrize("key,P", [("c1a", 32), ("c2", 256), ("c2", 512), ("c4", 2048)])
def test_append_split_block_tables_as_segments(key, P):
    """The split decode with the fused append on block tables written as segments:
    the new token's slot (the table append's) starts as the NaN sentinel and ends
    with the new rows; pools and slot ids bit for bit, the oracle's attention, the
    counters back at zero."""
    w, r, segs, nsegs = _tables_as_segments(key)
    c = w.cfg
    B = c.block_size
    print(f"[gpu] slotted split append from tables {key} P={P}", flush=True)
    kp0, vp0 = r["k_pool"].copy(), r["v_pool"].copy()
    for t, slot in enumerate(r["slots"]):
        if slot >= 0:
            kp0[slot // B, :, slot % B, :] = w.nan_bits
            vp0[slot // B, :, slot % B, :] = w.nan_bits
    gk, gv = to_dev(kp0, c.dtype, DEV), to_dev(vp0, c.dtype, DEV)
    got, slots, ctr = _gpu_split_append(w.q, gk, gv, w.k_new, w.v_new, segs, nsegs, c.dtype,
                                        scale_for(c.head_dim), P, B)
    assert np.array_equal(slots, r["slots"])
    assert not bool(ctr.any())
    ref_blocks = np.unique(segs[:, :, 0][segs[:, :, 2] > 0])
    idx = torch.from_numpy(ref_blocks.astype(np.int64)).to(DEV)
    assert np.array_equal(bits_of(gk[idx]), r["k_pool"][ref_blocks])
    assert np.array_equal(bits_of(gv[idx]), r["v_pool"][ref_blocks])
    ok, err, nbad = tol_ok(got, r["out"])
    assert ok, (err, nbad)


@pytest.mark.parametrize("case", APPEND_CASES, ids=[f"seed{c[0]}" for c in APPEND_CASES])
@pytest.mark.parametrize("P", [16, 48])
def test_append_split_random_node_lists(case, P):
    """Random node lists ending in private leaves, split mode with the fused append
    at partitions of 16 and 48 positions (the row n-1 in every position of its
    partition across the cases), against the oracle's slotted append and
    attention; the empty sequence gets slot -1."""
    seed, S, Hq, Hkv, B, dtype, hi, per = case
    c = _node_case(seed, S, Hq, Hkv, B, dtype, hi, per, trunks=seed >= 11, leaves=True)
    print(f"[gpu] slotted split append seed={seed} P={P} S={S} B={B}", flush=True)
    kp, vp, gk, gv = _pools_both(c["runs"], c["NB"], Hkv, B, dtype)
    scale = scale_for(128)
    ref_slots = O.append_slotted(kp, vp, c["k_new"], c["v_new"], c["segs"], c["nsegs"], B,
                                 c["NB"])
    ref = O.attention_slotted(c["q"], kp, vp, c["segs"], c["nsegs"], Hkv, B, c["NB"], scale,
                              dtype)
    got, slots, ctr = _gpu_split_append(c["q"], gk, gv, c["k_new"], c["v_new"], c["segs"],
                                        c["nsegs"], dtype, scale, P, B)
    assert np.array_equal(slots, ref_slots)
    assert slots[-1 if seed >= 11 else 0] == -1
    assert not bool(ctr.any())
    assert np.array_equal(bits_of(gk), kp) and np.array_equal(bits_of(gv), vp)
    ok, err, nbad = tol_ok(got, ref)
    assert ok, (err, nbad)
