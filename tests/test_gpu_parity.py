"""Parity of the HIP path (called through the C ABI) with the fp64 oracle.

Append and slot arithmetic: bit-exact.  Attention outputs (fp16/bf16) and
partition outputs: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| element by element.
Every workload runs at its full per-layer size, in the launch configuration the
benchmark times (single pass for the 7B and prefix workloads, split-context
partitions of 512 tokens for the edge workload and 2048 for the long-context one),
plus other partition sizes, ragged and empty sequences, every supported block
size and several GQA group sizes.
"""
import dataclasses
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import get_config, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from gpu_harness import (GpuStep, bits_of, fused_step, i32, merged_step, scale_for,  # noqa: E402
                         tol_ok, widen_out)
import paged_kv_cache_09_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

BENCH_P = {"c1a": 0, "c1b": 0, "c2": 512, "c3": 0, "c4": 2048, "c5": 0}
ALL = ["c1a", "c1b", "c2", "c3", "c4", "c5"]

_cache = {}


def oracle_for(key):
    """Oracle results of layer 0 of a workload (computed once per module)."""
    if key not in _cache:
        w = make_workload(get_config(key))
        c = w.cfg
        print(f"[oracle] {key}: S={c.num_seqs} NB={w.num_blocks}", flush=True)
        r = O.run_step(w, scale_for(c.head_dim))
        _cache[key] = (w, r)
    return _cache[key]


def referenced_blocks(w):
    return np.unique(w.tables[w.tables >= 0])


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("key", ALL)
def test_append_bit_exact(key):
    w, r = oracle_for(key)
    print(f"[gpu] append {key}", flush=True)
    g = GpuStep(w)
    torch.cuda.synchronize()
    assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
    ref = referenced_blocks(w)
    if w.num_blocks * w.cfg.num_kv_heads * w.cfg.block_size <= 64 * 1024 * 1024:
        assert np.array_equal(bits_of(g.k_pool), r["k_pool"])
        assert np.array_equal(bits_of(g.v_pool), r["v_pool"])
    else:
        # large pools: referenced blocks bit for bit, every other block untouched
        idx = torch.from_numpy(ref.astype(np.int64)).to(g.device)
        assert np.array_equal(bits_of(g.k_pool[idx]), r["k_pool"][ref])
        assert np.array_equal(bits_of(g.v_pool[idx]), r["v_pool"][ref])
        mask = torch.ones(w.num_blocks, dtype=torch.bool, device=g.device)
        mask[idx] = False
        sentinel = int(np.array([w.nan_bits], np.uint16).view(np.int16)[0])
        for pool in (g.k_pool, g.v_pool):
            v = pool.view(torch.int16)
            unref = torch.nonzero(mask).flatten()
            for a in range(0, unref.numel(), 2048):
                assert bool((v[unref[a:a + 2048]] == sentinel).all())


@pytest.mark.parametrize("key", ALL)
def test_decode_single_pass(key):
    w, r = oracle_for(key)
    print(f"[gpu] decode single {key}", flush=True)
    out, _, _ = GpuStep(w).decode(0)
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"{key}: max err {err}, {nbad} elements out of tolerance"


# c4 at P = 128 gives 128 partitions per row: the reduce's lse pass and its
# partition rows then run past the first 64 (and the first 8 requested up front)
PARTS = [("c1a", 32), ("c1b", 64), ("c2", 256), ("c2", 512), ("c3", 64), ("c3", 128), ("c3", 4096),
         ("c4", 128), ("c4", 1024), ("c4", 2048), ("c5", 128), ("c5", 256)]


@pytest.mark.parametrize("key,P", PARTS)
def test_decode_partitioned(key, P):
    w, r = oracle_for(key)
    c = w.cfg
    print(f"[gpu] decode partitioned {key} P={P}", flush=True)
    out, po, pl = GpuStep(w).decode(P)
    mp = po.shape[2]
    opo, opl = O.partials(w.q, r["k_pool"], r["v_pool"], w.tables, w.lengths, c.num_kv_heads,
                          c.block_size, w.num_blocks, scale_for(c.head_dim), c.dtype, P, mp)
    po, pl = po.cpu().numpy().astype(np.float64), pl.cpu().numpy().astype(np.float64)
    valid = ~np.isnan(opl)
    # partitions that hold no token are never written
    assert np.isnan(pl[~valid]).all() and np.isnan(po[~valid]).all()
    assert np.abs(pl[valid] - opl[valid]).max() <= 1e-3
    ok, err, nbad = tol_ok(po[valid], opo[valid])
    assert ok, f"partials: max err {err}, {nbad} bad"
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"merged: max err {err}, {nbad} bad"


# ---------------------------------------------------------------------------
FUSED = [(k, 0) for k in ALL] + [("c1b", 32), ("c2", 512), ("c3", 64), ("c4", 2048),
                                 ("c5", 128)]


@pytest.mark.parametrize("key,P", FUSED)
def test_fused_append_decode(key, P):
    """paged_attention_append_decode = paged_kv_append then paged_attention_decode:
    pools and slots bit-exact, output within tolerance of the oracle."""
    w, r = oracle_for(key)
    print(f"[gpu] fused {key} P={P}", flush=True)
    g = GpuStep(w, append=False)
    out = fused_step(g, P)
    torch.cuda.synchronize()
    assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
    ref = referenced_blocks(w)
    idx = torch.from_numpy(ref.astype(np.int64)).to(g.device)
    assert np.array_equal(bits_of(g.k_pool[idx]), r["k_pool"][ref])
    assert np.array_equal(bits_of(g.v_pool[idx]), r["v_pool"][ref])
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"{key} P={P}: max err {err}, {nbad} bad"


# ---------------------------------------------------------------------------
def _orders(n, seed, num_kv_heads):
    """Dispatch orders to try: the package's plan (long_first_order, the order the
    bench dispatches); sequences above twice the mean length first; the same with
    the shortest eighth of the batch last, longest of them first; the reverse of
    the batch; and a seeded random permutation."""
    S = len(n)
    big = [i for i in range(S) if n[i] > 2 * n.mean()]
    rest = [i for i in range(S) if i not in set(big)]
    shorts = sorted(sorted(rest, key=lambda i: n[i])[:S // 8], key=lambda i: -n[i])
    rng = np.random.default_rng(seed)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return {"plan": pkv.long_first_order(n, num_kv_heads, cus),
            "long_first": np.array(big + rest),
            "long_first_short_last": np.array(big + [i for i in rest if i not in set(shorts)]
                                              + shorts),
            "reversed": np.arange(S)[::-1].copy(), "random": rng.permutation(S)}


@pytest.mark.parametrize("key", ["c1a", "c2", "c3", "c4"])
def test_decode_ordered_equals_natural_order(key):
    """paged_attention_decode_ordered (fused append): pools and slots bit-exact
    against the oracle and the output within tolerance, for several dispatch
    orders; the output is also bit for bit the natural order's."""
    w, r = oracle_for(key)
    ref_blocks = referenced_blocks(w)
    idx = None
    natural = None
    for name, order in _orders(w.lengths, 7, w.cfg.num_kv_heads).items():
        print(f"[gpu] ordered decode {key} order={name}", flush=True)
        g = GpuStep(w, append=False)
        if natural is None:
            natural = fused_step(g, 0).cpu()
            g = GpuStep(w, append=False)
        out = torch.empty_like(g.q)
        pkv.paged_attention_decode_ordered(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens,
                                           i32(order, g.device), k_new=g.k_new,
                                           v_new=g.v_new, slot_out=g.slots)
        torch.cuda.synchronize()
        assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
        idx = torch.from_numpy(ref_blocks.astype(np.int64)).to(g.device)
        assert np.array_equal(bits_of(g.k_pool[idx]), r["k_pool"][ref_blocks])
        assert np.array_equal(bits_of(g.v_pool[idx]), r["v_pool"][ref_blocks])
        ok, err, nbad = tol_ok(widen_out(out), r["out"])
        assert ok, f"{key} {name}: max err {err}, {nbad} bad"
        assert torch.equal(out.cpu().view(torch.int16), natural.view(torch.int16)), name


def test_decode_ordered_debug_check_rejects_bad_orders(monkeypatch):
    w = _small(block_size=16, num_q_heads=12, num_kv_heads=2, lengths=(5, 40, 17))
    g = GpuStep(w)
    monkeypatch.setenv("PKV_DEBUG_CHECK", "1")
    out = torch.empty_like(g.q)
    good = i32(np.array([2, 0, 1]), g.device)
    pkv.paged_attention_decode_ordered(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens, good)
    for bad in ([0, 0, 1], [0, 1, 3], [-1, 1, 2]):  # a repeat, past the batch, negative
        with pytest.raises(pkv.PagedKVError) as e:
            pkv.paged_attention_decode_ordered(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens,
                                               i32(np.array(bad), g.device))
        assert e.value.status == -5


# ---------------------------------------------------------------------------
MERGED = [("c1b", 32), ("c2", 256), ("c2", 512), ("c3", 64), ("c3", 256), ("c4", 128),
          ("c4", 2048), ("c5", 128)]


@pytest.mark.parametrize("key,P", MERGED)
def test_split_decode_merged_in_launch(key, P):
    """paged_attention_split_decode: the partitions merged by the last work-group
    of each item give the oracle's output within tolerance, and the same bits as
    the split decode followed by the standalone merge; with the fused append, the
    pools and slots are bit-exact; the arrival counters end at zero, and a second
    call on the same counters gives the same bits."""
    w, r = oracle_for(key)
    print(f"[gpu] merged split {key} P={P}", flush=True)
    g = GpuStep(w, append=False)
    out, ctr = merged_step(g, P)
    torch.cuda.synchronize()
    assert not bool(ctr.any()), "arrival counters not back at zero"
    assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
    ref = referenced_blocks(w)
    idx = torch.from_numpy(ref.astype(np.int64)).to(g.device)
    assert np.array_equal(bits_of(g.k_pool[idx]), r["k_pool"][ref])
    assert np.array_equal(bits_of(g.v_pool[idx]), r["v_pool"][ref])
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"{key} P={P}: max err {err}, {nbad} bad"
    # the same pools now hold the appended rows: the plain split + standalone
    # merge and a second merged call (same counters) must give the same bits
    out2, _, _ = g.decode(P)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    out3, _ = merged_step(g, P, append=False, counters=ctr)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out3.view(torch.int16))
    assert not bool(ctr.any())


# ---------------------------------------------------------------------------
def _relabel(kbits, vbits, tables, seed):
    rng = np.random.default_rng(seed)
    pi = rng.permutation(kbits.shape[0])
    k2, v2 = np.empty_like(kbits), np.empty_like(vbits)
    k2[pi], v2[pi] = kbits, vbits
    t2 = np.where(tables >= 0, pi[np.maximum(tables, 0)], -1).astype(np.int32)
    return k2, v2, t2


@pytest.mark.parametrize("key,P", [("c1b", 0), ("c1b", 32), ("c5", 0), ("c2", 256)])
def test_block_relabelling_is_bitwise_invariant(key, P):
    w, _ = oracle_for(key)
    print(f"[gpu] relabel {key} P={P}", flush=True)
    g = GpuStep(w)
    out0, _, _ = g.decode(P)
    kb, vb = bits_of(g.k_pool), bits_of(g.v_pool)
    for seed in (1, 2):
        k2, v2, t2 = _relabel(kb, vb, w.tables, seed)
        g2 = GpuStep(w, tables=t2, k_pool_bits=k2, v_pool_bits=v2)
        out2, _, _ = g2.decode(P)
        assert torch.equal(out0.view(torch.int16), out2.view(torch.int16))


def _small(key="c1a", **kw):
    base = get_config(key)
    lens = kw.pop("lengths")
    B = kw.get("block_size", base.block_size)
    W = kw.pop("width", max(1, -(-max(lens) // B)))
    NB = kw.pop("pool", sum(-(-n // B) for n in lens) + 5)
    cfg = dataclasses.replace(base, key="edge", num_seqs=len(lens), fixed_lengths=tuple(lens),
                              max_blocks_per_seq=W, pool_blocks=NB, **kw)
    return make_workload(cfg, lengths=lens)


EDGE = [
    # (block_size, hq, hkv, dtype, lengths)
    (16, 2, 2, "fp16", (0, 1, 15, 16, 17, 31, 32, 33, 100)),
    (32, 4, 4, "bf16", (1, 31, 32, 33, 64, 65, 0, 300)),
    (64, 1, 1, "fp16", (1, 63, 64, 65, 200)),
    (128, 2, 2, "bf16", (127, 128, 129, 1, 0)),
    (256, 1, 1, "fp16", (255, 256, 257, 700)),
    (16, 12, 2, "fp16", (0, 1, 15, 16, 17, 47, 48, 49)),
    (32, 8, 4, "bf16", (1, 2, 31, 33, 95, 0)),
    (64, 16, 1, "fp16", (5, 64, 65, 190)),
    (128, 32, 8, "bf16", (1, 127, 129, 300)),
    (256, 6, 3, "fp16", (3, 256, 511, 513)),
    (16, 4, 2, "bf16", (16, 32, 48, 64, 80)),
    # odd group sizes: floor(16 / G) * G < 16 columns of the MFMA tile are used
    (16, 12, 4, "fp16", (0, 1, 15, 16, 17, 47, 48, 49, 130)),
    (128, 10, 2, "bf16", (1, 127, 128, 129, 300, 0)),
]


def _edge_params():
    """Each edge case single pass and at P = 256; block size 16 also at P = 16
    and 48 (partitions that are not a multiple of 32)."""
    out = []
    for e in EDGE:
        for P in [0, 256] + ([16, 48] if e[0] == 16 else []):
            out.append(e + (P,))
    return out


@pytest.mark.parametrize("B,hq,hkv,dt,lens,P", _edge_params())
def test_edge_cases(B, hq, hkv, dt, lens, P):
    print(f"[gpu] edge B={B} hq={hq} hkv={hkv} {dt} lens={lens} P={P}", flush=True)
    w = _small(block_size=B, num_q_heads=hq, num_kv_heads=hkv, dtype=dt, lengths=lens,
               width=max(-(-max(lens) // B), 1) + 1)
    c = w.cfg
    r = O.run_step(w, scale_for(c.head_dim))
    g = GpuStep(w)
    torch.cuda.synchronize()
    assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
    assert np.array_equal(bits_of(g.k_pool), r["k_pool"])
    assert np.array_equal(bits_of(g.v_pool), r["v_pool"])
    if P and P % B:
        return
    out, _, _ = g.decode(P)
    got = widen_out(out)
    ok, err, nbad = tol_ok(got, r["out"])
    assert ok, f"max err {err}, {nbad} bad"
    for s, n in enumerate(lens):
        if n == 0:
            assert (got[s] == 0).all()
    # the fused append + decode on a fresh copy gives the same pools and output
    g2 = GpuStep(w, append=False)
    out2 = fused_step(g2, P)
    torch.cuda.synchronize()
    assert np.array_equal(g2.slots.cpu().numpy(), r["slots"])
    assert np.array_equal(bits_of(g2.k_pool), r["k_pool"])
    assert np.array_equal(bits_of(g2.v_pool), r["v_pool"])
    ok, err, nbad = tol_ok(widen_out(out2), r["out"])
    assert ok, f"fused: max err {err}, {nbad} bad"
    if P:
        # the partitions merged in the launch: same bits as the split + merge
        g3 = GpuStep(w, append=False)
        out3, ctr = merged_step(g3, P)
        torch.cuda.synchronize()
        assert not bool(ctr.any())
        assert np.array_equal(bits_of(g3.k_pool), r["k_pool"])
        assert torch.equal(out3.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("P", [0, 1024])
def test_longest_context(P):
    """One sequence of 131,071 tokens (1,024 blocks of 128, the last one short of a
    token) beside a one-token sequence, at the long-context shapes (32 query / 8 KV
    heads, bf16): single pass (8,192 sub-tiles through one work-group per KV head)
    and 128 partitions.  Pools, slots and outputs against the oracle."""
    lens = (131071, 1)
    print(f"[gpu] longest context n={lens} P={P}", flush=True)
    w = _small("c4", lengths=lens, width=1025, pool=1030)
    c = w.cfg
    r = O.run_step(w, scale_for(c.head_dim))
    g = GpuStep(w, append=False)
    out = fused_step(g, P)
    torch.cuda.synchronize()
    assert np.array_equal(g.slots.cpu().numpy(), r["slots"])
    assert np.array_equal(bits_of(g.k_pool), r["k_pool"])
    assert np.array_equal(bits_of(g.v_pool), r["v_pool"])
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"max err {err}, {nbad} bad"


def test_scale_zero_is_mean_over_exactly_n_tokens():
    """A zero scale makes attention the plain mean of the n value rows; any
    leakage of masked slots (NaN sentinels) or missing token shows up here."""
    w = _small(block_size=16, num_q_heads=12, num_kv_heads=2, lengths=(1, 17, 33, 64))
    c = w.cfg
    r = O.run_step(w, 0.0)
    for P in (0, 32):
        out, _, _ = GpuStep(w).decode(P, scale=0.0)
        ok, err, nbad = tol_ok(widen_out(out), r["out"])
        assert ok, f"P={P}: max err {err}"
    del c


def test_debug_check_rejects_bad_contents(monkeypatch):
    w = _small(block_size=16, num_q_heads=12, num_kv_heads=2, lengths=(5, 40))
    g = GpuStep(w)
    monkeypatch.setenv("PKV_DEBUG_CHECK", "1")
    out = torch.empty_like(g.q)
    pkv.paged_attention_decode(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens)  # valid: passes
    bad = g.tables.clone()
    bad[1, 1] = w.num_blocks + 3  # entry outside the pool
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_decode(out, g.q, g.k_pool, g.v_pool, bad, g.lens)
    assert e.value.status == -5
    long = g.lens.clone()
    long[0] = w.cfg.max_blocks_per_seq * 16 + 1  # longer than the table row
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_kv_append(g.k_pool, g.v_pool, g.q[:, :2].contiguous(), g.q[:, :2].contiguous(),
                            g.tables, long)
    assert e.value.status == -5


def test_argument_errors():
    w = _small(block_size=16, num_q_heads=12, num_kv_heads=2, lengths=(5, 40))
    g = GpuStep(w)
    out = torch.empty_like(g.q)
    with pytest.raises(pkv.PagedKVError) as e:   # partition not a multiple of the block
        pkv.paged_attention_decode(None, g.q, g.k_pool, g.v_pool, g.tables, g.lens,
                                   partition_size=24, part_o=torch.empty(2, 12, 4, 128,
                                                                         device=g.device),
                                   part_lse=torch.empty(2, 12, 4, device=g.device))
    assert e.value.status == -1
    with pytest.raises(pkv.PagedKVError) as e:   # workspace too small
        pkv.paged_attention_decode(None, g.q, g.k_pool, g.v_pool, g.tables, g.lens,
                                   partition_size=32,
                                   part_o=torch.empty(2, 12, 1, 128, device=g.device),
                                   part_lse=torch.empty(2, 12, 1, device=g.device))
    assert e.value.status == -3
    with pytest.raises(pkv.PagedKVError) as e:   # 12 query heads over 5 KV heads
        kp5 = torch.empty((w.num_blocks, 5, 16, 128), dtype=torch.float16, device=g.device)
        pkv.paged_attention_decode(out, g.q, kp5, kp5, g.tables, g.lens)
    assert e.value.status == -1
    with pytest.raises(pkv.PagedKVError) as e:   # head_dim 64 is not built
        q64 = torch.empty((2, 12, 64), dtype=torch.float16, device=g.device)
        kp64 = torch.empty((w.num_blocks, 2, 16, 64), dtype=torch.float16, device=g.device)
        pkv.paged_attention_decode(q64.clone(), q64, kp64, kp64, g.tables, g.lens)
    assert e.value.status == -2


def test_no_cpu_fallback():
    w = _small(block_size=16, num_q_heads=12, num_kv_heads=2, lengths=(5, 40))
    g = GpuStep(w)
    with pytest.raises(ValueError):
        pkv.paged_attention_decode(torch.empty(2, 12, 128, dtype=torch.float16), g.q.cpu(),
                                   g.k_pool.cpu(), g.v_pool.cpu(), g.tables.cpu(), g.lens.cpu())


def test_library_loaded_from_tree():
    path = pkv.lib_path()
    assert os.path.dirname(path).endswith("paged_kv_cache_09_amd")
    with open("/proc/self/maps") as f:
        assert path in f.read()
