"""The seeded input generator: determinism, shapes of the five workloads and the
rounding of the draws to 16-bit formats."""
import math

import numpy as np
import pytest

from workloads import CONFIGS, get_config, make_workload
from workloads.gen import draw_lengths, f32_to_bf16_bits, f32_to_f16_bits, pool_blocks_for


@pytest.mark.parametrize("key", ["c1a", "c2", "c5"])
def test_deterministic(key):
    a = make_workload(get_config(key), layer=1)
    b = make_workload(get_config(key), layer=1, threads=1)
    for f in ("lengths", "tables", "q", "k_new", "v_new", "k_src", "v_src", "seg_cu"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = make_workload(get_config(key), layer=2)
    assert np.array_equal(a.tables, c.tables)      # tables are shared by all layers
    assert not np.array_equal(a.q, c.q)            # values are not


def test_lengths_of_each_config():
    assert list(draw_lengths(get_config("c1a"))) == [5, 16, 37, 64]
    assert list(draw_lengths(get_config("c1b"))) == [6, 17, 38, 65]
    n2 = draw_lengths(get_config("c2"))
    assert n2.min() >= 16 and n2.max() <= 2048 and len(n2) == 32
    c3 = get_config("c3")
    # the lognormal's own 90th percentile is 287 (hnwysp.cn page, §3.1)
    assert abs(math.exp(c3.lognormal_mu + 1.2815515655446004 * c3.lognormal_sigma) - 287) < 1e-9
    n3 = draw_lengths(c3)
    assert n3.min() >= 1 and n3.max() <= 4096 and len(n3) == 128
    assert 230 <= np.percentile(n3, 90) <= 340
    assert 4.5 <= np.mean(-(-n3 // 32)) <= 7.5     # "about six blocks per sequence"
    assert list(draw_lengths(get_config("c4"))) == [16384] * 8
    n5 = draw_lengths(get_config("c5"))
    priv = -(-(n5 - 512) // 16)
    assert priv.min() >= 1 and priv.max() <= 8 and len(n5) == 256


@pytest.mark.parametrize("key", sorted(CONFIGS))
def test_tables_are_valid(key):
    cfg = get_config(key)
    n = draw_lengths(cfg)
    NB = pool_blocks_for(cfg, n)
    if key == "c3":
        assert NB == 18842
    if key == "c4":
        assert NB == 1178
    from workloads.gen import draw_tables
    t = draw_tables(cfg, n, NB)
    need = -(-n // cfg.block_size)
    used = []
    for s in range(cfg.num_seqs):
        row = t[s]
        assert (row[:need[s]] >= 0).all() and (row[:need[s]] < NB).all()
        assert (row[need[s]:] == -1).all()
        used.extend(row[:need[s]].tolist())
    if key == "c5":
        npre = 512 // 16
        assert (t[:, :npre] == t[0, :npre]).all()
        private = [b for s in range(cfg.num_seqs) for b in t[s, npre:need[s]]]
        assert len(set(private)) == len(private)
        assert not set(private) & set(t[0, :npre].tolist())
    else:
        assert len(set(used)) == len(used)          # no block shared between sequences


def test_history_segments_cover_every_position_once():
    for key in ("c1a", "c1b", "c5"):
        w = make_workload(get_config(key))
        for s in range(w.cfg.num_seqs):
            K, V = w.logical_kv(s)
            assert K.shape[0] == w.lengths[s] == V.shape[0]


def test_value_distribution():
    w = make_workload(get_config("c2"))
    x = w.k_src.view(np.float16).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1.0) < 0.01
    w3 = make_workload(get_config("c1a"), layer=0)
    assert w3.q.dtype == np.uint16


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is exactly halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1)
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even (1 + 2^-6)
    x = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 0.0], np.float32)
    got = f32_to_bf16_bits(x)
    assert list(got) == [0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000]
    assert f32_to_bf16_bits(np.array([np.nan], np.float32))[0] & 0x7FC0 == 0x7FC0


def test_f16_rounding_is_nearest_even():
    x = np.array([1 + 2**-11, 1 + 3 * 2**-11, 65520.0], np.float32)
    assert list(f32_to_f16_bits(x)) == [0x3C00, 0x3C02, 0x7C00]
