"""The library's calls inside a HIP graph (torch.cuda.CUDAGraph capture on the
current stream): every replay must reproduce the eager result bit for bit, with
eager work and synchronisation between replays.  The calls enqueue kernels only
(no memset nodes, no allocation, no synchronisation), so they are capturable."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import get_config, make_workload  # noqa: E402
from gpu_harness import GpuStep, scale_for  # noqa: E402
import paged_kv_cache_09_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("key,P,merged", [("c1a", 0, False), ("c2", 512, False),
                                           ("c5", 0, False), ("c2", 512, True),
                                           ("c4", 2048, True), ("c3", 64, True)])
def test_graph_replays_match_eager(key, P, merged):
    """merged: paged_attention_split_decode, whose arrival counters must be back
    at zero after every call for the next replay to merge correctly."""
    w = make_workload(get_config(key))
    c = w.cfg
    print(f"[gpu] graph {key} P={P}", flush=True)
    g = GpuStep(w, append=False)
    S, Hq, D = c.num_seqs, c.num_q_heads, c.head_dim
    dt = g.q.dtype
    mp = pkv.max_partitions(c.max_blocks_per_seq, c.block_size, P) if P else 1
    po = torch.zeros((S, Hq, mp, D), dtype=torch.float32, device=g.device)
    pl = torch.zeros((S, Hq, mp), dtype=torch.float32, device=g.device)
    out = torch.zeros((S, Hq, D), dtype=dt, device=g.device)
    scale = scale_for(D)
    prefix = key == "c5"
    if prefix:
        cu = torch.tensor([0, S], dtype=torch.int32, device=g.device)
        plen = torch.tensor([c.prefix_tokens], dtype=torch.int32, device=g.device)
    ctr = torch.zeros((S, c.num_kv_heads), dtype=torch.int32, device=g.device)

    def step():
        if prefix:
            pkv.paged_attention_prefix_decode(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens, cu,
                                              plen, po, pl, k_new=g.k_new, v_new=g.v_new,
                                              slot_out=g.slots, scale=scale)
        elif merged:
            pkv.paged_attention_split_decode(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens, P,
                                             po, pl, ctr, k_new=g.k_new, v_new=g.v_new,
                                             slot_out=g.slots, scale=scale)
        elif P:
            pkv.paged_attention_append_decode(None, g.q, g.k_pool, g.v_pool, g.k_new, g.v_new,
                                              g.tables, g.lens, g.slots, scale=scale,
                                              partition_size=P, part_o=po, part_lse=pl)
            pkv.paged_attention_reduce(out, po, pl, g.lens, P)
        else:
            pkv.paged_attention_append_decode(out, g.q, g.k_pool, g.v_pool, g.k_new, g.v_new,
                                              g.tables, g.lens, g.slots, scale=scale)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    eager_k = g.k_pool.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), \
            f"replay {rep} differs from the eager result"
        # pools hold NaN sentinels in unused slots: compare bit patterns
        assert torch.equal(g.k_pool.view(torch.int16), eager_k.view(torch.int16))
        assert not bool(ctr.any()), "arrival counters not back at zero"
        scratch = (g.q.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        del scratch
    assert np.isfinite(out.float().cpu().numpy()).all()


@pytest.mark.parametrize("P", [0, 64])
def test_slotted_append_graph_replays_match_eager(P):
    """The fused slotted append in a graph: single pass (the tiled kernel on the
    radix batch) and split mode with the in-kernel merge (arrival counters back
    at zero after every replay); every replay equals the eager call bit for bit."""
    import dataclasses
    from workloads.slotted import make_slotted_workload
    cfg = get_config("c5")
    w = make_slotted_workload(cfg)
    perm = sorted(range(len(w.paths)), key=lambda t: w.paths[t])  # tree order
    w = dataclasses.replace(w, paths=[w.paths[t] for t in perm], q=w.q[perm],
                            segments=w.segments[perm], num_segments=w.num_segments[perm],
                            k_new=w.k_new[perm], v_new=w.v_new[perm])
    print(f"[gpu] graph slotted append P={P}", flush=True)
    dev = torch.device("cuda:0")
    dt = torch.float16

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(dt)

    kr, vr, cu, st, tb = w.runs()
    kp = torch.zeros((w.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim), dtype=dt,
                     device=dev)
    vp = torch.zeros_like(kp)
    pkv.paged_kv_append_tokens(kp, vp, up(kr), up(vr), torch.from_numpy(cu).to(dev),
                               torch.from_numpy(st).to(dev), torch.from_numpy(tb).to(dev))
    S, Hq, D = len(w.paths), cfg.num_q_heads, cfg.head_dim
    q, kn, vn = up(w.q), up(w.k_new), up(w.v_new)
    segs = torch.from_numpy(w.segments).to(dev)
    ns = torch.from_numpy(w.num_segments).to(dev)
    out = torch.zeros((S, Hq, D), dtype=dt, device=dev)
    slots = torch.zeros((S,), dtype=torch.int64, device=dev)
    mp = -(-w.segments.shape[1] * cfg.block_size // P) if P else 1
    po = torch.zeros((S, Hq, mp, D), dtype=torch.float32, device=dev)
    pl = torch.zeros((S, Hq, mp), dtype=torch.float32, device=dev)
    ctr = torch.zeros((S, cfg.num_kv_heads), dtype=torch.int32, device=dev)

    def step():
        if P:
            pkv.paged_attention_append_decode_slotted_split(out, q, kp, vp, kn, vn, segs, ns, P,
                                                            po, pl, ctr, slot_out=slots)
        else:
            pkv.paged_attention_append_decode_slotted(out, q, kp, vp, kn, vn, segs, ns,
                                                      slot_out=slots)

    step()
    torch.cuda.synchronize()
    eager, eager_k, eager_v, eager_s = out.clone(), kp.clone(), vp.clone(), slots.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        slots.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(kp.view(torch.int16), eager_k.view(torch.int16))
        assert torch.equal(vp.view(torch.int16), eager_v.view(torch.int16))
        assert torch.equal(slots, eager_s)
        assert not bool(ctr.any()), "arrival counters not back at zero"
        scratch = (q.float() * 2).sum()
        torch.cuda.synchronize()
        del scratch
    assert np.isfinite(out.float().cpu().numpy()).all()
