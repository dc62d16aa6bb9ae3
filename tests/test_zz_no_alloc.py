"""paged_attention_split_decode_noalloc (the entry point that allocates nothing:
partials and arrival counters in the library's fixed device array) through the
C ABI, against paged_attention_split_decode with a caller workspace: the same
output bits, pools and slots, on two calls in a row, the second with a smaller
batch; and within tolerance of the fp64 oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from workloads import get_config, make_workload  # noqa: E402
from oracle import oracle as O  # noqa: E402
from gpu_harness import (GpuStep, TORCH_DT, bits_of, merged_step, scale_for,  # noqa: E402
                         tol_ok, widen_out)
import paged_kv_cache_09_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)


def _compare(key, P):
    w = make_workload(get_config(key))
    c = w.cfg
    print(f"[gpu] no-alloc {key} P={P}", flush=True)
    g = GpuStep(w, append=False)
    ref, ctr = merged_step(g, P)
    g2 = GpuStep(w, append=False)
    out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=TORCH_DT[c.dtype],
                      device=g2.device)
    out.view(torch.int16).fill_(0x5555)
    pkv.paged_attention_split_decode_noalloc(out, g2.q, g2.k_pool, g2.v_pool, g2.tables, g2.lens,
                                             P, k_new=g2.k_new, v_new=g2.v_new,
                                             slot_out=g2.slots, scale=scale_for(c.head_dim))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(g2.slots, g.slots)
    assert torch.equal(g2.k_pool.view(torch.int16), g.k_pool.view(torch.int16))
    assert torch.equal(g2.v_pool.view(torch.int16), g.v_pool.view(torch.int16))
    r = O.run_step(w, scale_for(c.head_dim))
    assert np.array_equal(g2.slots.cpu().numpy(), r["slots"])
    ok, err, nbad = tol_ok(widen_out(out), r["out"])
    assert ok, f"{key} P={P}: max err {err}, {nbad} bad"
    assert np.array_equal(bits_of(g2.k_pool), r["k_pool"])


def test_noalloc_two_calls_second_smaller():
    """The edge batch (32 sequences, 4 partitions of 512 per row), then the tiny
    batch (4 sequences, partitions of 32) on the same scratch."""
    _compare("c2", 512)
    _compare("c1b", 32)
