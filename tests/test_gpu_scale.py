"""Launches of more than 65,535 work-groups: 16,384 short sequences (MHA with 8
heads, and GQA 4:1 with 8 KV heads: 131,072 work-groups each), the fused append
and single-pass decode through the C ABI.  Pools and slot ids are compared bit
for bit with the oracle over the whole batch, outputs on 256 sampled sequences
within |gpu - oracle| <= 1e-2 + 1e-2 |oracle|."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from workloads.gen import NAN_BITS  # noqa: E402
from gpu_harness import bits_of, i32, i64, scale_for, to_dev, tol_ok, widen_out  # noqa: E402
import paged_kv_cache_09_amd as pkv  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("no GPU", allow_module_level=True)

DEV = torch.device("cuda:0")


def _case(seed, S, Hq, Hkv, B, dtype, n_hi):
    """S sequences of 1..n_hi attended positions (the new token included), tables
    dealt from a shuffled free list, histories written into the oracle's pools."""
    rng = np.random.default_rng(seed)

    def draw(*shape):
        x = rng.standard_normal(shape, dtype=np.float32)
        if dtype == "fp16":
            return x.astype(np.float16).view(np.uint16)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    n = rng.integers(1, n_hi + 1, size=S).astype(np.int64)
    nb = -(-n // B)
    W = int(nb.max())
    NB = int(nb.sum()) + 8
    free = rng.permutation(NB).astype(np.int32)
    tables = np.full((S, W), -1, np.int32)
    pos = 0
    for s in range(S):
        tables[s, :nb[s]] = free[pos:pos + nb[s]]
        pos += nb[s]
    hist = n - 1
    rows_k, rows_v = draw(int(hist.sum()), Hkv, 128), draw(int(hist.sum()), Hkv, 128)
    cu = np.concatenate([[0], np.cumsum(hist)]).astype(np.int64)
    kp, vp = O.new_pools(NB, Hkv, B, 128, NAN_BITS[dtype])
    O.append_tokens(kp, vp, rows_k, rows_v, cu, np.zeros(S, np.int32), tables, B, NB)
    return dict(n=n.astype(np.int32), tables=tables, NB=NB, kp=kp, vp=vp, q=draw(S, Hq, 128),
                kn=draw(S, Hkv, 128), vn=draw(S, Hkv, 128))


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8)], ids=["mha", "gqa4"])
def test_fused_decode_beyond_65535_work_groups(Hq, Hkv):
    S, B, dtype = 16384, 16, "fp16"
    c = _case(90 + Hq, S, Hq, Hkv, B, dtype, 32)
    print(f"[gpu] scale S={S} Hq={Hq} Hkv={Hkv} NB={c['NB']} work-groups={S * Hkv}", flush=True)
    gk, gv = to_dev(c["kp"], dtype, DEV), to_dev(c["vp"], dtype, DEV)
    slots_ref = O.append(c["kp"], c["vp"], c["kn"], c["vn"], c["tables"], c["n"], B, c["NB"])
    sample = np.random.default_rng(91).choice(S, size=256, replace=False)
    ref = O.attention(c["q"][sample], c["kp"], c["vp"], c["tables"][sample], c["n"][sample], Hkv,
                      B, c["NB"], scale_for(128), dtype)
    out = torch.empty((S, Hq, 128), dtype=torch.float16, device=DEV)
    slots = torch.full((S,), -7, dtype=torch.int64, device=DEV)
    pkv.paged_attention_append_decode(out, to_dev(c["q"], dtype, DEV), gk, gv,
                                      to_dev(c["kn"], dtype, DEV), to_dev(c["vn"], dtype, DEV),
                                      i32(c["tables"], DEV), i32(c["n"], DEV), slot_out=slots)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), slots_ref)
    assert np.array_equal(bits_of(gk), c["kp"]) and np.array_equal(bits_of(gv), c["vp"])
    ok, err, nbad = tol_ok(widen_out(out)[sample], ref)
    assert ok, (err, nbad)


def test_merged_split_decode_beyond_65535_work_groups():
    """The split decode with the in-kernel merge over 131,072 (sequence, KV head)
    items: partitions of 16 positions, so most items merge two partitions; the
    arrival counters are left zero."""
    S, Hq, Hkv, B, dtype, P = 16384, 32, 8, 16, "fp16", 16
    c = _case(95, S, Hq, Hkv, B, dtype, 32)
    print(f"[gpu] scale merged split S={S} Hq={Hq} Hkv={Hkv} P={P}", flush=True)
    gk, gv = to_dev(c["kp"], dtype, DEV), to_dev(c["vp"], dtype, DEV)
    slots_ref = O.append(c["kp"], c["vp"], c["kn"], c["vn"], c["tables"], c["n"], B, c["NB"])
    sample = np.random.default_rng(96).choice(S, size=256, replace=False)
    ref = O.attention(c["q"][sample], c["kp"], c["vp"], c["tables"][sample], c["n"][sample], Hkv,
                      B, c["NB"], scale_for(128), dtype)
    mp = -(-c["tables"].shape[1] * B // P)
    out = torch.empty((S, Hq, 128), dtype=torch.float16, device=DEV)
    po = torch.empty((S, Hq, mp, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((S, Hq, mp), dtype=torch.float32, device=DEV)
    ctr = torch.zeros((S, Hkv), dtype=torch.int32, device=DEV)
    slots = torch.full((S,), -7, dtype=torch.int64, device=DEV)
    pkv.paged_attention_split_decode(out, to_dev(c["q"], dtype, DEV), gk, gv, i32(c["tables"], DEV),
                                     i32(c["n"], DEV), P, po, pl, ctr,
                                     k_new=to_dev(c["kn"], dtype, DEV),
                                     v_new=to_dev(c["vn"], dtype, DEV), slot_out=slots)
    torch.cuda.synchronize()
    assert not bool(ctr.any())
    assert np.array_equal(slots.cpu().numpy(), slots_ref)
    assert np.array_equal(bits_of(gk), c["kp"]) and np.array_equal(bits_of(gv), c["vp"])
    ok, err, nbad = tol_ok(widen_out(out)[sample], ref)
    assert ok, (err, nbad)
