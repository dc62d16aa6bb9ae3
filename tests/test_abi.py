"""The C-ABI library loads, exports every symbol include/paged_kv.h declares, and
rejects invalid arguments on the host before touching the device (so these run
without a GPU; no compute call is made)."""
import ctypes as C
import os

import pytest

import paged_kv_cache_09_amd as pkv

EINVAL, ENOTSUP, EWORKSPACE = -1, -2, -3
P = C.c_void_p


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


# The argument-error tests pass placeholder addresses that are never dereferenced
# because validation rejects them on the host.  They are meant for machines
# without a GPU; on a GPU machine they are skipped so that a validation bug could
# never turn into a launch with placeholder pointers.
host_only = pytest.mark.skipif(_gpu_present(), reason="host-validation tests run without a GPU")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkv.lib_path()):
        from paged_kv_cache_09_amd import build
        build.build()
    return pkv.load()


def test_every_declared_symbol_is_exported(lib):
    declared = pkv.header_symbols()
    assert {"paged_kv_append", "paged_kv_append_tokens", "paged_kv_copy_blocks",
            "paged_attention_decode", "paged_attention_append_decode",
            "paged_attention_prefix_decode", "paged_attention_decode_slotted",
            "paged_attention_reduce", "paged_attention_split_decode",
            "paged_attention_split_decode_noalloc", "paged_kv_copy_slots",
            "paged_attention_decode_slotted_split", "paged_attention_prefix_split_decode",
            "paged_attention_decode_ordered", "paged_attention_append_decode_slotted",
            "paged_attention_append_decode_slotted_split",
            "pkv_status_string",
            "pkv_max_partitions"} <= set(declared)
    assert pkv.exported_symbols() == declared


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert pkv.status_string(code) and pkv.status_string(code) != "unknown status"
    assert pkv.status_string(7) == "unknown status"


def test_max_partitions(lib):
    assert pkv.max_partitions(128, 128, 1024) == 16
    assert pkv.max_partitions(5, 16, 32) == 3
    assert pkv.max_partitions(0, 16, 32) == 0


A = P(1 << 20)  # a 16-byte-aligned non-null address; never dereferenced by these calls


def decode(lib, **kw):
    args = dict(out=A, q=A, k=A, v=A, t=A, n=A, S=2, Hq=12, Hkv=2, D=128, B=16, W=5, NB=64,
                scale=0.088, P=0, MP=0, po=None, pl=None, dt=0)
    args.update(kw)
    return lib.paged_attention_decode(args["out"], args["q"], args["k"], args["v"], args["t"],
                                      args["n"], args["S"], args["Hq"], args["Hkv"], args["D"],
                                      args["B"], args["W"], args["NB"], args["scale"], args["P"],
                                      args["MP"], args["po"], args["pl"], args["dt"], None)


@host_only
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), EINVAL),
    (dict(k=None), EINVAL),
    (dict(out=None), EINVAL),
    (dict(Hq=12, Hkv=5), EINVAL),
    (dict(D=64), ENOTSUP),
    (dict(B=24), ENOTSUP),
    (dict(B=8), ENOTSUP),
    (dict(Hq=34, Hkv=2), ENOTSUP),          # group of 17 query heads
    (dict(dt=3), ENOTSUP),
    (dict(S=-1), EINVAL),
    (dict(NB=0), EINVAL),
    (dict(P=24, MP=4, po=A, pl=A), EINVAL),  # partition not a multiple of the block (16)
    (dict(P=32, B=64, W=2, MP=4, po=A, pl=A), EINVAL),  # not a multiple of the block
    (dict(P=32, MP=1, po=A, pl=A), EWORKSPACE),
    (dict(P=32, MP=3, po=None, pl=A), EWORKSPACE),
    (dict(q=P((1 << 20) + 2)), EINVAL),      # misaligned
    (dict(scale=float("inf")), EINVAL),
    (dict(scale=float("-inf")), EINVAL),
    (dict(S=0), 0),                          # nothing to do
])
def test_decode_argument_errors(lib, kw, code):
    assert decode(lib, **kw) == code


@host_only
def test_append_argument_errors(lib):
    f = lib.paged_kv_append
    ok = dict(S=2, Hkv=2, D=128, B=16, W=5, NB=64, dt=0)

    def call(kp=A, vp=A, kn=A, vn=A, t=A, n=A, slot=None, **kw):
        a = dict(ok)
        a.update(kw)
        return f(kp, vp, kn, vn, t, n, slot, a["S"], a["Hkv"], a["D"], a["B"], a["W"], a["NB"],
                 a["dt"], None)

    assert call(kp=None) == EINVAL
    assert call(D=96) == ENOTSUP
    assert call(B=48) == ENOTSUP
    assert call(dt=2) == ENOTSUP
    assert call(slot=P((1 << 20) + 4)) == EINVAL
    assert call(S=0) == 0


@host_only
def test_append_tokens_argument_errors(lib):
    f = lib.paged_kv_append_tokens
    assert f(None, A, A, A, A, A, A, 2, 10, 2, 128, 16, 5, 64, 0, None) == EINVAL
    assert f(A, A, None, A, A, A, A, 2, 10, 2, 128, 16, 5, 64, 0, None) == EINVAL
    assert f(A, A, A, A, A, A, A, 2, -1, 2, 128, 16, 5, 64, 0, None) == EINVAL
    assert f(A, A, A, A, A, A, A, 2, 10, 2, 64, 16, 5, 64, 0, None) == ENOTSUP
    assert f(A, A, A, A, A, A, A, 0, 0, 2, 128, 16, 5, 64, 0, None) == 0


@host_only
def test_copy_blocks_argument_errors(lib):
    f = lib.paged_kv_copy_blocks
    two = (P * 2)(A, A)

    def call(kp=two, vp=two, L=2, src=A, dst=A, n=3, Hkv=2, D=128, B=16, NB=64, dt=0):
        return f(kp, vp, L, src, dst, n, Hkv, D, B, NB, dt, None)

    assert call(kp=None) == EINVAL
    assert call(L=0) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(src=None) == EINVAL
    assert call(dst=P((1 << 20) + 2)) == EINVAL                 # misaligned ids
    assert call(kp=(P * 2)(A, None)) == EINVAL                  # a null pool
    assert call(vp=(P * 2)(A, P((1 << 20) + 8))) == EINVAL     # a misaligned pool
    assert call(D=64) == ENOTSUP
    assert call(B=8) == ENOTSUP
    assert call(dt=4) == ENOTSUP
    many = (P * 129)(*([A] * 129))
    assert call(kp=many, vp=many, L=129) == ENOTSUP            # more layers than one launch takes
    assert call(n=0, src=None, dst=None) == 0                   # nothing to copy


@host_only
def test_split_decode_argument_errors(lib):
    f = lib.paged_attention_split_decode

    def call(out=A, kn=None, vn=None, ctr=A, S=2, Hq=12, Hkv=2, B=16, W=5, P_=32, MP=3, po=A,
             pl=A, scale=0.088, dt=0):
        return f(out, A, A, A, kn, vn, None, A, A, S, Hq, Hkv, 128, B, W, 64, scale, P_, MP,
                 po, pl, ctr, dt, None)

    assert call(ctr=None) == EINVAL              # the arrival counters are required
    assert call(out=None) == EINVAL              # the merge writes `out`
    assert call(P_=0) == EINVAL                  # a split mode: partitions required
    assert call(P_=24) == EINVAL                 # not a multiple of the block
    assert call(kn=A) == EINVAL                  # k_new without v_new
    assert call(ctr=P((1 << 20) + 2)) == EINVAL  # misaligned counters
    assert call(MP=2) == EWORKSPACE              # 80 positions need 3 partitions of 32
    assert call(po=None) == EWORKSPACE
    assert call(Hq=34) == ENOTSUP
    assert call(scale=float("inf")) == EINVAL
    assert call(S=0) == 0


@host_only
def test_decode_ordered_argument_errors(lib):
    f = lib.paged_attention_decode_ordered

    def call(out=A, kn=None, vn=None, order=A, S=2, Hq=12, Hkv=2, B=16, W=5, scale=0.088,
             dt=0):
        return f(out, A, A, A, kn, vn, None, A, A, order, S, Hq, Hkv, 128, B, W, 64, scale, dt,
                 None)

    assert call(order=None) == EINVAL               # the order is required
    assert call(order=P((1 << 20) + 2)) == EINVAL   # misaligned order
    assert call(out=None) == EINVAL
    assert call(kn=A) == EINVAL                     # k_new without v_new
    assert call(Hq=34) == ENOTSUP
    assert call(B=24) == ENOTSUP
    assert call(scale=float("inf")) == EINVAL
    assert call(S=0) == 0


@host_only
def test_split_decode_noalloc_argument_errors(lib):
    f = lib.paged_attention_split_decode_noalloc

    def call(out=A, kn=None, vn=None, S=2, Hq=12, Hkv=2, B=16, W=5, P_=32, scale=0.088, dt=0):
        return f(out, A, A, A, kn, vn, None, A, A, S, Hq, Hkv, 128, B, W, 64, scale, P_, dt,
                 None)

    assert call(out=None) == EINVAL
    assert call(P_=0) == EINVAL
    assert call(P_=24) == EINVAL                 # not a multiple of the block
    assert call(kn=A) == EINVAL                  # k_new without v_new
    assert call(Hq=34) == ENOTSUP
    assert call(B=24) == ENOTSUP
    # beyond the fixed scratch: 65,536 (sequence, KV head) counters, 32,768
    # (sequence, query head, partition) partial rows
    assert call(S=32769, Hq=4, Hkv=4, W=1) == EWORKSPACE
    assert call(S=128, Hq=32, Hkv=32, B=32, W=128, P_=256) == EWORKSPACE  # 65,536 rows
    assert call(S=0) == 0


@host_only
def test_copy_slots_argument_errors(lib):
    f = lib.paged_kv_copy_slots
    two = (P * 2)(A, A)

    def call(kp=two, vp=two, L=2, c=A, n=3, Hkv=2, D=128, B=16, NB=64, dt=0):
        return f(kp, vp, L, c, n, Hkv, D, B, NB, dt, None)

    assert call(kp=None) == EINVAL
    assert call(L=0) == EINVAL
    assert call(n=-1) == EINVAL
    assert call(c=None) == EINVAL
    assert call(c=P((1 << 20) + 2)) == EINVAL                   # misaligned tuples
    assert call(vp=(P * 2)(A, None)) == EINVAL                  # a null pool
    assert call(D=64) == ENOTSUP
    assert call(B=24) == ENOTSUP
    assert call(dt=3) == ENOTSUP
    many = (P * 129)(*([A] * 129))
    assert call(kp=many, vp=many, L=129) == ENOTSUP
    assert call(n=0, c=None) == 0                                # nothing to copy


@host_only
def test_prefix_decode_argument_errors(lib):
    f = lib.paged_attention_prefix_decode

    def call(out=A, kn=None, vn=None, cu=A, pl=A, G=1, S=2, Hq=12, Hkv=2, B=16, W=5, PP=0,
             MP=1, po=A, plse=A, dt=0):
        return f(out, A, A, A, kn, vn, None, A, A, cu, pl, G, S, Hq, Hkv, 128, B, W, 64, 0.088,
                 PP, MP, po, plse, dt, None)

    assert call(cu=None) == EINVAL
    assert call(pl=None) == EINVAL
    assert call(G=0) == EINVAL
    assert call(G=3) == EINVAL                  # more groups than sequences
    assert call(kn=A) == EINVAL                 # k_new without v_new
    assert call(out=None) == EINVAL
    assert call(PP=24, MP=4) == EINVAL          # prefix partition not a multiple of 16
    assert call(PP=16, MP=4) == EWORKSPACE      # 80 positions need 5 partitions of 16
    assert call(PP=16, MP=5, po=None) == EWORKSPACE
    assert call(Hq=34) == ENOTSUP               # group of 17 query heads
    assert call(B=8) == ENOTSUP
    assert call(cu=P((1 << 20) + 2)) == EINVAL  # misaligned group offsets
    assert call(S=0, G=1) == 0                  # nothing to do


@host_only
def test_prefix_split_decode_argument_errors(lib):
    f = lib.paged_attention_prefix_split_decode

    def call(out=A, cu=A, pl=A, G=1, S=2, Hq=12, Hkv=2, B=16, W=5, PP=16, SP=16, MP=10, po=A,
             plse=A, ctr=A, dt=0):
        return f(out, A, A, A, None, None, None, A, A, cu, pl, G, S, Hq, Hkv, 128, B, W, 64,
                 0.088, PP, SP, MP, po, plse, ctr, dt, None)

    assert call(ctr=None) == EINVAL
    assert call(cu=None) == EINVAL
    assert call(PP=0) == EINVAL               # the suffix is split only in the two-pass form
    assert call(SP=0) == EINVAL
    assert call(SP=24) == EINVAL              # not a multiple of 16
    assert call(MP=9) == EWORKSPACE           # 80 positions: 5 prefix + 5 suffix partitions
    assert call(out=None) == EINVAL
    assert call(Hq=34) == ENOTSUP
    assert call(S=0, G=1) == 0


@host_only
def test_slotted_argument_errors(lib):
    f = lib.paged_attention_decode_slotted

    def call(out=A, sg=A, ns=A, S=2, Hq=12, Hkv=2, B=16, MS=4, NB=64, scale=0.088, dt=0):
        return f(out, A, A, A, sg, ns, S, Hq, Hkv, 128, B, MS, NB, scale, dt, None)

    assert call(sg=None) == EINVAL
    assert call(ns=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(MS=0) == EINVAL
    assert call(Hq=12, Hkv=5) == EINVAL
    assert call(Hq=34) == ENOTSUP
    assert call(B=24) == ENOTSUP
    assert call(dt=2) == ENOTSUP
    assert call(scale=float("inf")) == EINVAL
    assert call(sg=P((1 << 20) + 2)) == EINVAL
    assert call(S=0) == 0


@host_only
def test_append_decode_slotted_argument_errors(lib):
    f = lib.paged_attention_append_decode_slotted

    def call(out=A, kn=A, vn=A, so=None, sg=A, S=2, Hq=12, Hkv=2, B=16, MS=4, dt=0):
        return f(out, A, A, A, kn, vn, so, sg, A, S, Hq, Hkv, 128, B, MS, 64, 0.088, dt, None)

    assert call(kn=None, vn=None) == EINVAL          # the new rows are required
    assert call(vn=None) == EINVAL                   # k_new without v_new
    assert call(kn=P((1 << 20) + 8)) == EINVAL       # k_new not 16-byte aligned
    assert call(so=P((1 << 20) + 4)) == EINVAL       # slot_out not 8-byte aligned
    assert call(sg=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(Hq=34) == ENOTSUP
    assert call(B=24) == ENOTSUP
    assert call(dt=2) == ENOTSUP
    assert call(S=0) == 0


@host_only
def test_append_decode_slotted_split_argument_errors(lib):
    f = lib.paged_attention_append_decode_slotted_split

    def call(kn=A, vn=A, so=None, P_=32, MP=2, ctr=A, dt=0):
        return f(A, A, A, A, kn, vn, so, A, A, 2, 12, 2, 128, 16, 4, 64, 0.088, P_, MP, A, A,
                 ctr, dt, None)

    assert call(kn=None, vn=None) == EINVAL          # the new rows are required
    assert call(vn=None) == EINVAL
    assert call(P_=0) == EINVAL                      # split mode only
    assert call(P_=24) == EINVAL                     # not a multiple of 16
    assert call(so=P((1 << 20) + 4)) == EINVAL       # slot_out not 8-byte aligned
    assert call(ctr=None) == EINVAL
    assert call(MP=1) == EWORKSPACE
    assert call(dt=2) == ENOTSUP


@host_only
def test_slotted_split_argument_errors(lib):
    f = lib.paged_attention_decode_slotted_split

    def call(out=A, sg=A, ns=A, S=2, Hq=12, Hkv=2, B=16, MS=4, NB=64, P_=32, MP=2, po=A, pl=A,
             ctr=A, dt=0):
        return f(out, A, A, A, sg, ns, S, Hq, Hkv, 128, B, MS, NB, 0.088, P_, MP, po, pl, ctr,
                 dt, None)

    assert call(P_=0) == EINVAL
    assert call(P_=24) == EINVAL              # not a multiple of 16
    assert call(ctr=None) == EINVAL
    assert call(out=None) == EINVAL
    assert call(MP=1) == EWORKSPACE           # 4 segments x 16 positions need 2 partitions of 32
    assert call(po=None) == EWORKSPACE
    assert call(Hq=34) == ENOTSUP
    assert call(ctr=P((1 << 20) + 2)) == EINVAL
    assert call(S=0) == 0


@host_only
def test_reduce_argument_errors(lib):
    f = lib.paged_attention_reduce
    assert f(None, A, A, A, 2, 12, 128, 32, 3, 0, None) == EINVAL
    assert f(A, A, A, A, 2, 12, 64, 32, 3, 0, None) == ENOTSUP
    assert f(A, A, A, A, 2, 12, 128, 0, 3, 0, None) == EINVAL
    assert f(A, A, A, A, 2, 12, 128, 32, 0, 0, None) == EINVAL
    assert f(A, A, A, A, 2, 12, 128, 32, 3, 5, None) == ENOTSUP
    assert f(A, A, A, A, 0, 12, 128, 32, 3, 0, None) == 0


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(2, 12, 128, dtype=torch.float16)
    with pytest.raises(ValueError):
        pkv.paged_attention_decode(x, x, x.view(1, 2, 16, 96)[:, :, :, :],
                                   x.view(1, 2, 16, 96), torch.zeros(2, 5, dtype=torch.int32),
                                   torch.zeros(2, dtype=torch.int32))


# ---- binding: tensor shapes are checked before the device is touched -----------------
# CPU tensors suffice: every shape or dtype mismatch below is reported before the
# binding's device check, and a consistent call then fails only on that check.
def _t(*shape, dtype="f16"):
    import torch
    dt = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32,
          "i64": torch.int64}[dtype]
    return torch.zeros(shape, dtype=dt)


def _decode_args(S=2, Hq=4, Hkv=2, NB=8, B=16, W=3):
    return dict(out=_t(S, Hq, 128), q=_t(S, Hq, 128), k_pool=_t(NB, Hkv, B, 128),
                v_pool=_t(NB, Hkv, B, 128), block_tables=_t(S, W, dtype="i32"),
                context_lens=_t(S, dtype="i32"))


def test_binding_rejects_mismatched_decode_tensors():
    a = _decode_args()
    with pytest.raises(ValueError, match="GPU"):       # consistent: only the device is wrong
        pkv.paged_attention_decode(**a)
    bad = [
        dict(out=_t(2, 4, 64)),                              # output smaller than q
        dict(v_pool=_t(8, 2, 16, 64)),                       # V pool of another shape
        dict(block_tables=_t(1, 3, dtype="i32")),            # fewer table rows than sequences
        dict(context_lens=_t(3, dtype="i32")),               # one length too many
        dict(q=_t(2, 4, 64), out=_t(2, 4, 64)),              # head_dim unlike the pools
    ]
    for b in bad:
        with pytest.raises(ValueError):
            pkv.paged_attention_decode(**{**a, **b})
    with pytest.raises(TypeError):                       # output dtype unlike the pools
        pkv.paged_attention_decode(**{**a, "out": _t(2, 4, 128, dtype="f32")})


def test_binding_rejects_mismatched_workspace_and_new_rows():
    a = _decode_args()
    a["out"] = None
    with pytest.raises(ValueError):                      # part_lse for fewer partitions
        pkv.paged_attention_decode(**a, partition_size=32, part_o=_t(2, 4, 3, 128, dtype="f32"),
                                   part_lse=_t(2, 4, 2, dtype="f32"))
    with pytest.raises(TypeError):                       # fp16 workspace
        pkv.paged_attention_decode(**a, partition_size=32, part_o=_t(2, 4, 3, 128),
                                   part_lse=_t(2, 4, 3, dtype="f32"))
    a = _decode_args()
    with pytest.raises(ValueError):                      # new rows for one sequence only
        pkv.paged_attention_append_decode(**a, k_new=_t(1, 2, 128), v_new=_t(1, 2, 128))
    with pytest.raises(ValueError):                      # slot output of the wrong length
        pkv.paged_attention_append_decode(**a, k_new=_t(2, 2, 128), v_new=_t(2, 2, 128),
                                          slot_out=_t(3, dtype="i64"))
    with pytest.raises(ValueError):                      # reduce into a smaller output
        pkv.paged_attention_reduce(_t(2, 4, 64), _t(2, 4, 3, 128, dtype="f32"),
                                   _t(2, 4, 3, dtype="f32"), _t(2, dtype="i32"), 32)
    with pytest.raises(ValueError):                      # append: V rows of another shape
        pkv.paged_kv_append(_t(8, 2, 16, 128), _t(8, 2, 16, 128), _t(2, 2, 128),
                            _t(2, 1, 128), _t(2, 3, dtype="i32"), _t(2, dtype="i32"))
    with pytest.raises(ValueError):                      # prefix groups: offsets for 2 groups
        pkv.paged_attention_prefix_decode(**a, group_cu=_t(2, dtype="i32"),
                                          prefix_lens=_t(2, dtype="i32"))
    with pytest.raises(ValueError):                      # slotted: segments for 3 sequences
        pkv.paged_attention_decode_slotted(a["out"], a["q"], a["k_pool"], a["v_pool"],
                                           _t(3, 4, 3, dtype="i32"), _t(2, dtype="i32"))
    with pytest.raises(ValueError):                      # slotted append: no V rows
        pkv.paged_attention_append_decode_slotted(a["out"], a["q"], a["k_pool"], a["v_pool"],
                                                  _t(2, 2, 128), None, _t(2, 4, 3, dtype="i32"),
                                                  _t(2, dtype="i32"))
    with pytest.raises(ValueError):                      # slotted append: rows of one sequence
        pkv.paged_attention_append_decode_slotted(a["out"], a["q"], a["k_pool"], a["v_pool"],
                                                  _t(1, 2, 128), _t(1, 2, 128),
                                                  _t(2, 4, 3, dtype="i32"), _t(2, dtype="i32"))
