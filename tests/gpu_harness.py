"""Drives the HIP path through the C ABI (via the package's binding) on a workload,
and compares against the oracle.  Used by the GPU tests and the smoke check.

Nothing here computes any part of the method: the GPU side runs only library
entry points, the expectations come only from oracle/.
"""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_09_amd as pkv

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def scale_for(head_dim: int) -> float:
    return float(np.float32(1.0 / np.sqrt(head_dim)))


def to_dev(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(TORCH_DT[dtype])


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def widen_out(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def i32(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def i64(a, device):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(device)


class GpuStep:
    """Device state of one layer of a workload: pools filled with the NaN
    sentinel, then history runs and the new token written by the library."""

    def __init__(self, w, device="cuda:0", tables=None, k_pool_bits=None, v_pool_bits=None,
                 append=True):
        c = w.cfg
        self.w, self.c, self.device = w, c, torch.device(device)
        dt = TORCH_DT[c.dtype]
        shape = w.pool_shape()
        self.tables = i32(w.tables if tables is None else tables, self.device)
        self.lens = i32(w.lengths, self.device)
        self.q = to_dev(w.q, c.dtype, self.device)
        if k_pool_bits is not None:
            self.k_pool = to_dev(k_pool_bits, c.dtype, self.device)
            self.v_pool = to_dev(v_pool_bits, c.dtype, self.device)
            self.slots = None
            return
        sentinel = np.array([w.nan_bits], np.uint16).view(np.int16)[0]
        self.k_pool = torch.empty(shape, dtype=dt, device=self.device)
        self.v_pool = torch.empty(shape, dtype=dt, device=self.device)
        self.k_pool.view(torch.int16).fill_(int(sentinel))
        self.v_pool.view(torch.int16).fill_(int(sentinel))
        if w.total_history_tokens() > 0:
            pkv.paged_kv_append_tokens(
                self.k_pool, self.v_pool, to_dev(w.k_src, c.dtype, self.device),
                to_dev(w.v_src, c.dtype, self.device), i64(w.seg_cu, self.device),
                i32(w.seg_start, self.device), i32(w.seg_tables, self.device))
        self.slots = torch.full((c.num_seqs,), -7, dtype=torch.int64, device=self.device)
        self.k_new = to_dev(w.k_new, c.dtype, self.device)
        self.v_new = to_dev(w.v_new, c.dtype, self.device)
        if append:
            pkv.paged_kv_append(self.k_pool, self.v_pool, self.k_new, self.v_new, self.tables,
                                self.lens, self.slots)

    def decode(self, partition_size: int = 0, scale=None, max_parts=None):
        c = self.c
        scale = scale_for(c.head_dim) if scale is None else scale
        out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=TORCH_DT[c.dtype],
                          device=self.device)
        out.view(torch.int16).fill_(0x5555)
        if partition_size == 0:
            pkv.paged_attention_decode(out, self.q, self.k_pool, self.v_pool, self.tables,
                                       self.lens, scale=scale)
            return out, None, None
        mp = max_parts or pkv.max_partitions(c.max_blocks_per_seq, c.block_size, partition_size)
        po = torch.full((c.num_seqs, c.num_q_heads, mp, c.head_dim), float("nan"),
                        dtype=torch.float32, device=self.device)
        pl = torch.full((c.num_seqs, c.num_q_heads, mp), float("nan"), dtype=torch.float32,
                        device=self.device)
        pkv.paged_attention_decode(None, self.q, self.k_pool, self.v_pool, self.tables, self.lens,
                                   scale=scale, partition_size=partition_size, part_o=po,
                                   part_lse=pl)
        pkv.paged_attention_reduce(out, po, pl, self.lens, partition_size)
        return out, po, pl


def fused_step(g: GpuStep, partition_size: int = 0, scale=None):
    """Append + decode in one launch (paged_attention_append_decode) on a GpuStep
    built with append=False; returns the output (merged in split mode)."""
    c = g.c
    scale = scale_for(c.head_dim) if scale is None else scale
    out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=TORCH_DT[c.dtype],
                      device=g.device)
    out.view(torch.int16).fill_(0x5555)
    if partition_size == 0:
        pkv.paged_attention_append_decode(out, g.q, g.k_pool, g.v_pool, g.k_new, g.v_new,
                                          g.tables, g.lens, g.slots, scale=scale)
        return out
    mp = pkv.max_partitions(c.max_blocks_per_seq, c.block_size, partition_size)
    po = torch.full((c.num_seqs, c.num_q_heads, mp, c.head_dim), float("nan"),
                    dtype=torch.float32, device=g.device)
    pl = torch.full((c.num_seqs, c.num_q_heads, mp), float("nan"), dtype=torch.float32,
                    device=g.device)
    pkv.paged_attention_append_decode(None, g.q, g.k_pool, g.v_pool, g.k_new, g.v_new, g.tables,
                                      g.lens, g.slots, scale=scale,
                                      partition_size=partition_size, part_o=po, part_lse=pl)
    pkv.paged_attention_reduce(out, po, pl, g.lens, partition_size)
    return out


def tol_ok(got: np.ndarray, ref: np.ndarray, atol=1e-2, rtol=1e-2):
    err = np.abs(got - ref)
    bad = ~(err <= atol + rtol * np.abs(ref))
    return (not bad.any()), float(np.nanmax(err)) if err.size else 0.0, int(bad.sum())


def merged_step(g: GpuStep, partition_size: int, append: bool = True, scale=None,
                counters=None):
    """paged_attention_split_decode on a GpuStep (built with append=False when
    `append`): split-context decode merged in the same launch.  Returns the
    output and the arrival counters (zero after a completed call)."""
    c = g.c
    scale = scale_for(c.head_dim) if scale is None else scale
    out = torch.empty((c.num_seqs, c.num_q_heads, c.head_dim), dtype=TORCH_DT[c.dtype],
                      device=g.device)
    out.view(torch.int16).fill_(0x5555)
    mp = pkv.max_partitions(c.max_blocks_per_seq, c.block_size, partition_size)
    po = torch.full((c.num_seqs, c.num_q_heads, mp, c.head_dim), float("nan"),
                    dtype=torch.float32, device=g.device)
    pl = torch.full((c.num_seqs, c.num_q_heads, mp), float("nan"), dtype=torch.float32,
                    device=g.device)
    if counters is None:
        counters = torch.zeros((c.num_seqs, c.num_kv_heads), dtype=torch.int32, device=g.device)
    kw = dict(k_new=g.k_new, v_new=g.v_new, slot_out=g.slots) if append else {}
    pkv.paged_attention_split_decode(out, g.q, g.k_pool, g.v_pool, g.tables, g.lens,
                                     partition_size, po, pl, counters, scale=scale, **kw)
    return out, counters
