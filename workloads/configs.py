"""The five synthetic workload shapes of the paged decode step.

Shapes come from the model descriptions on the source pages:

* the 1.1B edge model of the page "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量
  PagedAttention 与 KV 缓存分块" (pwwt.cn), section "KV Cache 的物理膨胀账本":
  24 layers, 12 query heads, 2 KV heads, head_dim 1536/12 = 128, fp16, and its
  section "嵌入式轻量 Block 分配器设计": 16 tokens per block;
* the Llama-2-7B shape of the hnwysp.cn KV-Cache/BlockManager page, §3.3
  (head_dim 128, 32 heads, fp16, block_size 32, pool sized
  (max_num_seqs x max_blocks_per_seq + 15 %) blocks) and §3.1 (P90 length 287,
  128 concurrent sequences, about six blocks per sequence);
* the prefix-sharing tables of the pwwt.cn page, section "共享前缀块" (a
  256-token system prompt held in shared blocks that every session's table points
  at) and the fork/Copy-on-Write figure of the page "显存虚拟化革命：PagedAttention
  内存池管理与显存碎片终结" (blog.llmgo.top), section 四.

Lengths are the attended length n of the decode step, counting the token that is
appended in the same step (it sits at logical position n-1).  Config 1 also has a
"b" variant where the listed numbers are the history length, so n is one larger;
that variant exercises the "block full -> fresh block, offset 0" path of the
sequence diagram in section 三 of the blog.llmgo.top page.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    key: str                 # short name used by tests and the benchmark
    cfg_id: int              # seed namespace, 1..5
    title: str
    num_seqs: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str               # "fp16" or "bf16"
    max_blocks_per_seq: int  # width W of the block-table rows
    value_scale: float       # Q/K/V ~ N(0,1) * value_scale
    length_kind: str         # "fixed", "uniform", "lognormal", "prefix"
    fixed_lengths: Tuple[int, ...] = ()
    uniform_lo: int = 0
    uniform_hi: int = 0
    lognormal_mu: float = 0.0
    lognormal_sigma: float = 0.0
    clip_lo: int = 1
    clip_hi: int = 1 << 30
    prefix_tokens: int = 0           # shared prefix length (prefix configs)
    pool_blocks: Optional[int] = None  # None -> derived from lengths
    pool_slack: float = 1.15          # pool = ceil(blocks needed * slack)
    # distinct layer data sets the benchmark cycles through so that the
    # cycled working set is well above the 256 MB last-level cache
    bench_distinct_layers: int = 1
    bench_partition_size: int = 0
    bench_prefix_partition: int = 0  # prefix partition of the shared-prefix path
    notes: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2

    @property
    def max_context(self) -> int:
        return self.max_blocks_per_seq * self.block_size

    def blocks_for(self, n: int) -> int:
        return -(-n // self.block_size)


CONFIGS = {
    "c1a": Config(
        key="c1a", cfg_id=1, title="tiny paged decode (lengths count the new token)",
        num_seqs=4, num_layers=1, num_q_heads=12, num_kv_heads=2, head_dim=128,
        block_size=16, dtype="fp16", max_blocks_per_seq=5, value_scale=1.0,
        length_kind="fixed", fixed_lengths=(5, 16, 37, 64), pool_blocks=64,
    ),
    "c1b": Config(
        key="c1b", cfg_id=1, title="tiny paged decode (lengths are history; +1 new token)",
        num_seqs=4, num_layers=1, num_q_heads=12, num_kv_heads=2, head_dim=128,
        block_size=16, dtype="fp16", max_blocks_per_seq=5, value_scale=1.0,
        length_kind="fixed", fixed_lengths=(6, 17, 38, 65), pool_blocks=64,
    ),
    "c2": Config(
        key="c2", cfg_id=2, title="edge SLM shape, 24 layers, GQA 6:1",
        num_seqs=32, num_layers=24, num_q_heads=12, num_kv_heads=2, head_dim=128,
        block_size=16, dtype="fp16", max_blocks_per_seq=128, value_scale=1.0,
        length_kind="uniform", uniform_lo=16, uniform_hi=2048, pool_blocks=4096,
        bench_distinct_layers=24, bench_partition_size=512,
    ),
    "c3": Config(
        key="c3", cfg_id=3, title="Llama-2-7B attention shape, 32 layers, MHA",
        num_seqs=128, num_layers=32, num_q_heads=32, num_kv_heads=32, head_dim=128,
        block_size=32, dtype="fp16", max_blocks_per_seq=128, value_scale=0.5,
        length_kind="lognormal",
        # P90 = 287 with sigma 0.5: mu = ln 287 - z_0.9 * 0.5
        lognormal_mu=math.log(287.0) - 1.2815515655446004 * 0.5,
        lognormal_sigma=0.5, clip_lo=1, clip_hi=4096,
        pool_blocks=math.ceil(128 * 128 * 1.15),
        bench_distinct_layers=8, bench_partition_size=0,
    ),
    "c4": Config(
        key="c4", cfg_id=4, title="long context split-partition, bf16",
        num_seqs=8, num_layers=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=128, dtype="bf16", max_blocks_per_seq=128, value_scale=1.0,
        length_kind="fixed", fixed_lengths=(16384,) * 8,
        pool_blocks=math.ceil(8 * 128 * 1.15),
        bench_distinct_layers=2, bench_partition_size=2048,
    ),
    "c5": Config(
        key="c5", cfg_id=5, title="prefix-sharing tables, 512-token shared prefix",
        num_seqs=256, num_layers=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
        block_size=16, dtype="fp16", max_blocks_per_seq=40, value_scale=1.0,
        length_kind="prefix", prefix_tokens=512, uniform_lo=5, uniform_hi=128,
        pool_blocks=None, bench_distinct_layers=8, bench_partition_size=0,
    ),
}


def get_config(key: str) -> Config:
    try:
        return CONFIGS[key]
    except KeyError:
        raise KeyError(f"unknown workload {key!r}; known: {sorted(CONFIGS)}") from None
