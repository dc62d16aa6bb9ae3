"""Host-side dispatch order for paged_attention_decode_ordered.

The ordered decode launches one work-group per (sequence, KV head) in the order
a caller gives, and its results do not depend on that order.  A batch of very
different lengths runs faster when the work-groups that take longest start
first and the shortest start last: the launch then ends on short work instead
of on a long sequence dispatched late.  This module builds that order from the
context lengths the caller already holds on the host.
"""
from typing import Sequence

import numpy as np


def long_first_order(lengths: Sequence[int], num_kv_heads: int, num_cus: int) -> np.ndarray:
    """Sequence indices for `seq_order`: the sequences longer than twice the batch
    mean first (in batch order), then the rest in batch order, except the shortest
    k of them, which go last, longest of those first.  k gives about one
    work-group per compute unit (ceil(num_cus / num_kv_heads)), at most an eighth
    of the batch.  Returns a permutation of 0 .. len(lengths)-1 as int32."""
    n = np.asarray(lengths, np.int64)
    if n.ndim != 1:
        raise ValueError("lengths must be one-dimensional")
    if num_kv_heads <= 0 or num_cus <= 0:
        raise ValueError("num_kv_heads and num_cus must be positive")
    S = int(n.size)
    if S == 0:
        return np.zeros(0, np.int32)
    mean = n.mean()
    longs = [i for i in range(S) if n[i] > 2 * mean]
    rest = [i for i in range(S) if n[i] <= 2 * mean]
    k = min(-(-num_cus // num_kv_heads), S // 8, len(rest))
    # the k shortest (ties by batch index), then longest first among them
    shorts = sorted(sorted(rest, key=lambda i: (n[i], i))[:k], key=lambda i: (-n[i], i))
    short_set = set(shorts)
    mid = [i for i in rest if i not in short_set]
    return np.array(longs + mid + shorts, np.int32)
