/*
 * paged_kv.h -- C ABI of the MI355X (gfx950) paged KV-cache decode library
 * (libpagedkv.so).
 *
 * The library implements the decode-step hot path of PagedAttention: the KV cache
 * of every sequence lives in fixed-size physical blocks of one pre-allocated pool,
 * and a per-sequence block table maps logical block i to a physical block id
 * (page "显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结", blog.llmgo.top,
 * §二.1 and §三.1; page "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量
 * PagedAttention 与 KV 缓存分块", pwwt.cn, section "注意力寻址").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory. Every pointer argument except `stream` is a DEVICE pointer, allocated
 *   and owned by the caller.  The library allocates nothing and keeps no state
 *   between calls; calls on different streams are independent.
 * Asynchrony. Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *   stream) and the call returns without synchronising.  The return value only
 *   reports argument errors and launch failures.
 * Data types. `dtype` is PKV_FP16 (IEEE binary16) or PKV_BF16 (bfloat16) and
 *   applies to the pools, q, the new K/V rows and the output.  Arithmetic is
 *   fp32; outputs are rounded to `dtype` with round-to-nearest-even.
 * Pool layout. One K pool and one V pool per layer, each
 *     [num_blocks][num_kv_heads][block_size][head_dim]
 *   row-major with head_dim contiguous, 16-byte aligned.  Token t of a sequence
 *   lives in physical block table[t / block_size] at offset t % block_size.
 * Block tables. int32 [num_seqs][max_blocks_per_seq], row-major (the flat 2-D
 *   int32 tensor of the kernel sketch in §五.1 of the blog.llmgo.top page).  Only
 *   entries of blocks that hold tokens are read; other entries may be anything
 *   (-1 is conventional).
 * Context lengths. int32 [num_seqs]: n = the number of tokens the step attends
 *   to, INCLUDING the token appended in the same step (it sits at position n-1).
 *   n = 0 marks a padding sequence.
 * Caller contract (not checked unless PKV_DEBUG_CHECK=1 is set in the
 *   environment): 0 <= n <= max_blocks_per_seq * block_size; table entries of
 *   blocks 0 .. ceil(n/block_size)-1 lie in [0, num_blocks).  With
 *   PKV_DEBUG_CHECK=1 each call first runs a device-side check of these,
 *   synchronises `stream`, and returns PKV_EDEVICE if one fails.  Also the
 *   caller's, and never checked: no two sequences append to the same slot in one
 *   call (the row left in the slot is then either sequence's).  The check keeps
 *   its verdict in one flag per device:
 *   checked calls that run at the same time on one device (from several threads)
 *   may report each other's violations.
 * Supported shapes: head_dim = 128; block_size in {16, 32, 64, 128, 256};
 *   num_q_heads a multiple of num_kv_heads with a group of at most 16 query
 *   heads per KV head.  Others give PKV_ENOTSUP.
 * Softmax scale. Every attention entry point takes `scale`, the factor applied
 *   to q.k before the softmax.  A NaN (PKV_DEFAULT_SCALE) selects the usual
 *   1/sqrt(head_dim); an infinite scale gives PKV_EINVAL.  0 is valid (every
 *   score is then equal: the output is the mean of the attended V rows).
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PKV_OK 0
#define PKV_EINVAL (-1)     /* null pointer, non-positive size, bad ratio or alignment */
#define PKV_ENOTSUP (-2)    /* valid but unsupported shape or dtype */
#define PKV_EWORKSPACE (-3) /* partition workspace missing or too small */
#define PKV_ELAUNCH (-4)    /* the HIP runtime rejected a kernel launch */
#define PKV_EDEVICE (-5)    /* PKV_DEBUG_CHECK found a caller-contract violation */

/* storage formats */
#define PKV_FP16 0
#define PKV_BF16 1

/* `scale` argument that selects 1/sqrt(head_dim) */
#define PKV_DEFAULT_SCALE (__builtin_nanf(""))

/* Human-readable text of a status code (static storage). */
const char *pkv_status_string(int status);

/*
 * paged_kv_append -- the cache-append scatter of one decode step.
 *
 * For each sequence s with n = context_lens[s] >= 1, writes the new token's rows
 * k_new[s][h][:] and v_new[s][h][:] (all heads h) to position t = n-1, i.e. to
 * offset t % block_size of physical block block_tables[s][t / block_size] of
 * k_pool / v_pool.  A token that opens a new block lands at offset 0 of the block
 * the host has just appended to the table (blog.llmgo.top page, §三, sequence
 * diagram; hnwysp.cn KV-Cache/BlockManager page, §4.5, write_kv).  Bit copy.
 *
 *   k_pool, v_pool  [num_blocks][num_kv_heads][block_size][head_dim], written
 *   k_new, v_new    [num_seqs][num_kv_heads][head_dim]
 *   slot_out        optional (may be NULL), int64 [num_seqs]: receives
 *                   phys * block_size + offset, or -1 when n == 0
 * Sequences with n == 0 write nothing.
 */
int paged_kv_append(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                    const int32_t *block_tables, const int32_t *context_lens, int64_t *slot_out,
                    int num_seqs, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream);

/*
 * paged_kv_append_tokens -- scatter runs of consecutive tokens (a prompt, a
 * prefill chunk, or any history) into their blocks.
 *
 * Run r writes rows src_cu[r] .. src_cu[r+1]-1 of k_src / v_src to logical
 * positions start_pos[r], start_pos[r]+1, ... of table row r (a 38-token prompt
 * written to blocks [7, 3, 12] leaves block 12 holding 6 tokens: blog.llmgo.top
 * page, §三).  Bit copy with the same walk as paged_kv_append.
 *
 *   k_src, v_src   [total_tokens][num_kv_heads][head_dim]
 *   src_cu         int64 [num_runs + 1], src_cu[0] = 0, non-decreasing,
 *                  src_cu[num_runs] = total_tokens (host value passed as well)
 *   start_pos      int32 [num_runs], >= 0
 *   block_tables   int32 [num_runs][max_blocks_per_seq]
 * Positions past max_blocks_per_seq * block_size are a caller error.
 */
int paged_kv_append_tokens(void *k_pool, void *v_pool, const void *k_src, const void *v_src,
                           const int64_t *src_cu, const int32_t *start_pos,
                           const int32_t *block_tables, int num_runs, int64_t total_tokens,
                           int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream);

/*
 * paged_kv_copy_blocks -- copy-on-write duplication of whole blocks.
 *
 * For each pair i, physical block dst_blocks[i] of every layer's K pool and V
 * pool becomes a bit copy of block src_blocks[i] as it was before the call.  This
 * is the deep copy the block manager orders when a branch is about to append to
 * a partly filled block that another branch still references: the copy goes to a
 * fresh block, the appending branch's table entry is then pointed at it, and the
 * append writes into the copy (blog.llmgo.top page, §四, copy-on-write steps
 * 1-3).  A block id names the same block in every layer, hence the layer list.
 * The library changes no table and keeps no reference counts: the caller does.
 *
 *   k_pools, v_pools  HOST arrays of num_layers DEVICE pointers, each a pool
 *                     [num_blocks][num_kv_heads][block_size][head_dim] (16-byte
 *                     aligned); 1 <= num_layers <= 128, else PKV_EINVAL / ENOTSUP
 *   src_blocks, dst_blocks  DEVICE int32 [num_pairs]
 * Caller contract (checked only with PKV_DEBUG_CHECK=1, else undefined): every
 * id in [0, num_blocks); no destination appears twice or as any pair's source (a
 * source may be copied to several destinations, e.g. one prompt forked into
 * several samples).  num_pairs == 0 does nothing.
 */
int paged_kv_copy_blocks(void *const *k_pools, void *const *v_pools, int num_layers,
                         const int32_t *src_blocks, const int32_t *dst_blocks, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         int dtype, void *stream);

/*
 * paged_kv_copy_slots -- copy-on-write split of nodes held in shared slots.
 *
 * Radix-tree caches pack short nodes as slots of shared blocks (see
 * paged_attention_decode_slotted).  When such a node is about to be appended to,
 * it is split off into a block of its own, so the shared slots stay read-only and
 * the write cannot touch them (mhpq.cn Radix-Tree page, "核心设计原则",
 * copy-on-write on append): its rows move to the new block, usually at offset 0,
 * and the append then continues in place there.  For each copy i, rows
 * src_offset .. src_offset+length-1 of block src_block become rows dst_offset ..
 * dst_offset+length-1 of block dst_block, in every KV head of every layer's K and
 * V pool, as they were before the call; every other row is left as it was.  The
 * library changes no segment list: the caller repoints the node.
 *
 *   k_pools, v_pools  HOST arrays of num_layers DEVICE pool pointers, as for
 *                     paged_kv_copy_blocks (1 <= num_layers <= 128)
 *   copies            DEVICE int32 [num_copies][5]: (src_block, src_offset,
 *                     dst_block, dst_offset, length)
 * Caller contract (checked only with PKV_DEBUG_CHECK=1): blocks in
 * [0, num_blocks); offsets and length >= 0 with offset + length <= block_size
 * (the kernel clamps the rows to the block in any case); no destination row is
 * a source row of any copy or a destination row of another copy.
 * num_copies == 0 does nothing.
 */
int paged_kv_copy_slots(void *const *k_pools, void *const *v_pools, int num_layers,
                        const int32_t *copies, int num_copies, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int dtype, void *stream);

/*
 * paged_attention_decode -- decode attention over the paged pools.
 *
 * For every sequence s and query head h (KV head g = h / (num_q_heads /
 * num_kv_heads)):  out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t) V_t over the
 * logical tokens t = 0 .. n-1, each fetched through the block table (the kernel
 * sketch of §五.1 of the blog.llmgo.top page: loop over logical blocks, look up
 * the physical block, load its K/V tile, accumulate QK^T with a running softmax,
 * normalise, store).  The result equals ordinary attention over the contiguous
 * logical sequence.
 *
 *   out            [num_seqs][num_q_heads][head_dim], dtype (single-pass mode)
 *   q              [num_seqs][num_q_heads][head_dim], dtype
 *   scale          softmax scale (NaN: 1/sqrt(head_dim))
 *   partition_size 0: single pass, each (sequence, KV head) is handled whole and
 *                  `out` is written; part_o/part_lse/max_partitions are ignored.
 *                  > 0: split-context mode; must be a multiple of block_size
 *                  (else PKV_EINVAL).  Partition p covers tokens [p*P, min(n, (p+1)*P)) and
 *                  writes part_o[s][h][p][:] (fp32, that partition's normalised
 *                  attention output) and part_lse[s][h][p] (fp32, natural-log
 *                  log-sum-exp of the partition's scaled scores).  Partitions
 *                  p >= ceil(n/P) are not written, and `out` is not touched:
 *                  call paged_attention_reduce afterwards.
 *   max_partitions row stride of the workspace; must be at least
 *                  ceil(max_blocks_per_seq * block_size / partition_size),
 *                  else PKV_EWORKSPACE.
 *   part_o         fp32 [num_seqs][num_q_heads][max_partitions][head_dim]
 *   part_lse       fp32 [num_seqs][num_q_heads][max_partitions]
 * n == 0 gives an all-zero output row in single-pass mode.
 */
int paged_attention_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int max_blocks_per_seq, int64_t num_blocks,
                           float scale, int partition_size, int max_partitions, float *part_o,
                           float *part_lse, int dtype, void *stream);

/*
 * paged_attention_append_decode -- the step's cache-append scatter and decode
 * attention in one launch.
 *
 * Same result as paged_kv_append(k_pool, v_pool, k_new, v_new, block_tables,
 * context_lens, slot_out, ...) followed by paged_attention_decode(...) with the
 * same arguments: the new rows end up in the pools bit for bit, and attention
 * covers positions 0 .. n-1 with position n-1 being the new token.  The work-group
 * that handles position n-1 of (sequence, KV head) writes the new rows to their
 * slot and uses them from registers, so the slot is never read before it is
 * written.  Fusing removes one launch and its dependent-latency chain per layer.
 *
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim], required (non-NULL)
 *   slot_out       optional int64 [num_seqs] as for paged_kv_append
 * Other arguments and the split-context mode are as for paged_attention_decode
 * (in split mode the append is done by the partition holding position n-1).
 */
int paged_attention_append_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                  const void *k_new, const void *v_new, int64_t *slot_out,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int64_t num_blocks,
                                  float scale, int partition_size, int max_partitions,
                                  float *part_o, float *part_lse, int dtype, void *stream);

/*
 * paged_attention_split_decode -- split-context decode whose partitions are
 * merged in the same launch.
 *
 * Same result as paged_attention_decode (or, with k_new / v_new, as
 * paged_attention_append_decode) in split-context mode followed by
 * paged_attention_reduce, with `out` written by this one launch: partition p of
 * (sequence s, KV head g) covers tokens [p*P, min(n, (p+1)*P)), each of the
 * item's work-groups writes its partitions' fp32 partials to the workspace and
 * counts itself in counters[s][g]; the last one to arrive merges the item's
 * partials by the log-sum-exp rule of paged_attention_reduce (the same
 * operations, so the same bits) and puts the counter back to 0.  A context of at
 * most one partition (n <= P) is written to `out` directly, without partials.
 * The pages describe no partitioning; the merge is the exact identity of
 * paged_attention_reduce.
 *
 *   out            [num_seqs][num_q_heads][head_dim], dtype, required
 *   k_new, v_new   optional (both or neither): append the step's new rows as
 *                  paged_attention_append_decode does; slot_out only with them
 *   partition_size > 0, a multiple of block_size
 *   max_partitions, part_o, part_lse   the workspace, as for
 *                  paged_attention_decode, at most 2^31 - 1 bytes of part_o
 *                  (else PKV_EWORKSPACE); its contents afterwards are
 *                  unspecified
 *   counters       device int32 [num_seqs][num_kv_heads], ALL ZERO when the call
 *                  starts; every call that completes leaves them zero, so one
 *                  zero-filled array serves any number of consecutive calls
 *                  (and graph replays).  Calls that run at the same time must
 *                  use different counters and workspaces.
 */
int paged_attention_split_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                 const void *k_new, const void *v_new, int64_t *slot_out,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int64_t num_blocks,
                                 float scale, int partition_size, int max_partitions,
                                 float *part_o, float *part_lse, int32_t *counters, int dtype,
                                 void *stream);

/*
 * paged_attention_decode_ordered -- the single-pass decode (with the append
 * fused when k_new / v_new are given) with a caller-chosen dispatch order.
 *
 * Work items are one per (sequence, KV head), launched in grid order; the
 * sequences of a batch are otherwise dispatched in batch order, so a long
 * sequence near the end of the batch finishes last and the launch waits for it.
 * A caller that keeps its lengths on the host (any serving engine does) can put
 * the longest sequences first: the work items of sequence seq_order[i] take the
 * place of sequence i's.  The output, pools and slots are the same, bit for bit,
 * for every order (each item's arithmetic does not depend on where it runs).
 * The address walk and attention are those of paged_attention_decode
 * ("显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结", blog.llmgo.top, §五.1).
 *
 *   seq_order      device int32 [num_seqs], 4-byte aligned, a permutation of
 *                  0 .. num_seqs-1 (entries are clamped to that range on the
 *                  device; PKV_DEBUG_CHECK=1 rejects any entry out of range or
 *                  repeated with PKV_EDEVICE).  Null gives PKV_EINVAL.
 *   k_new, v_new   optional, both or neither (PKV_EINVAL otherwise): the fused
 *                  append of paged_attention_append_decode, with slot_out
 *   out            [num_seqs][num_q_heads][head_dim], dtype; required
 * Other arguments, layouts and errors as for paged_attention_append_decode in
 * single-pass mode (partition_size 0).
 */
int paged_attention_decode_ordered(void *out, const void *q, void *k_pool, void *v_pool,
                                   const void *k_new, const void *v_new, int64_t *slot_out,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   const int32_t *seq_order, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int max_blocks_per_seq, int64_t num_blocks, float scale,
                                   int dtype, void *stream);

/*
 * paged_attention_split_decode_noalloc -- paged_attention_split_decode with no
 * workspace argument and no allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).
 *
 * Same arguments and result as paged_attention_split_decode without
 * max_partitions, part_o, part_lse and counters: the partials and the arrival
 * counters live in a fixed device array inside the library (16.4 MiB per GPU,
 * held until the process ends), with max_partitions =
 * ceil(max_blocks_per_seq * block_size / partition_size).  Limits: num_seqs *
 * num_kv_heads <= 65536 and num_seqs * num_q_heads * max_partitions <= 32768
 * (16 MiB of fp32 partial rows); larger calls return PKV_EWORKSPACE.  The call
 * allocates nothing: the first call on a device resolves that device's copy of
 * the array (hipGetSymbolAddress, with the device current) and clears its
 * counters with a kernel on `stream`; later calls only launch the decode.
 * `stream` must belong to the current device.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give undefined results.
 */
int paged_attention_split_decode_noalloc(void *out, const void *q, void *k_pool, void *v_pool,
                                         const void *k_new, const void *v_new,
                                         int64_t *slot_out, const int32_t *block_tables,
                                         const int32_t *context_lens, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_blocks_per_seq,
                                         int64_t num_blocks, float scale, int partition_size,
                                         int dtype, void *stream);

/*
 * paged_attention_prefix_decode -- decode attention for batches whose sequences
 * share a prefix, reading each shared block once per tile of sequences.
 *
 * Sequences group_cu[k] .. group_cu[k+1]-1 form group k and share the K/V of
 * their first prefix_lens[k] positions: their tables point at the same physical
 * blocks there (a system prompt cached once in blocks every session's table
 * points at: pwwt.cn page, section "共享前缀块（Prefix Caching）"; forked branches
 * reading blocks with reference count > 1: blog.llmgo.top page, §四).  The result
 * is the same as paged_attention_decode (or, with k_new / v_new, as
 * paged_attention_append_decode) on the same tables; only the reads differ.
 *
 * prefix_partition == 0: one launch.  A work-group takes a 16-row query tile
 *   made of the query heads of floor(16/G) consecutive member sequences (G =
 *   num_q_heads / num_kv_heads) and one KV head; it streams the group's prefix
 *   (read through the table row of sequence group_cu[k]) with every member's
 *   rows active, then each member's own positions prefix_lens[k] .. n-1 with
 *   only that member's rows active, appends the new tokens when k_new is given,
 *   and writes `out`.  The workspace is not used (part_o / part_lse may be NULL).
 * prefix_partition > 0: two launches, for prefixes long enough to need more
 *   parallelism than tiles x KV heads:
 *   1. prefix pass: the same tiles over partitions of prefix_partition tokens of
 *      the prefix; each partition's fp32 partial (normalised o, natural-log lse)
 *      goes to part_o[s][h][p] / part_lse[s][h][p];
 *   2. suffix pass: each (sequence, KV head) attends over positions
 *      prefix_lens[k] .. n-1 (with the optional append), merges that with the
 *      prefix partials by the log-sum-exp rule and writes `out`.
 *
 *   group_cu       device int32 [num_groups + 1]: 0 = group_cu[0] <= ... <=
 *                  group_cu[num_groups] = num_seqs (groups are contiguous)
 *   prefix_lens    device int32 [num_groups], >= 0 (0: the group shares nothing)
 *   k_new, v_new   optional (both or neither), as for paged_attention_append_decode;
 *                  slot_out is used only with them
 *   prefix_partition  0 or a multiple of 16
 *   max_partitions    (prefix_partition > 0) row stride of the workspace, at least
 *                  ceil(max_blocks_per_seq * block_size / prefix_partition),
 *                  else PKV_EWORKSPACE
 *   part_o, part_lse  (prefix_partition > 0) fp32 workspace
 *                  [num_seqs][num_q_heads][max_partitions][head_dim] and
 *                  [num_seqs][num_q_heads][max_partitions]
 *   out            [num_seqs][num_q_heads][head_dim], dtype
 * Caller contract (checked with PKV_DEBUG_CHECK=1 like the other entry points):
 * every member's table agrees with the first member's on the blocks holding the
 * prefix, and n >= prefix_lens[k] for every member (n > prefix_lens[k] when
 * appending, so the new token never lands in a shared block).  Unlike
 * paged_attention_decode, positions below a sequence's prefix length that share
 * a 16-position tile with its own positions are read (and masked), so they must
 * hold finite values -- they do whenever the table is valid for the prefix.
 */
int paged_attention_prefix_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                  const void *k_new, const void *v_new, int64_t *slot_out,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *group_cu, const int32_t *prefix_lens,
                                  int num_groups, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int prefix_partition, int max_partitions, float *part_o,
                                  float *part_lse, int dtype, void *stream);

/*
 * paged_attention_prefix_split_decode -- the two-pass shared-prefix decode with
 * its second pass in split-context mode, for members whose own positions are
 * long.
 *
 * Same result as paged_attention_prefix_decode with prefix_partition > 0: pass 1
 * writes each group's prefix partitions (prefix_partition tokens each) to the
 * workspace; pass 2 cuts each member's own positions -- from the last multiple
 * of 16 at or below its prefix length to n-1 -- into partitions of
 * suffix_partition tokens spread over several work-groups per (sequence, KV
 * head), keeps their partials after the prefix partials in the same workspace
 * row, and the last work-group of each (sequence, KV head) merges prefix and
 * suffix partials as paged_attention_split_decode does (arrival counters; a
 * suffix of at most one partition is merged by its own work-group).
 *
 *   prefix_partition, suffix_partition  > 0, multiples of 16
 *   max_partitions  row stride of the workspace, at least
 *                   ceil(ctx / prefix_partition) + ceil(ctx / suffix_partition)
 *                   with ctx = max_blocks_per_seq * block_size, else
 *                   PKV_EWORKSPACE; at most 2^31 - 1 bytes of part_o
 *   counters        device int32 [num_seqs][num_kv_heads], all zero when the call
 *                   starts and left zero, as for paged_attention_split_decode
 * Other arguments and the caller contract as for paged_attention_prefix_decode.
 */
int paged_attention_prefix_split_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                        const void *k_new, const void *v_new, int64_t *slot_out,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *group_cu, const int32_t *prefix_lens,
                                        int num_groups, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int max_blocks_per_seq, int64_t num_blocks, float scale,
                                        int prefix_partition, int suffix_partition,
                                        int max_partitions, float *part_o, float *part_lse,
                                        int32_t *counters, int dtype, void *stream);

/*
 * paged_attention_decode_slotted -- decode attention over slotted segments.
 *
 * Radix-tree prefix caches pack short nodes as slots of shared blocks: a node
 * of fewer tokens than a block occupies `length` consecutive positions starting
 * at `slot_offset` of some block, and is addressed by the triple (block_id,
 * slot_offset, length) (mhpq.cn page on Radix-Tree fragmentation, sections
 * "Slotted Block 分槽与微块共享架构" and "核心设计原则").  Here each sequence is
 * the concatenation of its segments; logical token t lies in the segment whose
 * running start s satisfies s <= t < s + length, at in-block offset
 * slot_offset + (t - s), of physical block block_id.  A whole block is the
 * segment (id, 0, block_size), so an ordinary block table is a special case.
 * out[s][h] = softmax(scale * q.K^T) V over those n = sum(length) tokens; n = 0
 * gives zeros.  Single pass; all head-group sizes run on the matrix-core path.
 *
 * Consecutive sequences whose lists begin with the same triples (the shared path
 * of a radix tree) have those rows read once per tile of 2 * floor(16 / G)
 * sequences, whenever a tile's sub-tile list fits the kernel's LDS
 * (2 * floor(16 / G) * max_segments * ceil(block_size / 16) <= 1024) and the
 * tiles still give at least half of min(num_seqs * num_kv_heads, compute units)
 * work-groups; otherwise one work-group per (sequence, KV head).  The
 * environment variable PKV_SLOTTED_TILES=1 takes the tiles whenever the list
 * fits, PKV_SLOTTED_TILES=0 never.  Both give the same attention up to summation
 * order.
 *
 *   segments       device int32 [num_seqs][max_segments][3]: (block_id,
 *                  slot_offset, length); only the first num_segments[s] are read
 *   num_segments   device int32 [num_seqs], 0 .. max_segments
 *   out, q         as for paged_attention_decode
 * Caller contract (checked with PKV_DEBUG_CHECK=1): block_id in [0, num_blocks),
 * slot_offset >= 0, length >= 0, slot_offset + length <= block_size.  Rows of a
 * block outside a sequence's segments are never read.
 */
int paged_attention_decode_slotted(void *out, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *segments,
                                   const int32_t *num_segments, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int max_segments, int64_t num_blocks, float scale, int dtype,
                                   void *stream);

/*
 * paged_attention_append_decode_slotted -- the step's cache append fused into the
 * slotted decode: each sequence's new K/V row is written to its position n-1 and
 * then attended to with the rest, in one launch.
 *
 * The lengths of a sequence's segments count its new token, as block-table
 * lengths do (n = the sum of its segment lengths, clamped to their blocks):
 * position n-1 is the last row of its last non-empty segment, and the new rows
 * k_new[s] / v_new[s] are written there for every KV head, bit for bit.  That
 * row must be the node's own slot: a node held in a shared slot is split into a
 * block of its own first (paged_kv_copy_slots), since an append must not touch
 * the shared slots ("碎片化的双重绞杀…" mhpq.cn Radix-Tree page, "核心设计原则";
 * the append at the sequence's current position: blog.llmgo.top PagedAttention
 * page, §三).  Attention is that of paged_attention_decode_slotted.
 *
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim], dtype, 16-byte aligned;
 *                  required (PKV_EINVAL otherwise)
 *   slot_out       optional int64 [num_seqs], 8-byte aligned: block * block_size +
 *                  offset of the written row, -1 for a sequence with n = 0
 *                  (nothing written)
 * Other arguments, limits and errors as for paged_attention_decode_slotted
 * (PKV_DEBUG_CHECK=1 validates the segments as there).  Two sequences whose
 * position n-1 is the same slot are a caller error: the row written is then
 * either's.
 */
int paged_attention_append_decode_slotted(void *out, const void *q, void *k_pool, void *v_pool,
                                          const void *k_new, const void *v_new,
                                          int64_t *slot_out, const int32_t *segments,
                                          const int32_t *num_segments, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int max_segments, int64_t num_blocks,
                                          float scale, int dtype, void *stream);

/*
 * paged_attention_decode_slotted_split -- slotted decode in split-context mode,
 * the partitions merged in the same launch.
 *
 * Same result as paged_attention_decode_slotted, for long sequences: each
 * sequence's positions (the concatenation of its segments, n = sum of lengths)
 * are cut into partitions of partition_size positions, partition p covering
 * [p*P, min(n, (p+1)*P)); a segment that straddles a boundary is split between
 * two partitions.  Partitions are spread over several work-groups per
 * (sequence, KV head) and merged as in paged_attention_split_decode (arrival
 * counters, log-sum-exp merge by the last work-group; n <= P is written
 * directly).  Always one work-group per (sequence, KV head, partition group):
 * the tiles of paged_attention_decode_slotted are not used.
 *
 *   partition_size > 0, a multiple of 16
 *   max_partitions row stride of the workspace, at least
 *                  ceil(max_segments * block_size / partition_size), else
 *                  PKV_EWORKSPACE; at most 2^31 - 1 bytes of part_o
 *   part_o, part_lse  fp32 workspace [num_seqs][num_q_heads][max_partitions][head_dim]
 *                  and [num_seqs][num_q_heads][max_partitions]; contents afterwards
 *                  unspecified
 *   counters       device int32 [num_seqs][num_kv_heads], all zero when the call
 *                  starts and left zero, as for paged_attention_split_decode
 * Other arguments as for paged_attention_decode_slotted.
 */
int paged_attention_decode_slotted_split(void *out, const void *q, const void *k_pool,
                                         const void *v_pool, const int32_t *segments,
                                         const int32_t *num_segments, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_segments, int64_t num_blocks,
                                         float scale, int partition_size, int max_partitions,
                                         float *part_o, float *part_lse, int32_t *counters,
                                         int dtype, void *stream);

/*
 * paged_attention_append_decode_slotted_split -- the slotted split decode with
 * the step's append fused: each sequence's new K/V rows are written to its
 * position n-1 (as in paged_attention_append_decode_slotted, the same contract on
 * that row) by the one work-group that reads it, the one whose partitions
 * include the last, before any of its loads; the others never read that row.
 *
 *   k_new, v_new   [num_seqs][num_kv_heads][head_dim], dtype, 16-byte aligned;
 *                  required
 *   slot_out       optional int64 [num_seqs], 8-byte aligned, as for
 *                  paged_attention_append_decode_slotted
 *   partition_size > 0 (PKV_EINVAL otherwise)
 * Other arguments, workspace and counters as for
 * paged_attention_decode_slotted_split.
 */
int paged_attention_append_decode_slotted_split(
    void *out, const void *q, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
    int64_t *slot_out, const int32_t *segments, const int32_t *num_segments, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int max_segments,
    int64_t num_blocks, float scale, int partition_size, int max_partitions, float *part_o,
    float *part_lse, int32_t *counters, int dtype, void *stream);

/*
 * paged_attention_reduce -- log-sum-exp merge of split-context partitions.
 *
 * For each (s, h) with P = partition_size and np = ceil(n/P) partitions:
 *   M = max_p part_lse[s][h][p],  w_p = exp(part_lse[s][h][p] - M),
 *   out[s][h][:] = sum_p w_p part_o[s][h][p][:] / sum_p w_p   (p < np),
 * rounded to dtype; n == 0 gives zeros.  Only partitions p < max_partitions are
 * read (np > max_partitions is a caller error).  Exact in real arithmetic: softmax over
 * a union of token ranges is the lse-weighted mean of the per-range softmaxes
 * (not on the pages; the pages describe no partitioning).
 */
int paged_attention_reduce(void *out, const float *part_o, const float *part_lse,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int head_dim, int partition_size, int max_partitions, int dtype,
                           void *stream);

/* Smallest valid max_partitions for a table width and partition size (0 if the
 * arguments are invalid). */
int pkv_max_partitions(int max_blocks_per_seq, int block_size, int partition_size);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
