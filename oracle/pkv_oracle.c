/*
 * pkv_oracle.c -- plain fp64 CPU oracle for the paged KV-cache decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference the HIP kernels are
 * checked against.  Only the test suite, the smoke check of the package entry
 * file and the CPU-baseline leg of the benchmark may load it.  The product path
 * never calls it, and it shares no code, header, table or constant with the HIP
 * sources: every stride and formula below is written out here on its own.
 *
 * What it computes, step by step, and where the pages say so:
 *
 *  - Address walk (page "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量 PagedAttention
 *    与 KV 缓存分块", pwwt.cn, section "注意力寻址"): for logical token T,
 *    block index = T / TOKENS_PER_BLOCK, offset = T % TOKENS_PER_BLOCK,
 *    physical block = block_table[block index].  The same lookup appears in the
 *    kernel sketch of the page "显存虚拟化革命：PagedAttention 内存池管理与显存碎片
 *    终结" (blog.llmgo.top), §五.1, where the table is a flat
 *    [num_seqs][max_num_blocks_per_seq] int32 array.  Block index uses floor
 *    division and the offset must satisfy 0 <= offset < block_size (hnwysp.cn
 *    KV-Cache/BlockManager page, §3.2 and §5.1).
 *  - Pool layout: one pre-allocated K pool and one V pool per layer, cut into
 *    fixed-size blocks (blog.llmgo.top page, §三.1).  Inside a block this oracle
 *    uses [num_kv_heads][block_size][head_dim] with head_dim contiguous; the pages
 *    do not fix the order inside a block for V, and for K only permute elements
 *    inside the same per-(block, head) slab.
 *  - Append: the new token of a decode step is written at (physical block,
 *    offset) of logical position n-1; a full last block means the host has
 *    appended a fresh block and the token lands at offset 0 (blog.llmgo.top page,
 *    §三, sequence diagram).  Bit copy.
 *  - Attention: PagedAttention computes ordinary attention over the sequence's
 *    logical order (blog.llmgo.top page, §二.1 "逻辑块" and §五 intro); this oracle
 *    evaluates softmax(scale * q.K^T) V in fp64 token by token through the walk,
 *    with a two-pass softmax (max, then sum of exp).
 *  - Block copy (copy-on-write): before a branch appends to a partly filled
 *    block that another branch still references, the whole block is duplicated
 *    into a fresh physical block and only the appending branch's table entry is
 *    pointed at the copy (blog.llmgo.top page, §四, steps 1-3 of the
 *    copy-on-write mechanism).  Every element of every head of the block is
 *    copied, in K and in V.
 *  - Slotted blocks: a short radix-tree node is packed as a slot inside a shared
 *    block and addressed by a (block id, slot offset, length) triple (mhpq.cn
 *    page on Radix-Tree fragmentation, sections "Slotted Block 分槽与微块共享架构"
 *    and "核心设计原则").  A sequence's KV is the concatenation of its segments in
 *    order; logical token t lies in the segment whose running start s satisfies
 *    s <= t < s + length, at in-block offset slot_offset + (t - s).
 *  - Slot copy (copy-on-write split of a shared slot): when a node that sits in
 *    a slot of a shared block is appended to, it is split off into a block of
 *    its own, so the shared slots stay read-only and the write cannot touch them
 *    (mhpq.cn page, "核心设计原则", copy-on-write on append).  The node's `length`
 *    rows move from (block, slot offset) to offset 0 of the dedicated block,
 *    every head, in K and in V; the source rows are left as they are.  Written
 *    here for any destination offset.
 *  - Slotted append: a decode step's new token goes to the sequence's last
 *    position n-1, n being the sum of its segment lengths (the lengths count the
 *    new token, as for block tables); the walk over the segments gives its (block,
 *    offset), which must be the node's own slot (a shared one is split first, as
 *    above).  Bit copy, every head, K and V.
 *  - Partials and merge: attention over the token range of one partition, its
 *    log-sum-exp, and the exact log-sum-exp combination of partitions.  The
 *    pages do not describe partitions; the merge is the algebraic identity
 *    softmax over a union = weighted mean of per-part softmaxes with weights
 *    exp(lse_p - max lse).
 *
 * Storage formats: fp16 is IEEE 754 binary16; bf16 is the top half of a binary32.
 * Both are widened to double exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_OK 0
#define OR_EARG (-1)      /* bad scalar argument */
#define OR_ETABLE (-10)   /* table entry outside [0, num_blocks) or past the row */
#define OR_EOFFSET (-11)  /* offset outside [0, block_size) */
#define OR_EDUP (-12)     /* two writes target the same slot */
#define OR_ENOMEM (-13)

#define OR_FP16 0
#define OR_BF16 1

/* ---- storage formats ---------------------------------------------------- */
double oracle_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);  /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double widen(uint16_t bits, int dtype)
{
    return dtype == OR_BF16 ? oracle_bf16_to_double(bits) : oracle_fp16_to_double(bits);
}

/* ---- layout and address walk --------------------------------------------- */
/* Element offset of (physical block, kv head, offset in block, dim) in one pool. */
int64_t oracle_elem_offset(int64_t phys, int64_t h, int64_t off, int64_t d,
                           int64_t num_kv_heads, int64_t block_size, int64_t head_dim)
{
    return ((phys * num_kv_heads + h) * block_size + off) * head_dim + d;
}

/* Walk the table row for logical token t: physical block and in-block offset. */
int oracle_locate(const int32_t *table_row, int64_t max_blocks_per_seq, int64_t block_size,
                  int64_t num_blocks, int64_t t, int64_t *phys, int64_t *off)
{
    if (t < 0 || block_size <= 0)
        return OR_EARG;
    int64_t blk = t / block_size;
    int64_t o = t % block_size;
    if (blk >= max_blocks_per_seq)
        return OR_ETABLE;
    if (!(0 <= o && o < block_size))
        return OR_EOFFSET;
    int64_t p = table_row[blk];
    if (p < 0 || p >= num_blocks)
        return OR_ETABLE;
    *phys = p;
    *off = o;
    return OR_OK;
}

static int check_dims(int64_t num_kv_heads, int64_t head_dim, int64_t block_size,
                      int64_t max_blocks_per_seq, int64_t num_blocks)
{
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return OR_EARG;
    return OR_OK;
}

/* Mark slot phys*B+off in a byte map; a second mark of the same slot is a duplicate. */
static int mark_slot(unsigned char *map, int64_t slot)
{
    if (map[slot])
        return OR_EDUP;
    map[slot] = 1;
    return OR_OK;
}

/* ---- append (one token per sequence, at position n-1) --------------------- */
int oracle_append(uint16_t *k_pool, uint16_t *v_pool, const uint16_t *k_new,
                  const uint16_t *v_new, const int32_t *block_tables, const int32_t *context_lens,
                  int64_t *slot_out, int64_t num_seqs, int64_t num_kv_heads, int64_t head_dim,
                  int64_t block_size, int64_t max_blocks_per_seq, int64_t num_blocks)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks);
    if (rc)
        return rc;
    unsigned char *map = calloc((size_t)(num_blocks * block_size), 1);
    if (!map)
        return OR_ENOMEM;
    for (int64_t s = 0; s < num_seqs && rc == OR_OK; ++s) {
        int64_t n = context_lens[s];
        if (n <= 0) {
            if (slot_out)
                slot_out[s] = -1;
            continue;
        }
        int64_t phys, off;
        rc = oracle_locate(block_tables + s * max_blocks_per_seq, max_blocks_per_seq,
                           block_size, num_blocks, n - 1, &phys, &off);
        if (rc)
            break;
        rc = mark_slot(map, phys * block_size + off);
        if (rc)
            break;
        for (int64_t h = 0; h < num_kv_heads; ++h)
            for (int64_t d = 0; d < head_dim; ++d) {
                int64_t e = oracle_elem_offset(phys, h, off, d, num_kv_heads, block_size, head_dim);
                k_pool[e] = k_new[(s * num_kv_heads + h) * head_dim + d];
                v_pool[e] = v_new[(s * num_kv_heads + h) * head_dim + d];
            }
        if (slot_out)
            slot_out[s] = phys * block_size + off;
    }
    free(map);
    return rc;
}

/* ---- append of runs of tokens (history written before the decode step) ---- */
/* Segment i writes rows [cu[i], cu[i+1]) of k_src/v_src ([T][Hkv][D]) to logical
 * positions start_pos[i], start_pos[i]+1, ... of table row i. */
int oracle_append_tokens(uint16_t *k_pool, uint16_t *v_pool, const uint16_t *k_src,
                         const uint16_t *v_src, const int64_t *cu, const int32_t *start_pos,
                         const int32_t *block_tables, int64_t num_segs, int64_t num_kv_heads,
                         int64_t head_dim, int64_t block_size, int64_t max_blocks_per_seq,
                         int64_t num_blocks)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks);
    if (rc)
        return rc;
    unsigned char *map = calloc((size_t)(num_blocks * block_size), 1);
    if (!map)
        return OR_ENOMEM;
    for (int64_t i = 0; i < num_segs && rc == OR_OK; ++i) {
        for (int64_t r = cu[i]; r < cu[i + 1] && rc == OR_OK; ++r) {
            int64_t t = start_pos[i] + (r - cu[i]);
            int64_t phys, off;
            rc = oracle_locate(block_tables + i * max_blocks_per_seq, max_blocks_per_seq,
                               block_size, num_blocks, t, &phys, &off);
            if (rc)
                break;
            rc = mark_slot(map, phys * block_size + off);
            if (rc)
                break;
            for (int64_t h = 0; h < num_kv_heads; ++h)
                for (int64_t d = 0; d < head_dim; ++d) {
                    int64_t e = oracle_elem_offset(phys, h, off, d, num_kv_heads, block_size,
                                                   head_dim);
                    k_pool[e] = k_src[(r * num_kv_heads + h) * head_dim + d];
                    v_pool[e] = v_src[(r * num_kv_heads + h) * head_dim + d];
                }
        }
    }
    free(map);
    return rc;
}

/* ---- block copy (copy-on-write) ------------------------------------------ */
/* For each pair i, block dst[i] of both pools becomes a copy of block src[i] as
 * it was before the call.  A destination that is also a source, or that appears
 * twice, would make the result depend on the copy order: OR_EDUP. */
int oracle_copy_blocks(uint16_t *k_pool, uint16_t *v_pool, const int32_t *src,
                       const int32_t *dst, int64_t num_pairs, int64_t num_kv_heads,
                       int64_t head_dim, int64_t block_size, int64_t num_blocks)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, 1, num_blocks);
    if (rc)
        return rc;
    if (num_pairs < 0)
        return OR_EARG;
    for (int64_t i = 0; i < num_pairs; ++i)
        if (src[i] < 0 || src[i] >= num_blocks || dst[i] < 0 || dst[i] >= num_blocks)
            return OR_ETABLE;
    for (int64_t i = 0; i < num_pairs; ++i)
        for (int64_t j = 0; j < num_pairs; ++j)
            if (dst[i] == src[j] || (j != i && dst[i] == dst[j]))
                return OR_EDUP;
    for (int64_t i = 0; i < num_pairs; ++i)
        for (int64_t h = 0; h < num_kv_heads; ++h)
            for (int64_t off = 0; off < block_size; ++off)
                for (int64_t d = 0; d < head_dim; ++d) {
                    int64_t from = oracle_elem_offset(src[i], h, off, d, num_kv_heads, block_size,
                                                      head_dim);
                    int64_t to = oracle_elem_offset(dst[i], h, off, d, num_kv_heads, block_size,
                                                    head_dim);
                    k_pool[to] = k_pool[from];
                    v_pool[to] = v_pool[from];
                }
    return OR_OK;
}

/* ---- slot copy (copy-on-write split of a shared slot) ---------------------- */
/* Copy i = copies[5*i .. 5*i+4] = (src block, src offset, dst block, dst offset,
 * length): rows src offset .. src offset+length-1 of the source block become rows
 * dst offset .. dst offset+length-1 of the destination block, in every head of
 * both pools, as they were before the call.  Blocks must lie in the pool and both
 * row ranges inside their block.  A destination row that is also a source row of
 * any copy, or a destination row of another copy, would make the result depend
 * on the copy order: OR_EDUP. */
static int rows_overlap(int64_t b0, int64_t o0, int64_t n0, int64_t b1, int64_t o1, int64_t n1)
{
    return b0 == b1 && o0 < o1 + n1 && o1 < o0 + n0;
}

int oracle_copy_slots(uint16_t *k_pool, uint16_t *v_pool, const int32_t *copies,
                      int64_t num_copies, int64_t num_kv_heads, int64_t head_dim,
                      int64_t block_size, int64_t num_blocks)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, 1, num_blocks);
    if (rc)
        return rc;
    if (num_copies < 0)
        return OR_EARG;
    for (int64_t i = 0; i < num_copies; ++i) {
        const int32_t *c = copies + 5 * i;
        if (c[0] < 0 || c[0] >= num_blocks || c[2] < 0 || c[2] >= num_blocks)
            return OR_ETABLE;
        if (c[1] < 0 || c[3] < 0 || c[4] < 0 || c[1] + c[4] > block_size ||
            c[3] + c[4] > block_size)
            return OR_EOFFSET;
    }
    for (int64_t i = 0; i < num_copies; ++i)
        for (int64_t j = 0; j < num_copies; ++j) {
            const int32_t *a = copies + 5 * i, *b = copies + 5 * j;
            if (rows_overlap(a[2], a[3], a[4], b[0], b[1], b[4]) ||
                (j != i && rows_overlap(a[2], a[3], a[4], b[2], b[3], b[4])))
                return OR_EDUP;
        }
    for (int64_t i = 0; i < num_copies; ++i) {
        const int32_t *c = copies + 5 * i;
        for (int64_t h = 0; h < num_kv_heads; ++h)
            for (int64_t r = 0; r < c[4]; ++r)
                for (int64_t d = 0; d < head_dim; ++d) {
                    int64_t from = oracle_elem_offset(c[0], h, c[1] + r, d, num_kv_heads,
                                                      block_size, head_dim);
                    int64_t to = oracle_elem_offset(c[2], h, c[3] + r, d, num_kv_heads,
                                                    block_size, head_dim);
                    k_pool[to] = k_pool[from];
                    v_pool[to] = v_pool[from];
                }
    }
    return OR_OK;
}

/* ---- attention over tokens [t0, t1) of one (sequence, query head) --------- */
/* Writes o[0..D) = sum_t w_t v_t / sum_t w_t with w_t = exp(z_t - max z) and
 * z_t = scale * q.k_t, and returns lse = max z + ln(sum w) through *lse.
 * An empty range gives o = 0 and lse = -inf. */
static int attend_range(double *o, double *lse, const uint16_t *q_row, const uint16_t *k_pool,
                        const uint16_t *v_pool, const int32_t *table_row, int64_t g,
                        int64_t t0, int64_t t1, int64_t num_kv_heads, int64_t head_dim,
                        int64_t block_size, int64_t max_blocks_per_seq, int64_t num_blocks,
                        double scale, int dtype, double *z)
{
    for (int64_t d = 0; d < head_dim; ++d)
        o[d] = 0.0;
    if (t1 <= t0) {
        *lse = -INFINITY;
        return OR_OK;
    }
    /* pass 1: scores */
    double m = -INFINITY;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t phys, off;
        int rc = oracle_locate(table_row, max_blocks_per_seq, block_size, num_blocks, t, &phys,
                               &off);
        if (rc)
            return rc;
        const uint16_t *k = k_pool + oracle_elem_offset(phys, g, off, 0, num_kv_heads,
                                                        block_size, head_dim);
        double acc = 0.0;
        for (int64_t d = 0; d < head_dim; ++d)
            acc += widen(q_row[d], dtype) * widen(k[d], dtype);
        z[t - t0] = scale * acc;
        if (z[t - t0] > m)
            m = z[t - t0];
    }
    /* pass 2: weights and weighted sum of V */
    double l = 0.0;
    for (int64_t t = t0; t < t1; ++t) {
        int64_t phys, off;
        oracle_locate(table_row, max_blocks_per_seq, block_size, num_blocks, t, &phys, &off);
        const uint16_t *v = v_pool + oracle_elem_offset(phys, g, off, 0, num_kv_heads,
                                                        block_size, head_dim);
        double w = exp(z[t - t0] - m);
        l += w;
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] += w * widen(v[d], dtype);
    }
    for (int64_t d = 0; d < head_dim; ++d)
        o[d] /= l;
    *lse = m + log(l);
    return OR_OK;
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* Number of threads a parallel region of the oracle would use. */
int oracle_max_threads(int nthreads) { return set_threads(nthreads); }

/* out: double [S][Hq][D]. */
int oracle_attention(double *out, const uint16_t *q, const uint16_t *k_pool,
                     const uint16_t *v_pool, const int32_t *block_tables,
                     const int32_t *context_lens, int64_t num_seqs, int64_t num_q_heads,
                     int64_t num_kv_heads, int64_t head_dim, int64_t block_size,
                     int64_t max_blocks_per_seq, int64_t num_blocks, double scale, int dtype,
                     int nthreads)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks);
    if (rc)
        return rc;
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
        return OR_EARG;
    int64_t group = num_q_heads / num_kv_heads;
    int64_t max_n = max_blocks_per_seq * block_size;
    int err = OR_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
        if (!z) {
#pragma omp atomic write
            err = OR_ENOMEM;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < num_seqs * num_q_heads; ++i) {
            if (!z)
                continue;
            int64_t s = i / num_q_heads, h = i % num_q_heads;
            int64_t n = context_lens[s];
            double lse;
            int r;
            if (n > max_n)
                r = OR_ETABLE;
            else
                r = attend_range(out + i * head_dim, &lse, q + i * head_dim, k_pool, v_pool,
                                 block_tables + s * max_blocks_per_seq, h / group, 0, n,
                                 num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                 num_blocks, scale, dtype, z);
            if (r) {
#pragma omp atomic write
                err = r;
            }
        }
        free(z);
    }
    return err;
}

/* Per-partition attention: partition p covers tokens [p*P, min(n, (p+1)*P)).
 * part_o: double [S][Hq][MP][D], part_lse: double [S][Hq][MP]; partitions
 * p >= ceil(n/P) are left untouched. */
int oracle_partials(double *part_o, double *part_lse, const uint16_t *q,
                    const uint16_t *k_pool, const uint16_t *v_pool,
                    const int32_t *block_tables, const int32_t *context_lens, int64_t num_seqs,
                    int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                    int64_t block_size, int64_t max_blocks_per_seq, int64_t num_blocks,
                    double scale, int dtype, int64_t partition_size, int64_t max_partitions,
                    int nthreads)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks);
    if (rc)
        return rc;
    if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0 || partition_size <= 0 ||
        max_partitions <= 0)
        return OR_EARG;
    int64_t group = num_q_heads / num_kv_heads;
    int err = OR_OK;
    set_threads(nthreads);
#pragma omp parallel
    {
        double *z = malloc(sizeof(double) * (size_t)partition_size);
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < num_seqs * num_q_heads; ++i) {
            int64_t s = i / num_q_heads, h = i % num_q_heads;
            int64_t n = context_lens[s];
            int64_t np = (n + partition_size - 1) / partition_size;
            if (np > max_partitions || !z) {
#pragma omp atomic write
                err = z ? OR_EARG : OR_ENOMEM;
                continue;
            }
            for (int64_t p = 0; p < np; ++p) {
                int64_t t0 = p * partition_size;
                int64_t t1 = t0 + partition_size < n ? t0 + partition_size : n;
                int r = attend_range(part_o + (i * max_partitions + p) * head_dim,
                                     part_lse + i * max_partitions + p, q + i * head_dim,
                                     k_pool, v_pool, block_tables + s * max_blocks_per_seq,
                                     h / group, t0, t1, num_kv_heads, head_dim, block_size,
                                     max_blocks_per_seq, num_blocks, scale, dtype, z);
                if (r) {
#pragma omp atomic write
                    err = r;
                }
            }
        }
        free(z);
    }
    return err;
}

/* Log-sum-exp merge of partitions p < ceil(n/P): out = sum_p w_p o_p / sum_p w_p
 * with w_p = exp(lse_p - max_p lse_p).  n == 0 gives zeros.  out: double [S][Hq][D]. */
int oracle_merge(double *out, const double *part_o, const double *part_lse,
                 const int32_t *context_lens, int64_t num_seqs, int64_t num_q_heads,
                 int64_t head_dim, int64_t partition_size, int64_t max_partitions)
{
    if (partition_size <= 0 || max_partitions <= 0 || head_dim <= 0)
        return OR_EARG;
    for (int64_t i = 0; i < num_seqs * num_q_heads; ++i) {
        int64_t s = i / num_q_heads;
        int64_t n = context_lens[s];
        int64_t np = (n + partition_size - 1) / partition_size;
        double *o = out + i * head_dim;
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        if (np <= 0)
            continue;
        if (np > max_partitions)
            return OR_EARG;
        const double *lse = part_lse + i * max_partitions;
        double M = -INFINITY;
        for (int64_t p = 0; p < np; ++p)
            if (lse[p] > M)
                M = lse[p];
        double wsum = 0.0;
        for (int64_t p = 0; p < np; ++p) {
            double w = exp(lse[p] - M);
            wsum += w;
            const double *op = part_o + (i * max_partitions + p) * head_dim;
            for (int64_t d = 0; d < head_dim; ++d)
                o[d] += w * op[d];
        }
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] /= wsum;
    }
    return OR_OK;
}

/* ---- slotted segments ------------------------------------------------------ */
/* Physical block and in-block offset of logical token t of a sequence whose KV is
 * the segments segs[0..num_segs) = (block id, slot offset, length) triples. */
int oracle_locate_slotted(const int32_t *segs, int64_t num_segs, int64_t block_size,
                          int64_t num_blocks, int64_t t, int64_t *phys, int64_t *off)
{
    if (t < 0 || block_size <= 0 || num_segs < 0)
        return OR_EARG;
    int64_t start = 0;
    for (int64_t i = 0; i < num_segs; ++i) {
        int64_t blk = segs[3 * i], so = segs[3 * i + 1], len = segs[3 * i + 2];
        if (so < 0 || len < 0 || so + len > block_size)
            return OR_EOFFSET;
        if (t < start + len) {
            if (blk < 0 || blk >= num_blocks)
                return OR_ETABLE;
            *phys = blk;
            *off = so + (t - start);
            return OR_OK;
        }
        start += len;
    }
    return OR_ETABLE;  /* t is past the sequence */
}

/* Append of each sequence's new token to its slotted segments: position n-1 of the
 * concatenated segments (n = sum of the first num_segs[s] lengths), every head,
 * K and V; slot_out[s] = block * block_size + offset, or -1 when n = 0.  Two
 * sequences writing one slot is an error (OR_EDUP).  segs: [num_seqs][max_segs][3]. */
int oracle_append_slotted(uint16_t *k_pool, uint16_t *v_pool, const uint16_t *k_new,
                          const uint16_t *v_new, const int32_t *segs, const int32_t *num_segs,
                          int64_t *slot_out, int64_t num_seqs, int64_t max_segs,
                          int64_t num_kv_heads, int64_t head_dim, int64_t block_size,
                          int64_t num_blocks)
{
    int rc = check_dims(num_kv_heads, head_dim, block_size, 1, num_blocks);
    if (rc)
        return rc;
    if (num_seqs < 0 || max_segs < 0)
        return OR_EARG;
    unsigned char *map = calloc((size_t)(num_blocks * block_size), 1);
    if (!map)
        return OR_ENOMEM;
    for (int64_t s = 0; s < num_seqs && rc == OR_OK; ++s) {
        const int32_t *row = segs + s * max_segs * 3;
        const int64_t ns = num_segs[s];
        if (ns < 0 || ns > max_segs) {
            rc = OR_EARG;
            break;
        }
        int64_t n = 0;
        for (int64_t i = 0; i < ns; ++i)
            n += row[3 * i + 2];
        if (n <= 0) {
            if (slot_out)
                slot_out[s] = -1;
            continue;
        }
        int64_t phys, off;
        rc = oracle_locate_slotted(row, ns, block_size, num_blocks, n - 1, &phys, &off);
        if (rc)
            break;
        rc = mark_slot(map, phys * block_size + off);
        if (rc)
            break;
        for (int64_t h = 0; h < num_kv_heads; ++h) {
            const uint16_t *kn = k_new + (s * num_kv_heads + h) * head_dim;
            const uint16_t *vn = v_new + (s * num_kv_heads + h) * head_dim;
            for (int64_t d = 0; d < head_dim; ++d) {
                const int64_t at =
                    oracle_elem_offset(phys, h, off, d, num_kv_heads, block_size, head_dim);
                k_pool[at] = kn[d];
                v_pool[at] = vn[d];
            }
        }
        if (slot_out)
            slot_out[s] = phys * block_size + off;
    }
    free(map);
    return rc;
}

/* Decode attention over slotted segments: out[s][h] = softmax(scale q.K^T) V over
 * the n = sum of lengths tokens of sequence s, in logical order, two-pass fp64
 * softmax as in oracle_attention.  segs: [num_seqs][max_segs][3]. */
int oracle_attention_slotted(double *out, const uint16_t *q, const uint16_t *k_pool,
                             const uint16_t *v_pool, const int32_t *segs,
                             const int32_t *num_segs, int64_t num_seqs, int64_t num_q_heads,
                             int64_t num_kv_heads, int64_t head_dim, int64_t block_size,
                             int64_t max_segs, int64_t num_blocks, double scale, int dtype,
                             int nthreads)
{
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads || head_dim <= 0 ||
        max_segs < 0)
        return OR_EARG;
    const int64_t group = num_q_heads / num_kv_heads;
    int err = OR_OK;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic)
    for (int64_t sh = 0; sh < num_seqs * num_q_heads; ++sh) {
        const int64_t s = sh / num_q_heads, h = sh % num_q_heads, g = h / group;
        const int32_t *row = segs + s * max_segs * 3;
        const int64_t ns = num_segs[s];
        double *o = out + sh * head_dim;
        const uint16_t *qr = q + sh * head_dim;
        if (ns < 0 || ns > max_segs) {
#pragma omp atomic write
            err = OR_EARG;
            continue;
        }
        int64_t n = 0;
        for (int64_t i = 0; i < ns; ++i)
            n += row[3 * i + 2];
        double *z = malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!z) {
#pragma omp atomic write
            err = OR_ENOMEM;
            continue;
        }
        double m = -INFINITY;
        int bad = 0;
        for (int64_t t = 0; t < n && !bad; ++t) {
            int64_t phys, off;
            if (oracle_locate_slotted(row, ns, block_size, num_blocks, t, &phys, &off)) {
                bad = 1;
                break;
            }
            const uint16_t *k = k_pool + oracle_elem_offset(phys, g, off, 0, num_kv_heads,
                                                            block_size, head_dim);
            double acc = 0.0;
            for (int64_t d = 0; d < head_dim; ++d)
                acc += widen(qr[d], dtype) * widen(k[d], dtype);
            z[t] = scale * acc;
            if (z[t] > m)
                m = z[t];
        }
        for (int64_t d = 0; d < head_dim; ++d)
            o[d] = 0.0;
        if (bad) {
#pragma omp atomic write
            err = OR_ETABLE;
            free(z);
            continue;
        }
        double l = 0.0;
        for (int64_t t = 0; t < n; ++t) {
            int64_t phys, off;
            oracle_locate_slotted(row, ns, block_size, num_blocks, t, &phys, &off);
            const uint16_t *v = v_pool + oracle_elem_offset(phys, g, off, 0, num_kv_heads,
                                                            block_size, head_dim);
            const double w = exp(z[t] - m);
            l += w;
            for (int64_t d = 0; d < head_dim; ++d)
                o[d] += w * widen(v[d], dtype);
        }
        if (n > 0)
            for (int64_t d = 0; d < head_dim; ++d)
                o[d] /= l;
        free(z);
    }
    return err;
}
