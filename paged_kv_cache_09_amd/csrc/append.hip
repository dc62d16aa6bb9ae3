// append.hip -- cache-append scatters: the new token of a decode step, and runs
// of tokens (prompts, prefill chunks, any history).
//
// A token at logical position t of a sequence is written to offset t % B of
// physical block table[t / B] (page "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量
// PagedAttention 与 KV 缓存分块", pwwt.cn, section "注意力寻址"); a decode step
// writes position n-1 of each sequence, which is offset 0 of a freshly appended
// block whenever the previous block was full (page "显存虚拟化革命：PagedAttention
// 内存池管理与显存碎片终结", blog.llmgo.top, §三, sequence diagram).  The copy is
// bit-exact.
//
// gfx950 design.  Single-token append: one thread moves one 16-byte chunk (8
// elements of one head's row), so a wave stores whole 256-byte head rows with
// dwordx4 stores.  Runs of tokens: a work-group takes up to 64 consecutive
// source rows; its first wave finds the run of the first row with a 64-way
// search, walks each row's slot once and leaves the destination offsets in LDS;
// then all lanes stream the rows with four 16-byte loads in flight each.  The
// runs' loads and stores are nontemporal (each source row is read once and each
// slot written once): 5.0-5.3 TB/s against 4.8-5.1 TB/s cached, alternated on
// one MI355X.  The single-token append keeps cached stores: its scattered rows
// are few and land amid the decode's reads.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kChunks = kHeadDim / 8;  // 16-byte chunks per head row

struct AppendArgs {
    uint16_t *k_pool;
    uint16_t *v_pool;
    const uint16_t *k_new;
    const uint16_t *v_new;
    const int32_t *tables;
    const int32_t *lens;
    int64_t *slot_out;
    int num_seqs, num_kv_heads, block_size, width;
};

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_seq = a.num_kv_heads * 2 * kChunks;
    const int64_t total = (int64_t)a.num_seqs * per_seq;
    if (idx >= total)
        return;
    const int s = (int)(idx / per_seq);
    const int rem = (int)(idx % per_seq);
    const int kv = rem / (a.num_kv_heads * kChunks);          // 0: K, 1: V
    const int h = (rem / kChunks) % a.num_kv_heads;
    const int c = rem % kChunks;
    const int n = a.lens[s];
    if (n <= 0) {
        if (rem == 0 && a.slot_out)
            a.slot_out[s] = -1;
        return;
    }
    const int t = n - 1;
    const int blk = t / a.block_size;
    const int off = t % a.block_size;
    const int64_t phys = a.tables[(int64_t)s * a.width + blk];
    const int64_t dst = ((phys * a.num_kv_heads + h) * a.block_size + off) * kHeadDim + c * 8;
    const int64_t src = ((int64_t)s * a.num_kv_heads + h) * kHeadDim + c * 8;
    if (kv == 0)
        *(u32x4 *)(a.k_pool + dst) = *(const u32x4 *)(a.k_new + src);
    else
        *(u32x4 *)(a.v_pool + dst) = *(const u32x4 *)(a.v_new + src);
    if (rem == 0 && a.slot_out)
        a.slot_out[s] = phys * a.block_size + off;
}

struct AppendTokensArgs {
    uint16_t *k_pool;
    uint16_t *v_pool;
    const uint16_t *k_src;
    const uint16_t *v_src;
    const int64_t *cu;
    const int32_t *start_pos;
    const int32_t *tables;
    int num_runs, num_kv_heads, block_size, width;
    int64_t total_tokens;
    int rows_per_group;  // consecutive source rows handled by one work-group (<= 64)
};

constexpr int kRunThreads = 256;
constexpr int kRunUnroll = 4;
constexpr int kMaxRowsPerGroup = 64;

// Largest run index r with cu[r] <= row (the run holding source row `row`; empty
// runs before it share its start and are skipped by taking the largest).  `row`
// is uniform; the wave probes 63 evenly spaced entries per round, so 4096 runs
// take two rounds of one load each instead of twelve dependent loads.
__device__ int find_run(const int64_t *cu, int num_runs, int64_t row, int lane)
{
    int lo = 0, hi = num_runs;  // cu[lo] <= row < cu[hi]
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const bool le = lane > 0 && idx < hi && cu[idx] <= row;
        const int k = __popcll(__ballot(le));  // probes 1..k satisfy cu <= row
        const int nlo = lo + k * step;
        const int nhi = lo + (k + 1) * step;
        lo = nlo;
        hi = nhi < hi ? nhi : hi;
    }
    return lo;
}

__global__ __launch_bounds__(kRunThreads) void append_tokens_kernel(AppendTokensArgs a)
{
    __shared__ int64_t dst_row[kMaxRowsPerGroup];  // pool offset of (phys, head 0, off, dim 0)
    const int tid = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * a.rows_per_group;
    const int64_t left = a.total_tokens - row0;
    const int nrows = left < a.rows_per_group ? (int)left : a.rows_per_group;
    if (tid < 64) {
        int r = find_run(a.cu, a.num_runs, row0, tid);
        if (tid < nrows) {
            const int64_t row = row0 + tid;
            while (r + 1 < a.num_runs && a.cu[r + 1] <= row)
                ++r;
            const int64_t t = a.start_pos[r] + (row - a.cu[r]);
            const int64_t blk = t / a.block_size;
            const int64_t off = t % a.block_size;
            const int64_t phys = a.tables[(int64_t)r * a.width + blk];
            dst_row[tid] = (phys * a.num_kv_heads * a.block_size + off) * kHeadDim;
        }
    }
    __syncthreads();
    // unit u = (row i, K or V, head h, chunk c) in that order, so consecutive
    // lanes read consecutive 16-byte chunks of a source row and write whole
    // 256-byte head rows of a block
    const int per_kv = a.num_kv_heads * kChunks;
    const int per_row = 2 * per_kv;
    const int units = nrows * per_row;
    const int64_t head_stride = (int64_t)a.block_size * kHeadDim;
    for (int base = 0; base < units; base += kRunThreads * kRunUnroll) {
        u32x4 val[kRunUnroll];
        int64_t dst[kRunUnroll];
        int kv[kRunUnroll];
#pragma unroll
        for (int j = 0; j < kRunUnroll; ++j) {
            const int u = base + j * kRunThreads + tid;
            kv[j] = -1;
            if (u < units) {
                const int i = u / per_row;
                const int rem = u - i * per_row;
                kv[j] = rem / per_kv;
                const int hc = rem - kv[j] * per_kv;  // h * kChunks + c
                const int h = hc / kChunks;
                const int c = hc - h * kChunks;
                const int64_t src = (row0 + i) * (int64_t)per_kv * 8 + (int64_t)hc * 8;
                dst[j] = dst_row[i] + h * head_stride + c * 8;
                val[j] = ldnt((const u32x4 *)((kv[j] ? a.v_src : a.k_src) + src));
            }
        }
#pragma unroll
        for (int j = 0; j < kRunUnroll; ++j)
            if (kv[j] >= 0)
                __builtin_nontemporal_store(val[j],
                                            (u32x4 *)((kv[j] ? a.v_pool : a.k_pool) + dst[j]));
    }
}

}  // namespace

hipError_t launch_append(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                         const int32_t *tables, const int32_t *lens, int64_t *slot_out,
                         int num_seqs, int num_kv_heads, int block_size, int width,
                         hipStream_t stream)
{
    AppendArgs a{(uint16_t *)k_pool, (uint16_t *)v_pool, (const uint16_t *)k_new,
                 (const uint16_t *)v_new, tables, lens, slot_out, num_seqs, num_kv_heads,
                 block_size, width};
    const int64_t total = (int64_t)num_seqs * num_kv_heads * 2 * kChunks;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       a);
    return hipGetLastError();
}

int64_t append_tokens_groups(int64_t total_tokens, int num_kv_heads, int *rows_per_group)
{
    // about 16 units (16-byte chunks) per thread: 4 rows of a 32-head model,
    // 64 rows of a 2-head one
    const int64_t per_row = 2 * (int64_t)num_kv_heads * kChunks;
    int64_t rows = (kRunThreads * 16) / per_row;
    rows = rows < 1 ? 1 : (rows > kMaxRowsPerGroup ? kMaxRowsPerGroup : rows);
    if (rows_per_group)
        *rows_per_group = (int)rows;
    return (total_tokens + rows - 1) / rows;
}

hipError_t launch_append_tokens(void *k_pool, void *v_pool, const void *k_src,
                                const void *v_src, const int64_t *cu, const int32_t *start_pos,
                                const int32_t *tables, int num_runs, int64_t total_tokens,
                                int num_kv_heads, int block_size, int width, hipStream_t stream)
{
    int rows = 1;
    const int64_t groups = append_tokens_groups(total_tokens, num_kv_heads, &rows);
    AppendTokensArgs a{(uint16_t *)k_pool, (uint16_t *)v_pool, (const uint16_t *)k_src,
                       (const uint16_t *)v_src, cu, start_pos, tables, num_runs, num_kv_heads,
                       block_size, width, total_tokens, rows};
    hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)groups), dim3(kRunThreads), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pkv
