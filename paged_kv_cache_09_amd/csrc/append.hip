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
// gfx950 design: one thread moves one 16-byte chunk (8 elements of one head's
// row), so a wave stores whole 256-byte head rows with dwordx4 stores; the slot
// arithmetic is a handful of scalar-friendly integer ops per thread.
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
};

__global__ __launch_bounds__(256) void append_tokens_kernel(AppendTokensArgs a)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int per_tok = a.num_kv_heads * 2 * kChunks;
    if (idx >= a.total_tokens * per_tok)
        return;
    const int64_t row = idx / per_tok;
    const int rem = (int)(idx % per_tok);
    const int kv = rem / (a.num_kv_heads * kChunks);
    const int h = (rem / kChunks) % a.num_kv_heads;
    const int c = rem % kChunks;
    // run holding this row: largest r with cu[r] <= row (runs may be empty)
    int lo = 0, hi = a.num_runs;  // invariant: cu[lo] <= row < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= row)
            lo = mid;
        else
            hi = mid;
    }
    const int64_t t = a.start_pos[lo] + (row - a.cu[lo]);
    const int64_t blk = t / a.block_size;
    const int off = (int)(t % a.block_size);
    const int64_t phys = a.tables[(int64_t)lo * a.width + blk];
    const int64_t dst = ((phys * a.num_kv_heads + h) * a.block_size + off) * kHeadDim + c * 8;
    const int64_t src = (row * a.num_kv_heads + h) * kHeadDim + c * 8;
    if (kv == 0)
        *(u32x4 *)(a.k_pool + dst) = *(const u32x4 *)(a.k_src + src);
    else
        *(u32x4 *)(a.v_pool + dst) = *(const u32x4 *)(a.v_src + src);
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

hipError_t launch_append_tokens(void *k_pool, void *v_pool, const void *k_src,
                                const void *v_src, const int64_t *cu, const int32_t *start_pos,
                                const int32_t *tables, int num_runs, int64_t total_tokens,
                                int num_kv_heads, int block_size, int width, hipStream_t stream)
{
    AppendTokensArgs a{(uint16_t *)k_pool, (uint16_t *)v_pool, (const uint16_t *)k_src,
                       (const uint16_t *)v_src, cu, start_pos, tables, num_runs, num_kv_heads,
                       block_size, width, total_tokens};
    const int64_t total = total_tokens * num_kv_heads * 2 * kChunks;
    hipLaunchKernelGGL(append_tokens_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace pkv
