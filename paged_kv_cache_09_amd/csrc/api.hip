// api.hip -- the C ABI of libpagedkv (declared in include/paged_kv.h): argument
// validation, kernel selection and launch on the caller's stream.
//
// Validation happens entirely on the host before any HIP call, so a bad argument
// returns a status without touching the device.  With PKV_DEBUG_CHECK=1 in the
// environment, each call additionally checks the device-resident caller contract
// (context lengths and block-table entries) with a small kernel, synchronises the
// stream and returns PKV_EDEVICE on a violation.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/paged_kv.h"
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

__device__ int g_debug_flag;  // set by the debug-check kernels, never by the hot path

__global__ void debug_clear_kernel() { g_debug_flag = 0; }

__global__ void debug_tables_kernel(const int32_t *tables, const int32_t *lens, int num_seqs,
                                    int width, int block_size, int64_t num_blocks)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= num_seqs)
        return;
    const int n = lens[s];
    if (n < 0 || (int64_t)n > (int64_t)width * block_size) {
        atomicOr(&g_debug_flag, 1);
        return;
    }
    const int nb = (n + block_size - 1) / block_size;
    for (int b = 0; b < nb; ++b) {
        const int32_t p = tables[(int64_t)s * width + b];
        if (p < 0 || p >= num_blocks)
            atomicOr(&g_debug_flag, 2);
    }
}

__global__ void debug_runs_kernel(const int64_t *cu, const int32_t *start_pos,
                                  const int32_t *tables, int num_runs, int64_t total_tokens,
                                  int width, int block_size, int64_t num_blocks)
{
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r > num_runs)
        return;
    if (r == 0 && cu[0] != 0)
        atomicOr(&g_debug_flag, 4);
    if (r == num_runs) {
        if (cu[num_runs] != total_tokens)
            atomicOr(&g_debug_flag, 4);
        return;
    }
    const int64_t cnt = cu[r + 1] - cu[r];
    const int64_t st = start_pos[r];
    if (cnt < 0 || st < 0 || st + cnt > (int64_t)width * block_size) {
        atomicOr(&g_debug_flag, 8);
        return;
    }
    if (cnt == 0)
        return;
    for (int64_t b = st / block_size; b <= (st + cnt - 1) / block_size; ++b) {
        const int32_t p = tables[(int64_t)r * width + b];
        if (p < 0 || p >= num_blocks)
            atomicOr(&g_debug_flag, 2);
    }
}

// Shared-prefix groups: group_cu runs from 0 to num_seqs without decreasing,
// prefix lengths are >= 0, and every member attends to at least its group's
// prefix (plus the appended token when the call appends).
__global__ void debug_groups_kernel(const int32_t *cu, const int32_t *prefix_lens,
                                    const int32_t *lens, int num_groups, int num_seqs,
                                    int extra)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= num_groups)
        return;
    const int lo = cu[k], hi = cu[k + 1];
    // bounds first: each thread sees only its own group, and the loop below must
    // stay short whatever the contents
    if ((k == 0 && lo != 0) || (k == num_groups - 1 && hi != num_seqs) || lo < 0 ||
        hi > num_seqs || hi < lo || prefix_lens[k] < 0) {
        atomicOr(&g_debug_flag, 32);
        return;
    }
    for (int s = lo; s < hi; ++s)
        if (lens[s] < prefix_lens[k] + extra)
            atomicOr(&g_debug_flag, 32);
}

// Slotted segment lists: counts within [0, max_segments], every segment inside
// the pool and inside its block.
__global__ void debug_segments_kernel(const int32_t *segs, const int32_t *nsegs, int num_seqs,
                                      int max_segs, int block_size, int64_t num_blocks)
{
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= num_seqs)
        return;
    const int n = nsegs[s];
    if (n < 0 || n > max_segs) {
        atomicOr(&g_debug_flag, 64);
        return;
    }
    for (int i = 0; i < n; ++i) {
        const int32_t *t = segs + ((int64_t)s * max_segs + i) * 3;
        if (t[0] < 0 || t[0] >= num_blocks || t[1] < 0 || t[2] < 0 || t[1] + t[2] > block_size)
            atomicOr(&g_debug_flag, 64);
    }
}

// Copy pairs: ids inside the pool; a destination may be neither another pair's
// destination nor any pair's source (the result would depend on copy order).
__global__ void debug_copies_kernel(const int32_t *src, const int32_t *dst, int num_pairs,
                                    int64_t num_blocks)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= num_pairs)
        return;
    const int32_t d = dst[i], s = src[i];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) {
        atomicOr(&g_debug_flag, 2);
        return;
    }
    for (int j = 0; j < num_pairs; ++j)
        if (src[j] == d || (j != i && dst[j] == d))
            atomicOr(&g_debug_flag, 16);
}

// A dispatch order: every entry inside the batch and no sequence twice (so it is
// a permutation of 0 .. num_seqs-1).
__global__ void debug_order_kernel(const int32_t *order, int num_seqs)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= num_seqs)
        return;
    const int32_t v = order[i];
    if (v < 0 || v >= num_seqs) {
        atomicOr(&g_debug_flag, 2);
        return;
    }
    for (int j = 0; j < i; ++j)
        if (order[j] == v)
            atomicOr(&g_debug_flag, 16);
}

// Slot copies: blocks inside the pool, both row ranges inside their block, and no
// destination row that is a source row of any copy or a destination row of
// another (the result would depend on copy order).
__device__ bool rows_overlap(const int32_t *a, int ab, int ao, const int32_t *b, int bb, int bo)
{
    return a[ab] == b[bb] && a[ao] < b[bo] + b[4] && b[bo] < a[ao] + a[4];
}

__global__ void debug_slot_copies_kernel(const int32_t *copies, int num_copies, int block_size,
                                         int64_t num_blocks)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= num_copies)
        return;
    const int32_t *c = copies + 5 * (int64_t)i;
    if (c[0] < 0 || c[0] >= num_blocks || c[2] < 0 || c[2] >= num_blocks) {
        atomicOr(&g_debug_flag, 2);
        return;
    }
    if (c[1] < 0 || c[3] < 0 || c[4] < 0 || c[1] + c[4] > block_size ||
        c[3] + c[4] > block_size) {
        atomicOr(&g_debug_flag, 128);
        return;
    }
    for (int j = 0; j < num_copies; ++j) {
        const int32_t *o = copies + 5 * (int64_t)j;
        if (rows_overlap(c, 2, 3, o, 0, 1) || (j != i && rows_overlap(c, 2, 3, o, 2, 3)))
            atomicOr(&g_debug_flag, 16);
    }
}

int read_debug_flag(hipStream_t stream)
{
    int flag = 0;
    if (hipMemcpyFromSymbolAsync(&flag, HIP_SYMBOL(g_debug_flag), sizeof(int), 0,
                                 hipMemcpyDeviceToHost, stream) != hipSuccess)
        return PKV_ELAUNCH;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return PKV_ELAUNCH;
    return flag ? PKV_EDEVICE : PKV_OK;
}

}  // namespace

int debug_check_tables(const int32_t *tables, const int32_t *lens, int num_seqs, int width,
                       int block_size, int64_t num_blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_tables_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, stream,
                       tables, lens, num_seqs, width, block_size, num_blocks);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_runs(const int64_t *cu, const int32_t *start_pos, const int32_t *tables,
                     int num_runs, int64_t total_tokens, int width, int block_size,
                     int64_t num_blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_runs_kernel, dim3((num_runs + 1 + 255) / 256), dim3(256), 0, stream,
                       cu, start_pos, tables, num_runs, total_tokens, width, block_size,
                       num_blocks);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_groups(const int32_t *group_cu, const int32_t *prefix_lens,
                       const int32_t *lens, int num_groups, int num_seqs, int extra,
                       hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_groups_kernel, dim3((num_groups + 255) / 256), dim3(256), 0, stream,
                       group_cu, prefix_lens, lens, num_groups, num_seqs, extra);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_segments(const int32_t *segs, const int32_t *nsegs, int num_seqs, int max_segs,
                         int block_size, int64_t num_blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_segments_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, stream,
                       segs, nsegs, num_seqs, max_segs, block_size, num_blocks);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_copies(const int32_t *src, const int32_t *dst, int num_pairs,
                       int64_t num_blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_copies_kernel, dim3((num_pairs + 255) / 256), dim3(256), 0, stream,
                       src, dst, num_pairs, num_blocks);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_order(const int32_t *order, int num_seqs, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_order_kernel, dim3((num_seqs + 255) / 256), dim3(256), 0, stream,
                       order, num_seqs);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

int debug_check_slot_copies(const int32_t *copies, int num_copies, int block_size,
                            int64_t num_blocks, hipStream_t stream)
{
    hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream);
    hipLaunchKernelGGL(debug_slot_copies_kernel, dim3((num_copies + 255) / 256), dim3(256), 0,
                       stream, copies, num_copies, block_size, num_blocks);
    if (hipGetLastError() != hipSuccess)
        return PKV_ELAUNCH;
    return read_debug_flag(stream);
}

}  // namespace pkv

namespace {

// Read on every call so that a process can switch the check on and off.
bool debug_enabled()
{
    const char *e = getenv("PKV_DEBUG_CHECK");
    return e && e[0] && strcmp(e, "0") != 0;
}

// PKV_SLOTTED_TILES: "0" never takes the tiled slotted kernel, "1" takes it
// whenever a tile's list fits, anything else (the default) also asks for enough
// work-groups (see slotted_impl).
int slotted_tiles_mode()
{
    const char *e = getenv("PKV_SLOTTED_TILES");
    if (e && strcmp(e, "0") == 0)
        return 0;
    if (e && strcmp(e, "1") == 0)
        return 1;
    return 2;
}

// Compute units of the current device (cached per device; 256 on MI355X).
int device_cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool supported_block(int b) { return b == 16 || b == 32 || b == 64 || b == 128 || b == 256; }

// Checks shared by the pool-facing entry points.
int check_pool_shape(int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                     int64_t num_blocks, int dtype)
{
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return PKV_EINVAL;
    if (dtype != PKV_FP16 && dtype != PKV_BF16)
        return PKV_ENOTSUP;
    if (head_dim != pkv::kHeadDim || !supported_block(block_size))
        return PKV_ENOTSUP;
    // the largest element offset must fit the 64-bit address arithmetic
    if (num_blocks > (int64_t)1 << 40)
        return PKV_EINVAL;
    return PKV_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ELAUNCH; }

// The softmax scale of a call: a NaN selects 1/sqrt(head_dim); an infinite scale
// is an error (returns false).
bool resolve_scale(float &scale, int head_dim)
{
    if (scale != scale) {
        scale = 1.0f / __builtin_sqrtf((float)head_dim);
        return true;
    }
    return !__builtin_isinf(scale);
}

}  // namespace

extern "C" {

const char *pkv_status_string(int status)
{
    switch (status) {
    case PKV_OK:
        return "ok";
    case PKV_EINVAL:
        return "invalid argument";
    case PKV_ENOTSUP:
        return "unsupported shape or dtype";
    case PKV_EWORKSPACE:
        return "partition workspace missing or too small";
    case PKV_ELAUNCH:
        return "kernel launch failed";
    case PKV_EDEVICE:
        return "device-side check failed (context length, block-table entry, segment, copy "
               "pair, slot copy or prefix group out of range, or overlapping copies)";
    default:
        return "unknown status";
    }
}

int pkv_max_partitions(int max_blocks_per_seq, int block_size, int partition_size)
{
    if (max_blocks_per_seq <= 0 || block_size <= 0 || partition_size <= 0)
        return 0;
    const int64_t ctx = (int64_t)max_blocks_per_seq * block_size;
    const int64_t mp = (ctx + partition_size - 1) / partition_size;
    return mp > INT32_MAX ? 0 : (int)mp;
}

int paged_kv_append(void *k_pool, void *v_pool, const void *k_new, const void *v_new,
                    const int32_t *block_tables, const int32_t *context_lens, int64_t *slot_out,
                    int num_seqs, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream)
{
    if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens)
        return PKV_EINVAL;
    if (num_seqs < 0)
        return PKV_EINVAL;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                              dtype);
    if (rc)
        return rc;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new) ||
        ((uintptr_t)slot_out & 7u))
        return PKV_EINVAL;
    if ((int64_t)num_seqs * num_kv_heads * 2 * (pkv::kHeadDim / 8) > ((int64_t)1 << 31) * 255)
        return PKV_EINVAL;
    if (num_seqs == 0)
        return PKV_OK;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                     block_size, num_blocks, st);
        if (rc)
            return rc;
    }
    return launch_status(pkv::launch_append(k_pool, v_pool, k_new, v_new, block_tables,
                                            context_lens, slot_out, num_seqs, num_kv_heads,
                                            block_size, max_blocks_per_seq, st));
}

int paged_kv_append_tokens(void *k_pool, void *v_pool, const void *k_src, const void *v_src,
                           const int64_t *src_cu, const int32_t *start_pos,
                           const int32_t *block_tables, int num_runs, int64_t total_tokens,
                           int num_kv_heads, int head_dim, int block_size,
                           int max_blocks_per_seq, int64_t num_blocks, int dtype, void *stream)
{
    if (!k_pool || !v_pool || !src_cu || !start_pos || !block_tables)
        return PKV_EINVAL;
    if (num_runs < 0 || total_tokens < 0)
        return PKV_EINVAL;
    if (total_tokens > 0 && (!k_src || !v_src))
        return PKV_EINVAL;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                              dtype);
    if (rc)
        return rc;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_src) || !aligned16(v_src))
        return PKV_EINVAL;
    // one work-group per few rows; the grid must stay below 2^32 threads
    if (pkv::append_tokens_groups(total_tokens, num_kv_heads, nullptr) >= ((int64_t)1 << 24))
        return PKV_EINVAL;
    if (num_runs == 0 || total_tokens == 0)
        return PKV_OK;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_runs(src_cu, start_pos, block_tables, num_runs, total_tokens,
                                   max_blocks_per_seq, block_size, num_blocks, st);
        if (rc)
            return rc;
    }
    return launch_status(pkv::launch_append_tokens(k_pool, v_pool, k_src, v_src, src_cu,
                                                   start_pos, block_tables, num_runs,
                                                   total_tokens, num_kv_heads, block_size,
                                                   max_blocks_per_seq, st));
}

int paged_kv_copy_blocks(void *const *k_pools, void *const *v_pools, int num_layers,
                         const int32_t *src_blocks, const int32_t *dst_blocks, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         int dtype, void *stream)
{
    if (!k_pools || !v_pools || num_layers <= 0 || num_pairs < 0)
        return PKV_EINVAL;
    if (num_layers > pkv::kMaxCopyLayers)
        return PKV_ENOTSUP;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, 1, num_blocks, dtype);
    if (rc)
        return rc;
    for (int l = 0; l < num_layers; ++l)
        if (!k_pools[l] || !v_pools[l] || !aligned16(k_pools[l]) || !aligned16(v_pools[l]))
            return PKV_EINVAL;
    if (num_pairs == 0)
        return PKV_OK;
    if (!src_blocks || !dst_blocks || ((uintptr_t)src_blocks & 3u) || ((uintptr_t)dst_blocks & 3u))
        return PKV_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_copies(src_blocks, dst_blocks, num_pairs, num_blocks, st);
        if (rc)
            return rc;
    }
    const int64_t slab = (int64_t)num_kv_heads * block_size * head_dim;
    return launch_status(pkv::launch_copy_blocks(k_pools, v_pools, num_layers, src_blocks,
                                                 dst_blocks, num_pairs, slab, st));
}

int paged_kv_copy_slots(void *const *k_pools, void *const *v_pools, int num_layers,
                        const int32_t *copies, int num_copies, int num_kv_heads, int head_dim,
                        int block_size, int64_t num_blocks, int dtype, void *stream)
{
    if (!k_pools || !v_pools || num_layers <= 0 || num_copies < 0)
        return PKV_EINVAL;
    if (num_layers > pkv::kMaxCopyLayers)
        return PKV_ENOTSUP;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, 1, num_blocks, dtype);
    if (rc)
        return rc;
    if (num_kv_heads > (1 << 24))  // the grid's x dimension is heads x chunks
        return PKV_EINVAL;
    for (int l = 0; l < num_layers; ++l)
        if (!k_pools[l] || !v_pools[l] || !aligned16(k_pools[l]) || !aligned16(v_pools[l]))
            return PKV_EINVAL;
    if (num_copies == 0)
        return PKV_OK;
    if (!copies || ((uintptr_t)copies & 3u))
        return PKV_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_slot_copies(copies, num_copies, block_size, num_blocks, st);
        if (rc)
            return rc;
    }
    return launch_status(pkv::launch_copy_slots(k_pools, v_pools, num_layers, copies, num_copies,
                                                num_kv_heads, block_size, st));
}

}  // extern "C"

namespace {

// Shared by the decode entry points: validation, then one launch.  With k_new
// non-null the kernel also performs the step's append (fused mode).
// Shared-prefix arguments of paged_attention_prefix_decode (null group_cu for the
// other entry points).
struct PrefixGroups {
    const int32_t *group_cu = nullptr;
    const int32_t *prefix_lens = nullptr;
    int num_groups = 0;
    int suffix_partition = 0;  // > 0: the suffix pass in split mode (counters required)
};

// Work-groups per (sequence, KV head) in split mode: enough for about
// kTargetGroups work-groups in total, never more than the partitions a full table
// row could hold.  Each work-group strides over its item's partitions, so the
// result does not depend on this choice -- only the parallelism does (sizing the
// grid by the table width would launch mostly empty work-groups when contexts
// are much shorter than the row).
int split_parts(int64_t items, int need)
{
    constexpr int64_t kTargetGroups = 2048;
    const int64_t want = items > 0 ? (kTargetGroups + items - 1) / items : 1;
    return (int)(want < need ? want : need);
}

int decode_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                const void *k_new, const void *v_new, int64_t *slot_out,
                const int32_t *block_tables, const int32_t *context_lens, int num_seqs,
                int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                int max_blocks_per_seq, int64_t num_blocks, float scale, int partition_size,
                int max_partitions, float *part_o, float *part_lse, int dtype, void *stream,
                const PrefixGroups &pg = PrefixGroups(), int32_t *counters = nullptr,
                bool validate_only = false, const int32_t *seq_order = nullptr)
{
    const bool prefix = pg.group_cu != nullptr;
    if (seq_order && (((uintptr_t)seq_order & 3u) || prefix))
        return PKV_EINVAL;
    if (!q || !k_pool || !v_pool || !block_tables || !context_lens)
        return PKV_EINVAL;
    if (num_seqs < 0 || num_q_heads <= 0 || partition_size < 0)
        return PKV_EINVAL;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                              dtype);
    if (rc)
        return rc;
    if (num_q_heads % num_kv_heads != 0)
        return PKV_EINVAL;
    const int group = num_q_heads / num_kv_heads;
    if (group > 16)
        return PKV_ENOTSUP;
    if (!resolve_scale(scale, head_dim))
        return PKV_EINVAL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PKV_EINVAL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slot_out & 7u)))
        return PKV_EINVAL;
    if (counters && ((prefix && pg.suffix_partition <= 0) || partition_size <= 0 || !out ||
                     ((uintptr_t)out & 7u) || ((uintptr_t)counters & 3u)))
        return PKV_EINVAL;
    if (prefix && pg.suffix_partition != 0 && (!counters || pg.suffix_partition < 0 ||
                                                 pg.suffix_partition % 16 != 0))
        return PKV_EINVAL;
    int parts = 1;
    int prefix_part = 0, prefix_parts = 0;
    if (prefix) {
        // partition_size splits each group's prefix (0: one partition); the
        // suffix is a single pass that writes `out`
        if (!pg.prefix_lens || pg.num_groups <= 0 || (num_seqs > 0 && pg.num_groups > num_seqs))
            return PKV_EINVAL;
        if (((uintptr_t)pg.group_cu & 3u) || ((uintptr_t)pg.prefix_lens & 3u))
            return PKV_EINVAL;
        if (partition_size % 16 != 0)
            return PKV_EINVAL;
        const int64_t ctx = (int64_t)max_blocks_per_seq * block_size;
        if (ctx > ((int64_t)1 << 29))
            return PKV_EINVAL;
        if (partition_size > 0) {
            // two passes: prefix partitions into the workspace, then the suffixes
            // (in split mode their partitions follow the prefix partitions)
            prefix_part = partition_size;
            const int64_t need = (ctx + prefix_part - 1) / prefix_part;
            const int64_t need_suffix =
                pg.suffix_partition > 0 ? (ctx + pg.suffix_partition - 1) / pg.suffix_partition
                                        : 0;
            if (!part_o || !part_lse || max_partitions < need + need_suffix || need <= 0)
                return PKV_EWORKSPACE;
            if (!aligned16(part_o) || ((uintptr_t)part_lse & 3u))
                return PKV_EINVAL;
            if (pg.suffix_partition > 0 &&
                (int64_t)num_seqs * num_q_heads * max_partitions * head_dim * 4 > (int64_t)INT32_MAX)
                return PKV_EWORKSPACE;
            prefix_parts = (int)need;
            if (pg.suffix_partition > 0)
                parts = split_parts((int64_t)num_seqs * num_kv_heads, (int)need_suffix);
        } else if (pg.suffix_partition > 0) {
            return PKV_EINVAL;  // the suffix is split only in the two-pass form
        }
        if (!out || ((uintptr_t)out & 7u))
            return PKV_EINVAL;
    } else if (partition_size > 0) {
        if (partition_size % block_size != 0)
            return PKV_EINVAL;
        const int need = pkv_max_partitions(max_blocks_per_seq, block_size, partition_size);
        if (!part_o || !part_lse || max_partitions < need || need <= 0)
            return PKV_EWORKSPACE;
        if (!aligned16(part_o) || ((uintptr_t)part_lse & 3u))
            return PKV_EINVAL;
        parts = split_parts((int64_t)num_seqs * num_kv_heads, need);
        // the merged mode addresses the workspace with 31-bit byte offsets
        if (counters && (int64_t)num_seqs * num_q_heads * max_partitions * head_dim * 4 >
                            (int64_t)INT32_MAX)
            return PKV_EWORKSPACE;
    } else {
        if (!out || ((uintptr_t)out & 1u))
            return PKV_EINVAL;
    }
    const int64_t items = (int64_t)num_seqs * num_kv_heads * parts;
    if (items > INT32_MAX)
        return PKV_EINVAL;
    if (items == 0 || validate_only)
        return PKV_OK;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_tables(block_tables, context_lens, num_seqs, max_blocks_per_seq,
                                     block_size, num_blocks, st);
        if (rc == PKV_OK && prefix)
            rc = pkv::debug_check_groups(pg.group_cu, pg.prefix_lens, context_lens,
                                         pg.num_groups, num_seqs, k_new ? 1 : 0, st);
        if (rc == PKV_OK && seq_order)
            rc = pkv::debug_check_order(seq_order, num_seqs, st);
        if (rc)
            return rc;
    }
    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.tables = block_tables;
    a.lens = context_lens;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.width = max_blocks_per_seq;
    a.partition_size = partition_size;
    a.max_partitions = partition_size > 0 ? max_partitions : 0;
    a.parts_per_item = parts;
    a.n_items = (int)items;
    a.scale_log2 = scale * pkv::kLog2e;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_out = slot_out;
    a.block_size = block_size;
    a.counters = counters;
    a.seq_order = seq_order;
    if (prefix && partition_size == 0) {
        // one pass: each work-group streams its tile's prefix, then each member's
        // own positions, and writes `out`
        a.partition_size = 0;
        a.group_cu = pg.group_cu;
        a.prefix_lens = pg.prefix_lens;
        a.num_groups = pg.num_groups;
        a.seqs_per_tile = pkv::kPrefixHalves * (16 / group);
        const int64_t tiles = (num_seqs + a.seqs_per_tile - 1) / a.seqs_per_tile;
        const int64_t fitems = tiles * num_kv_heads;
        if (fitems > INT32_MAX)
            return PKV_EINVAL;
        return launch_status(
            pkv::launch_prefix_fused_mfma(a, (int)fitems, dtype, block_size, st));
    }
    if (prefix) {
        // pass 1: each group's prefix partitions, read once per 16-row tile of its
        // query heads; pass 2: each sequence's own positions, merged with the
        // prefix partials
        a.partition_size = 0;
        a.max_partitions = max_partitions;  // the workspace's row stride
        a.group_cu = pg.group_cu;
        a.prefix_lens = pg.prefix_lens;
        a.num_groups = pg.num_groups;
        a.prefix_part = prefix_part;
        a.seqs_per_tile = 16 / group;
        const int64_t tiles = (num_seqs + a.seqs_per_tile - 1) / a.seqs_per_tile;
        const int64_t pitems = tiles * num_kv_heads * prefix_parts;
        if (pitems > INT32_MAX)
            return PKV_EINVAL;
        a.parts_per_item = prefix_parts;  // prefix partitions per (tile, KV head)
        hipError_t e = pkv::launch_prefix_mfma(a, (int)pitems, dtype, block_size, st);
        if (e != hipSuccess)
            return PKV_ELAUNCH;
        // the suffix pass: one work-group per (sequence, KV head), or `parts` of them
        // over partitions of the suffix merged in the launch
        a.parts_per_item = parts;
        if (pg.suffix_partition > 0)
            a.partition_size = pg.suffix_partition;
        return launch_status(pkv::launch_decode_mfma(a, dtype, block_size, st));
    }
    const hipError_t e = group == 1 ? pkv::launch_decode_g1(a, dtype, block_size, st)
                                    : pkv::launch_decode_mfma(a, dtype, block_size, st);
    return launch_status(e);
}

}  // namespace

extern "C" {

int paged_attention_decode(void *out, const void *q, const void *k_pool, const void *v_pool,
                           const int32_t *block_tables, const int32_t *context_lens,
                           int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int max_blocks_per_seq, int64_t num_blocks,
                           float scale, int partition_size, int max_partitions, float *part_o,
                           float *part_lse, int dtype, void *stream)
{
    return decode_impl(out, q, k_pool, v_pool, nullptr, nullptr, nullptr, block_tables,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, scale, partition_size, max_partitions,
                       part_o, part_lse, dtype, stream);
}

int paged_attention_append_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                  const void *k_new, const void *v_new, int64_t *slot_out,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int64_t num_blocks,
                                  float scale, int partition_size, int max_partitions,
                                  float *part_o, float *part_lse, int dtype, void *stream)
{
    if (!k_new || !v_new)
        return PKV_EINVAL;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, slot_out, block_tables,
                       context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                       max_blocks_per_seq, num_blocks, scale, partition_size, max_partitions,
                       part_o, part_lse, dtype, stream);
}

int paged_attention_split_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                 const void *k_new, const void *v_new, int64_t *slot_out,
                                 const int32_t *block_tables, const int32_t *context_lens,
                                 int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int64_t num_blocks,
                                 float scale, int partition_size, int max_partitions,
                                 float *part_o, float *part_lse, int32_t *counters, int dtype,
                                 void *stream)
{
    if (!counters || !out || partition_size <= 0)
        return PKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                       block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, partition_size,
                       max_partitions, part_o, part_lse, dtype, stream, PrefixGroups(), counters);
}

int paged_attention_decode_ordered(void *out, const void *q, void *k_pool, void *v_pool,
                                   const void *k_new, const void *v_new, int64_t *slot_out,
                                   const int32_t *block_tables, const int32_t *context_lens,
                                   const int32_t *seq_order, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int max_blocks_per_seq, int64_t num_blocks, float scale,
                                   int dtype, void *stream)
{
    if (!seq_order || !out)
        return PKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                       block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, 0, 0, nullptr, nullptr,
                       dtype, stream, PrefixGroups(), nullptr, false, seq_order);
}

}  // extern "C"

// ---- the entry point that allocates nothing -------------------------------------
// paged_attention_split_decode_noalloc keeps the partials and the arrival
// counters of paged_attention_split_decode in this file-scope device array
// instead of a caller workspace: the arrival counters first, then the partials'
// lse values, then their rows (byte offsets 256-aligned).  Every GPU the library
// runs on holds its own copy until the process ends.
namespace {

constexpr int64_t kNoAllocItems = (int64_t)1 << 16;     // (sequence, KV head) counters
constexpr int64_t kNoAllocRows = (int64_t)1 << 15;      // (sequence, query head, partition) rows
constexpr int64_t kNoAllocLseOff = kNoAllocItems * 4;  // 256 KiB
constexpr int64_t kNoAllocRowOff = kNoAllocLseOff + kNoAllocRows * 4;
constexpr int64_t kScratchBytes = kNoAllocRowOff + kNoAllocRows * pkv::kHeadDim * 4;  // 16.4 MiB
static_assert(kNoAllocLseOff % 256 == 0 && kNoAllocRowOff % 256 == 0, "aligned regions");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` per device, resolved once per device (with that
// device current) by hipGetSymbolAddress.  In host code the array's name is only
// a host-side stand-in: the address used everywhere is the one resolved here.
constexpr int kMaxDevices = 64;
std::atomic<unsigned char *> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

__global__ void clear_counters_kernel(int32_t *c, int n)
{
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
        c[i] = 0;
}

// The current device's scratch, set up on its first use: the address is resolved
// and the arrival counters are cleared by a kernel on `stream` (every completed
// call leaves them zero afterwards).
int scratch_of_current_device(hipStream_t stream, unsigned char **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return PKV_ELAUNCH;
    if (dev < 0 || dev >= kMaxDevices)
        return PKV_ENOTSUP;
    unsigned char *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p) {
        *out = p;
        return PKV_OK;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        void *addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr)
            return PKV_ELAUNCH;
        p = (unsigned char *)addr;
        hipLaunchKernelGGL(clear_counters_kernel, dim3(64), dim3(256), 0, stream, (int32_t *)p,
                           (int)kNoAllocItems);
        if (hipGetLastError() != hipSuccess)
            return PKV_ELAUNCH;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PKV_OK;
}

}  // namespace

extern "C" {

int paged_attention_split_decode_noalloc(void *out, const void *q, void *k_pool, void *v_pool,
                                         const void *k_new, const void *v_new,
                                         int64_t *slot_out, const int32_t *block_tables,
                                         const int32_t *context_lens, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_blocks_per_seq,
                                         int64_t num_blocks, float scale, int partition_size,
                                         int dtype, void *stream)
{
    if (!out || partition_size <= 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0)
        return PKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    const int mp = pkv_max_partitions(max_blocks_per_seq, block_size, partition_size);
    if (mp <= 0)
        return PKV_EINVAL;
    if ((int64_t)num_seqs * num_kv_heads > kNoAllocItems ||
        (int64_t)num_seqs * num_q_heads * mp > kNoAllocRows)
        return PKV_EWORKSPACE;
    // every argument is checked before the device is touched (placeholder
    // workspace addresses: validation does not dereference them)
    float *const ph = (float *)(uintptr_t)256;
    int rc = decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                         block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                         head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                         partition_size, mp, ph, ph, dtype, stream, PrefixGroups(),
                         (int32_t *)ph, true);
    if (rc != PKV_OK || num_seqs == 0)
        return rc;
    unsigned char *base = nullptr;
    rc = scratch_of_current_device((hipStream_t)stream, &base);
    if (rc != PKV_OK)
        return rc;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                       block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, partition_size, mp,
                       (float *)(base + kNoAllocRowOff), (float *)(base + kNoAllocLseOff), dtype,
                       stream, PrefixGroups(), (int32_t *)base);
}

int paged_attention_prefix_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                  const void *k_new, const void *v_new, int64_t *slot_out,
                                  const int32_t *block_tables, const int32_t *context_lens,
                                  const int32_t *group_cu, const int32_t *prefix_lens,
                                  int num_groups, int num_seqs, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size,
                                  int max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int prefix_partition, int max_partitions, float *part_o,
                                  float *part_lse, int dtype, void *stream)
{
    if (!group_cu)
        return PKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    PrefixGroups pg;
    pg.group_cu = group_cu;
    pg.prefix_lens = prefix_lens;
    pg.num_groups = num_groups;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                       block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, prefix_partition,
                       max_partitions, part_o, part_lse, dtype, stream, pg);
}

int paged_attention_prefix_split_decode(void *out, const void *q, void *k_pool, void *v_pool,
                                        const void *k_new, const void *v_new, int64_t *slot_out,
                                        const int32_t *block_tables, const int32_t *context_lens,
                                        const int32_t *group_cu, const int32_t *prefix_lens,
                                        int num_groups, int num_seqs, int num_q_heads,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int max_blocks_per_seq, int64_t num_blocks, float scale,
                                        int prefix_partition, int suffix_partition,
                                        int max_partitions, float *part_o, float *part_lse,
                                        int32_t *counters, int dtype, void *stream)
{
    if (!group_cu || !counters || prefix_partition <= 0 || suffix_partition <= 0)
        return PKV_EINVAL;
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    PrefixGroups pg;
    pg.group_cu = group_cu;
    pg.prefix_lens = prefix_lens;
    pg.num_groups = num_groups;
    pg.suffix_partition = suffix_partition;
    return decode_impl(out, q, k_pool, v_pool, k_new, v_new, k_new ? slot_out : nullptr,
                       block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads, head_dim,
                       block_size, max_blocks_per_seq, num_blocks, scale, prefix_partition,
                       max_partitions, part_o, part_lse, dtype, stream, pg, counters);
}

}  // extern "C"

namespace {

// Shared by the slotted entry points: validation, then one launch.  With
// partition_size > 0 the split kernel runs (counters and workspace required).
int slotted_impl(void *out, const void *q, const void *k_pool, const void *v_pool,
                 const int32_t *segments, const int32_t *num_segments, int num_seqs,
                 int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_segments, int64_t num_blocks, float scale, int partition_size,
                 int max_partitions, float *part_o, float *part_lse, int32_t *counters, int dtype,
                 void *stream, const void *k_new = nullptr, const void *v_new = nullptr,
                 int64_t *slot_out = nullptr)
{
    if ((k_new == nullptr) != (v_new == nullptr))
        return PKV_EINVAL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slot_out & 7u)))
        return PKV_EINVAL;
    if (!out || !q || !k_pool || !v_pool || !segments || !num_segments)
        return PKV_EINVAL;
    if (num_seqs < 0 || num_q_heads <= 0 || max_segments <= 0 || partition_size < 0)
        return PKV_EINVAL;
    int rc = check_pool_shape(num_kv_heads, head_dim, block_size, 1, num_blocks, dtype);
    if (rc)
        return rc;
    if (num_q_heads % num_kv_heads != 0)
        return PKV_EINVAL;
    if (num_q_heads / num_kv_heads > 16)
        return PKV_ENOTSUP;
    if (!resolve_scale(scale, head_dim))
        return PKV_EINVAL;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || ((uintptr_t)out & 7u) ||
        ((uintptr_t)segments & 3u) || ((uintptr_t)num_segments & 3u))
        return PKV_EINVAL;
    if ((int64_t)max_segments * 3 * num_seqs > ((int64_t)1 << 40))
        return PKV_EINVAL;
    // a sequence's positions (at most max_segments x block_size) fit in 31 bits
    if ((int64_t)max_segments * block_size > ((int64_t)1 << 30))
        return PKV_EINVAL;
    int parts = 1;
    if (partition_size > 0) {
        if (partition_size % 16 != 0 || !counters || ((uintptr_t)counters & 3u))
            return PKV_EINVAL;
        const int64_t need64 =
            ((int64_t)max_segments * block_size + partition_size - 1) / partition_size;
        if (!part_o || !part_lse || max_partitions < need64)
            return PKV_EWORKSPACE;
        if (!aligned16(part_o) || ((uintptr_t)part_lse & 3u))
            return PKV_EINVAL;
        if ((int64_t)num_seqs * num_q_heads * max_partitions * head_dim * 4 > (int64_t)INT32_MAX)
            return PKV_EWORKSPACE;
        parts = split_parts((int64_t)num_seqs * num_kv_heads, (int)need64);
    }
    const int64_t items = (int64_t)num_seqs * num_kv_heads * parts;
    if (items > INT32_MAX)
        return PKV_EINVAL;
    if (items == 0)
        return PKV_OK;
    hipStream_t st = (hipStream_t)stream;
    if (debug_enabled()) {
        rc = pkv::debug_check_segments(segments, num_segments, num_seqs, max_segments, block_size,
                                       num_blocks, st);
        if (rc)
            return rc;
    }
    pkv::DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = num_kv_heads;
    a.n_items = (int)items;
    a.scale_log2 = scale * pkv::kLog2e;
    a.block_size = block_size;
    a.segments = segments;
    a.num_segments = num_segments;
    a.max_segments = max_segments;
    a.k_new = k_new;
    a.v_new = v_new;
    a.slot_out = k_new ? slot_out : nullptr;
    if (partition_size > 0) {
        a.partition_size = partition_size;
        a.max_partitions = max_partitions;
        a.parts_per_item = parts;
        a.part_o = part_o;
        a.part_lse = part_lse;
        a.counters = counters;
        return launch_status(pkv::launch_slotted_mfma(a, dtype, block_size, st));
    }
    // Tiles of consecutive sequences read their common leading segments once; they
    // need the whole list of a tile's sub-tiles in LDS, so a batch whose worst-case
    // tile exceeds it runs one work-group per sequence.  Tiles also cut the number
    // of work-groups by the sequences per tile (up to 32), which only pays when
    // sequences share segments: the host cannot see the segments, so by default
    // tiles are taken only while they still give at least half as many
    // work-groups as min(per-sequence work-groups, compute units).
    const int spt = pkv::kPrefixHalves * (16 / (num_q_heads / num_kv_heads));
    const int64_t tile_subs = (int64_t)spt * max_segments * ((block_size + 15) / 16);
    const int64_t tiles = (num_seqs + spt - 1) / spt;
    const int mode = slotted_tiles_mode();
    bool use_tiles = mode != 0 && tile_subs <= pkv::kSlottedTileSubs;
    if (use_tiles && mode == 2) {
        const int64_t per_seq = (int64_t)num_seqs * num_kv_heads;
        const int64_t cap = per_seq < device_cu_count() ? per_seq : device_cu_count();
        use_tiles = 2 * tiles * num_kv_heads >= cap;
    }
    if (use_tiles) {
        a.seqs_per_tile = spt;
        return launch_status(pkv::launch_slotted_tiled_mfma(a, (int)(tiles * num_kv_heads),
                                                            dtype, block_size, st));
    }
    return launch_status(pkv::launch_slotted_mfma(a, dtype, block_size, st));
}

}  // namespace

extern "C" {

int paged_attention_decode_slotted(void *out, const void *q, const void *k_pool,
                                   const void *v_pool, const int32_t *segments,
                                   const int32_t *num_segments, int num_seqs, int num_q_heads,
                                   int num_kv_heads, int head_dim, int block_size,
                                   int max_segments, int64_t num_blocks, float scale, int dtype,
                                   void *stream)
{
    return slotted_impl(out, q, k_pool, v_pool, segments, num_segments, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, max_segments, num_blocks, scale, 0, 0,
                        nullptr, nullptr, nullptr, dtype, stream);
}

int paged_attention_append_decode_slotted(void *out, const void *q, void *k_pool, void *v_pool,
                                          const void *k_new, const void *v_new,
                                          int64_t *slot_out, const int32_t *segments,
                                          const int32_t *num_segments, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int max_segments, int64_t num_blocks,
                                          float scale, int dtype, void *stream)
{
    if (!k_new || !v_new)
        return PKV_EINVAL;
    return slotted_impl(out, q, k_pool, v_pool, segments, num_segments, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, max_segments, num_blocks, scale, 0, 0,
                        nullptr, nullptr, nullptr, dtype, stream, k_new, v_new, slot_out);
}

int paged_attention_append_decode_slotted_split(
    void *out, const void *q, void *k_pool, void *v_pool, const void *k_new, const void *v_new,
    int64_t *slot_out, const int32_t *segments, const int32_t *num_segments, int num_seqs,
    int num_q_heads, int num_kv_heads, int head_dim, int block_size, int max_segments,
    int64_t num_blocks, float scale, int partition_size, int max_partitions, float *part_o,
    float *part_lse, int32_t *counters, int dtype, void *stream)
{
    if (!k_new || !v_new || partition_size <= 0)
        return PKV_EINVAL;
    return slotted_impl(out, q, k_pool, v_pool, segments, num_segments, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, max_segments, num_blocks, scale,
                        partition_size, max_partitions, part_o, part_lse, counters, dtype, stream,
                        k_new, v_new, slot_out);
}

int paged_attention_decode_slotted_split(void *out, const void *q, const void *k_pool,
                                         const void *v_pool, const int32_t *segments,
                                         const int32_t *num_segments, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim,
                                         int block_size, int max_segments, int64_t num_blocks,
                                         float scale, int partition_size, int max_partitions,
                                         float *part_o, float *part_lse, int32_t *counters,
                                         int dtype, void *stream)
{
    if (partition_size <= 0)
        return PKV_EINVAL;
    return slotted_impl(out, q, k_pool, v_pool, segments, num_segments, num_seqs, num_q_heads,
                        num_kv_heads, head_dim, block_size, max_segments, num_blocks, scale,
                        partition_size, max_partitions, part_o, part_lse, counters, dtype, stream);
}

int paged_attention_reduce(void *out, const float *part_o, const float *part_lse,
                           const int32_t *context_lens, int num_seqs, int num_q_heads,
                           int head_dim, int partition_size, int max_partitions, int dtype,
                           void *stream)
{
    if (!out || !part_o || !part_lse || !context_lens)
        return PKV_EINVAL;
    if (num_seqs < 0 || num_q_heads <= 0 || partition_size <= 0 || max_partitions <= 0)
        return PKV_EINVAL;
    if (dtype != PKV_FP16 && dtype != PKV_BF16)
        return PKV_ENOTSUP;
    if (head_dim != pkv::kHeadDim)
        return PKV_ENOTSUP;
    if (((uintptr_t)out & 3u) || ((uintptr_t)part_o & 7u) || ((uintptr_t)part_lse & 3u))
        return PKV_EINVAL;
    const int64_t waves = (int64_t)num_seqs * num_q_heads;
    if (waves > INT32_MAX / 64)
        return PKV_EINVAL;
    if (waves == 0)
        return PKV_OK;
    return launch_status(pkv::launch_reduce(out, part_o, part_lse, context_lens, num_seqs,
                                            num_q_heads, partition_size, max_partitions, dtype,
                                            (hipStream_t)stream));
}

}  // extern "C"
