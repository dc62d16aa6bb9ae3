// copy.hip -- copy-on-write block duplication, and the split of a shared slot.
//
// When a branch is about to append to a partly filled block that another branch
// still references, the block manager gives the branch a fresh physical block
// holding a deep copy of the shared one and repoints that branch's table entry
// (page "显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结", blog.llmgo.top,
// §四, copy-on-write steps 1-3).  A block id names the same block in every layer,
// so the copy runs over every layer's K and V pools.
//
// gfx950 design: in the [NB][Hkv][B][D] layout one block of one pool is a single
// contiguous slab of Hkv*B*D elements, so a copy is a set of slab-to-slab moves
// with no address walk.  Each work-group moves 16 KiB of one slab (256 lanes x
// four 16-byte loads in flight, then four 16-byte stores), the grid spans
// (slab chunk, pair, layer x {K, V}); pair ids are read with scalar loads.
// Loads and stores are nontemporal: a copy neither reads its source again nor
// its destination soon, and keeping both out of the caches measured 5.4 TB/s
// against 5.1 TB/s with cached stores (512 KiB blocks, MI355X).
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;
constexpr int kCopyVecPerGroup = kCopyThreads * kCopyUnroll;  // 16-byte vectors per group

struct CopyArgs {
    const int32_t *src;
    const int32_t *dst;
    int64_t slab_vec;  // 16-byte vectors per block slab
    int num_pairs;
    u32x4 *pools[2 * kMaxCopyLayers];  // layer l: K at 2l, V at 2l+1
};

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a)
{
    u32x4 *pool = a.pools[blockIdx.z];
    const int64_t v0 = (int64_t)blockIdx.x * kCopyVecPerGroup + threadIdx.x;
    for (int p = blockIdx.y; p < a.num_pairs; p += gridDim.y) {
        const u32x4 *from = pool + (int64_t)a.src[p] * a.slab_vec;
        u32x4 *to = pool + (int64_t)a.dst[p] * a.slab_vec;
        u32x4 r[kCopyUnroll];
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) {
            const int64_t v = v0 + j * kCopyThreads;
            if (v < a.slab_vec)
                r[j] = ldnt(from + v);
        }
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) {
            const int64_t v = v0 + j * kCopyThreads;
            if (v < a.slab_vec)
                __builtin_nontemporal_store(r[j], to + v);
        }
    }
}

// Copy-on-write split of a shared slot: a node held in rows [so, so + len) of a
// block shared with other nodes is moved to rows [do, do + len) of a block of
// its own before it is appended to, leaving the shared slots read-only (mhpq.cn
// Radix-Tree page, "核心设计原则", copy-on-write on append).  In the pool layout
// the node's rows of one KV head are len * 256 contiguous bytes, so each
// (copy, head) is one contiguous move: a work-group takes up to 1,024 16-byte
// vectors of it (four loads in flight per lane, then the stores); the grid spans
// (head x chunk, copy, layer x {K, V}) and the copy tuple is read with scalar
// loads.  Offsets and lengths are clamped to the block, so a bad tuple cannot
// reach another block's rows.
struct SlotCopyArgs {
    const int32_t *copies;  // [num_copies][5]: src block, src offset, dst block, dst offset, len
    int num_copies, num_kv_heads, block_size;
    int chunks;             // work-groups per (copy, head): ceil(block_size * 16 / 1024)
    u32x4 *pools[2 * kMaxCopyLayers];
};

__global__ __launch_bounds__(kCopyThreads) void copy_slots_kernel(SlotCopyArgs a)
{
    u32x4 *pool = a.pools[blockIdx.z];
    const int h = blockIdx.x / a.chunks;
    const int v0 = (blockIdx.x % a.chunks) * kCopyVecPerGroup + threadIdx.x;
    constexpr int kVecPerRow = kHeadDim * 2 / 16;
    for (int i = blockIdx.y; i < a.num_copies; i += gridDim.y) {
        const meta_ptr c = as_meta(a.copies) + 5 * (int64_t)i;
        const int B = a.block_size;
        const int so = min(max(c[1], 0), B), dof = min(max(c[3], 0), B);
        const int len = min(max(c[4], 0), min(B - so, B - dof));
        const int64_t from = (((int64_t)c[0] * a.num_kv_heads + h) * B + so) * kVecPerRow;
        const int64_t to = (((int64_t)c[2] * a.num_kv_heads + h) * B + dof) * kVecPerRow;
        const int nv = len * kVecPerRow;
        u32x4 r[kCopyUnroll];
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) {
            const int v = v0 + j * kCopyThreads;
            if (v < nv)
                r[j] = ldnt(pool + from + v);
        }
#pragma unroll
        for (int j = 0; j < kCopyUnroll; ++j) {
            const int v = v0 + j * kCopyThreads;
            if (v < nv)
                __builtin_nontemporal_store(r[j], pool + to + v);
        }
    }
}

}  // namespace

hipError_t launch_copy_slots(void *const *k_pools, void *const *v_pools, int num_layers,
                             const int32_t *copies, int num_copies, int num_kv_heads,
                             int block_size, hipStream_t stream)
{
    SlotCopyArgs a{};
    a.copies = copies;
    a.num_copies = num_copies;
    a.num_kv_heads = num_kv_heads;
    a.block_size = block_size;
    a.chunks = (block_size * (kHeadDim * 2 / 16) + kCopyVecPerGroup - 1) / kCopyVecPerGroup;
    for (int l = 0; l < num_layers; ++l) {
        a.pools[2 * l] = (u32x4 *)k_pools[l];
        a.pools[2 * l + 1] = (u32x4 *)v_pools[l];
    }
    const int gy = num_copies < 65535 ? num_copies : 65535;
    hipLaunchKernelGGL(copy_slots_kernel,
                       dim3((unsigned)(num_kv_heads * a.chunks), (unsigned)gy, 2u * num_layers),
                       dim3(kCopyThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void *const *k_pools, void *const *v_pools, int num_layers,
                              const int32_t *src, const int32_t *dst, int num_pairs,
                              int64_t slab_elems, hipStream_t stream)
{
    CopyArgs a{};
    a.src = src;
    a.dst = dst;
    a.slab_vec = slab_elems / 8;
    a.num_pairs = num_pairs;
    for (int l = 0; l < num_layers; ++l) {
        a.pools[2 * l] = (u32x4 *)k_pools[l];
        a.pools[2 * l + 1] = (u32x4 *)v_pools[l];
    }
    const int64_t gx = (a.slab_vec + kCopyVecPerGroup - 1) / kCopyVecPerGroup;
    const int gy = num_pairs < 65535 ? num_pairs : 65535;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)gx, (unsigned)gy, 2u * num_layers),
                       dim3(kCopyThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
