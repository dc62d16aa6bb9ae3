// pkv_device.h -- device-side helpers shared by the gfx950 kernels of libpagedkv.
//
// Pool layout used by every kernel (one K pool and one V pool per layer):
//   [num_blocks][num_kv_heads][block_size][head_dim], head_dim contiguous.
// Token t of a sequence lives in physical block table[t / block_size] at offset
// t % block_size (page "端侧 SLM 显存保活术：在 4GB 内存板卡上实现轻量 PagedAttention
// 与 KV 缓存分块", pwwt.cn, section "注意力寻址").  Element offsets are formed in
// 64-bit: a 7B-shaped layer pool holds more than 2^31 elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDim = 128;   // the only head size the kernels are built for
constexpr int kNumXcd = 8;      // MI355X: 8 accelerator complex dies, each with its own L2
constexpr int kFp16 = 0;
constexpr int kBf16 = 1;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---- 16-bit storage formats -------------------------------------------------
// Widen the low / high 16-bit half of a dword to fp32.
template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w)
{
    if constexpr (DT == kFp16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    else
        return __uint_as_float(w << 16);
}
template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w)
{
    if constexpr (DT == kFp16)
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    else
        return __uint_as_float(w & 0xFFFF0000u);
}

// fp32 -> 16-bit pattern, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t to_bits(float x)
{
    if constexpr (DT == kFp16)
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    else
        return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// c + a.lo*b.lo + a.hi*b.hi on packed 16-bit pairs, fp32 accumulate.
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (DT == kFp16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                      c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c, false);
}

// K/V tiles are read exactly once per step: stream them with nontemporal loads,
// which on MI355X sustain a markedly higher HBM read rate than default-policy loads
// (about 7.0 vs 6.2 TB/s measured for 8 KiB chunks in random order).
__device__ __forceinline__ u32x4 ldnt(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// Buffer resource over [base, base + bytes): a buffer load whose offset falls
// outside the range returns zeros without touching memory.  Used for the rows
// of a block that lie past the context length, so that they cost no HBM traffic.
// Word 3 of the descriptor is the gfx9-family default (32-bit data format, no
// swizzle), the base must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                             0x00020000);
}

// Cache policies of the buffer loads: data read once per step streams past the
// caches (nontemporal); data many work-groups re-read (a shared prefix) keeps the
// default policy so that the re-reads hit L2.
constexpr int kLoadStream = 2;  // nt
constexpr int kLoadReuse = 0;   // default

// 16-byte buffer load at byte offset `off` (0 beyond the range).
template <int CPOL = kLoadStream>
__device__ __forceinline__ u32x4 ldbuf(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL);
}

// ---- cross-lane -------------------------------------------------------------
// DPP row operations act inside rows of 16 lanes.  The four steps below give
// every lane of a row the same sum (each step adds a value and its mirror, and
// fp32 addition is commutative, so all 16 lanes agree bit for bit).
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_sum16(float x)
{
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);  // row_half_mirror
    x += dpp<0x140>(x);  // row_mirror
    return x;
}

__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Maximum of scores and running maxima, which are never signalling NaNs: the
// hardware max directly.  fmaxf makes the compiler quiet every operand it cannot
// prove canonical (a lane-swapped or selected value) with an extra v_max_f32
// x, x, x first, which cost 12 VALU operations per 16-token step of the GQA
// kernels' softmax.
__device__ __forceinline__ float vmax(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c)
{
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Max / sum over lanes l and l^16 (or l^32), the same bits in both lanes of the
// pair.  The gfx950 lane-swap instructions hand every lane both values of its
// pair in one VALU operation (lane layout checked on the GPU with an in-bounds
// probe: swap16(x, x) gives {x[l & ~16], x[l | 16]}, swap32 likewise with 32),
// where a shuffle would round-trip through the LDS crossbar.
__device__ __forceinline__ float pair_max16(float x)
{
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return vmax(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float pair_max32(float x)
{
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return vmax(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float pair_sum16(float x)
{
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
__device__ __forceinline__ float pair_sum32(float x)
{
    const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float flog2(float x) { return __builtin_amdgcn_logf(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Reference point for exp2 in the running softmax: the running max, or 0 while no
// token has been seen (so that exp2(-inf - ref) = 0 instead of NaN).
__device__ __forceinline__ float safe_ref(float m) { return m == kNegInf ? 0.f : m; }

// Work-group index -> work item, arranged so that each XCD (work-groups are dealt
// to the 8 XCDs round-robin) receives a contiguous range of items.  Items are
// ordered KV-head major, so the work-groups sharing an L2 also share KV heads.
__device__ __forceinline__ int xcd_item(int b, int n_items)
{
    const int x = b % kNumXcd, j = b / kNumXcd;
    const int q = n_items / kNumXcd, r = n_items % kNumXcd;
    return x * q + (x < r ? x : r) + j;
}

// Read-only metadata (block tables, lengths, group bounds, segment lists) does
// not change while a kernel runs.  Read through the constant address space, a
// wave-uniform entry compiles to a scalar load, whose wait (lgkmcnt) is separate
// from the vector-memory counter.  Read through a generic pointer it becomes a
// vector load, and since vmcnt retires in order, waiting for it also waits for
// every K/V load the wave has in flight, draining the pipeline once per tile.
typedef const __attribute__((address_space(4))) int32_t *meta_ptr;
__device__ __forceinline__ meta_ptr as_meta(const int32_t *p) { return (meta_ptr)p; }

// Kernel arguments of the decode kernels.
struct DecodeArgs {
    void *out;                  // [S][Hq][D] dtype (single pass)
    const void *q;              // [S][Hq][D] dtype
    const void *k_pool;         // [NB][Hkv][B][D]
    const void *v_pool;
    const int32_t *tables;      // [S][W]
    const int32_t *lens;        // [S]
    float *part_o;              // [S][Hq][MP][D] fp32 (partitioned)
    float *part_lse;            // [S][Hq][MP]
    int num_seqs, num_q_heads, num_kv_heads, width;
    int partition_size;         // 0 = single pass
    int max_partitions;
    int parts_per_item;         // partitions launched per (sequence, kv head)
    int n_items;
    float scale_log2;           // scale * log2(e)
    // fused append (null for plain decode): the new token's rows, written to
    // position n-1 of each sequence and used in registers for that position
    const void *k_new;          // [S][Hkv][D]
    const void *v_new;
    int64_t *slot_out;          // optional [S]
    int block_size;
    // shared-prefix mode (null group_cu otherwise): sequences group_cu[k] ..
    // group_cu[k+1]-1 share their first prefix_lens[k] positions, read through
    // the table row of sequence group_cu[k]; the prefix pass leaves fp32 partials
    // of prefix partitions of prefix_part tokens in part_o / part_lse, and the
    // suffix pass attends over positions prefix_lens[k] .. n-1 and merges them
    const int32_t *group_cu;    // [num_groups + 1]
    const int32_t *prefix_lens; // [num_groups]
    int num_groups;
    int prefix_part;            // tokens per prefix partition (multiple of 16)
    int seqs_per_tile;          // prefix pass: sequences per 16-row query tile
    // slotted mode: each sequence is a list of (block id, slot offset, length)
    // segments, [num_seqs][max_segments][3], with num_segments[s] in use
    const int32_t *segments;
    const int32_t *num_segments;
    int max_segments;
    // merged split mode (null otherwise): one arrival counter per (sequence, KV
    // head); the last work-group of an item to finish merges its partitions into
    // `out` and puts the counter back to 0
    int32_t *counters;
    // optional dispatch order (null: natural): the work items of sequence
    // seq_order[i] take the place of sequence i's in the grid; entries are
    // clamped to [0, num_seqs) so that a bad order cannot reach outside the batch
    const int32_t *seq_order;
};

// The sequence whose work items sit at position i of the grid's sequence order.
__device__ __forceinline__ int ordered_seq(const DecodeArgs &a, int i)
{
    return a.seq_order ? min(max(as_meta(a.seq_order)[i], 0), a.num_seqs - 1) : i;
}

// ---- merged split mode --------------------------------------------------------
// The work-groups of one item exchange their partials through the workspace.
// The partials are written and read with the agent-coherence cache policy (sc1:
// the accesses that relaxed atomics at agent scope compile to), which the gfx950
// memory hierarchy keeps coherent across the XCDs' L2 caches by itself.
// Release / acquire fences at agent scope would instead write back and
// invalidate the whole L2 of the XCD in every work-group, which was measured to
// serialise the work-groups of an XCD (a long-context launch went from 84 to
// 111 us).  The workspace is addressed through one buffer resource, so its byte
// offsets must fit in 31 bits (the host checks it).
constexpr int kAgentCoherent = 16;  // cache policy sc1

struct Workspace {
    __amdgpu_buffer_rsrc_t o, lse;
};

__device__ __forceinline__ Workspace workspace_rsrc(const DecodeArgs &a, int64_t rows)
{
    Workspace w;
    w.o = make_rsrc(a.part_o, (int)(rows * a.max_partitions * kHeadDim * 4));
    w.lse = make_rsrc(a.part_lse, (int)(rows * a.max_partitions * 4));
    return w;
}

__device__ __forceinline__ void st_ws4(__amdgpu_buffer_rsrc_t r, int off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0,
                                           kAgentCoherent);
}
__device__ __forceinline__ void st_ws1(__amdgpu_buffer_rsrc_t r, int off, float v)
{
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, kAgentCoherent);
}
__device__ __forceinline__ f32x4 ld_ws4(__amdgpu_buffer_rsrc_t r, int off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0,
                                                                           kAgentCoherent));
}
__device__ __forceinline__ float ld_ws1(__amdgpu_buffer_rsrc_t r, int off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kAgentCoherent));
}

// Arrival of a work-group that has stored its partitions' partials (st_ws*), in
// a launch where `expected` work-groups do so for the item counted by *ctr.
// Returns true, in every thread, in the last one to arrive, which may then read
// every partial of the item (ld_ws*).  Each wave first waits until its stores
// are complete (the work-group barrier itself waits only for LDS); then one
// relaxed increment counts the work-group, and the last arrival puts the counter
// back to 0, so consecutive launches (and graph replays) need no clearing.
__device__ __forceinline__ bool arrive_last(int32_t *ctr, int expected, int32_t *s_flag)
{
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == expected - 1;
        if (last)
            __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

// Log-sum-exp merge of np >= 1 partials (natural-log lse, normalised fp32 rows) of
// one query row, for 4 consecutive dims: `lse_off` is the byte offset of the
// row's lse[0] in the workspace, `o_off` that of dims d0..d0+3 of its partition
// 0.  The same operations in the same order as the standalone merge kernel (max
// first, then the weighted sum in partition order), so both give the same bits.
// Partials are requested kMergeChunk partitions at a time, so a merge of up to
// kMergeChunk partitions costs one memory round trip.
constexpr int kMergeChunk = 8;

__device__ __forceinline__ f32x4 merge_partials4(const Workspace &ws, int lse_off, int o_off,
                                                 int np)
{
    float l0[kMergeChunk];
    f32x4 v0[kMergeChunk];
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i) {
        const int p = min(i, np - 1);  // never past the row's partitions
        l0[i] = ld_ws1(ws.lse, lse_off + 4 * p);
        v0[i] = ld_ws4(ws.o, o_off + p * kHeadDim * 4);
    }
    float M = kNegInf;
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i)
        M = i < np ? fmaxf(M, l0[i]) : M;
    for (int p0 = kMergeChunk; p0 < np; p0 += kMergeChunk) {
        float l[kMergeChunk];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i)
            l[i] = ld_ws1(ws.lse, lse_off + 4 * min(p0 + i, np - 1));
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i)
            M = p0 + i < np ? fmaxf(M, l[i]) : M;
    }
    const float ref = safe_ref(M);
    float W = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](float lp, const f32x4 &v) {
        const float wgt = fexp2((lp - ref) * kLog2e);
        W += wgt;
        o[0] += wgt * v[0];
        o[1] += wgt * v[1];
        o[2] += wgt * v[2];
        o[3] += wgt * v[3];
    };
#pragma unroll
    for (int i = 0; i < kMergeChunk; ++i)
        if (i < np)
            add(l0[i], v0[i]);
    for (int p0 = kMergeChunk; p0 < np; p0 += kMergeChunk) {
        float l[kMergeChunk];
        f32x4 v[kMergeChunk];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
            const int p = min(p0 + i, np - 1);
            l[i] = ld_ws1(ws.lse, lse_off + 4 * p);
            v[i] = ld_ws4(ws.o, o_off + p * kHeadDim * 4);
        }
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i)
            if (p0 + i < np)
                add(l[i], v[i]);
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    return o * inv;
}

// Group of sequence s in shared-prefix mode: the largest k with group_cu[k] <= s.
// `s` is uniform, so the search runs on scalar loads.
__device__ __forceinline__ int group_of(meta_ptr cu, int num_groups, int s)
{
    int lo = 0, hi = num_groups;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (cu[mid] <= s)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

}  // namespace pkv
