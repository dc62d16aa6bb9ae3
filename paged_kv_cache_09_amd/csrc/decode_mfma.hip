// decode_mfma.hip -- paged decode attention for grouped-query attention (GQA).
//
// What it computes: the G = Hq/Hkv query heads that share KV head g attend over
// the logical tokens of their sequence, each K/V row fetched through the block
// table (page "显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结",
// blog.llmgo.top, §五.1 kernel sketch; GQA compatibility in its FAQ Q3; the
// 12-query / 2-KV-head edge model of the pwwt.cn page, section "KV Cache 的物理
// 膨胀账本").
//
// gfx950 design.  A GQA group turns Q.K^T and P.V into dense tiles, so both go to
// the matrix cores (the group of G <= 16 query rows is padded to 16):
//   * a work-group is 4 wave64s; one work-group per (sequence, KV head[, partition]);
//     the waves take 16-token sub-tiles round-robin, double-buffered in VGPRs (the
//     one-pass shared-prefix kernel uses 8 waves and 32 query columns: two 16-column
//     halves, each holding floor(16/G) member sequences);
//   * scores: S^T[16 tok x 16 q] = K[16 x 128] . Q^T with four
//     v_mfma_f32_16x16x32_{f16,bf16}.  K rows are the A operand and are loaded
//     straight from HBM with 16-byte loads (lane i+16j holds 8 dims of token i);
//     Q^T is the B operand, loaded once;
//   * the accumulator layout of S^T (lane j+16k holds tokens 4k..4k+3 of query
//     row j) is exactly the B-operand layout of v_mfma_f32_16x16x16 for P^T, so
//     the probabilities feed P.V without any data movement;
//   * the V tile must enter P.V with tokens along the contraction axis, i.e.
//     transposed with respect to the pool's row-major [token][dim] layout.  It is
//     staged through LDS: coalesced 16-byte global loads, 16-byte LDS writes into
//     a padded row-major tile, then 2-byte transposing reads (a row stride of 288
//     bytes keeps the lanes of one read on distinct banks; the K tile uses the same
//     stride when it is staged);
//   * online softmax per query row in the exp2 domain: the row max is reduced
//     across the four lane groups holding the row, the running sum is kept per
//     lane and reduced once at the end; waves are merged through LDS with the
//     log-sum-exp rule.
// Masked positions (tokens >= n in the last block, stale data of reused blocks)
// get score -inf and a zeroed V row, so a NaN there cannot reach the output.
#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kSub = 16;           // tokens per sub-tile
// LDS row stride of a staged V tile, in 16-bit elements: 288 bytes = 72 dwords,
// so the 16 rows of a transposing read start 8 banks apart and one pass of 8
// rows covers all 64 banks exactly once (likewise each 256-byte row write).
constexpr int kVStride = 144;
// LDS row stride of a staged K tile, in 16-bit elements: 288 bytes (72 dwords, the
// V tile's stride), 16-byte aligned.  Measured with SQ_LDS_BANK_CONFLICT: no bank
// conflicts for the row writes and the A-operand reads, where a 272-byte stride
// cost 0.78 conflict cycles per LDS instruction.
constexpr int kKStride = 144;
// LDS of one wave's staging area: the V tile, then the K tile.
constexpr int kStageElems = kSub * kVStride + kSub * kKStride;
// LDS row stride, in floats, of the waves' fp32 partial outputs [wave][query row]
// [dim]: 132 = 4 (mod 64), so the 16 lanes of each phase of a 16-byte write or read
// start 4 banks apart and cover all 64 banks once.
constexpr int kOStride = 132;
// Lazy online softmax: a column's reference max is raised only when a score
// exceeds it by more than this many log2 units, so most sub-tiles skip the
// accumulator rescale.  Probabilities then stay below 2^8, which fp16 and bf16
// represent with the same relative precision as values below 1.
constexpr float kRescaleSlack = 8.f;

template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const u32x4 &a, const u32x4 &b, f32x4 c)
{
    if constexpr (DT == kFp16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(const u32x2 &a, const u32x2 &b, f32x4 c)
{
    if constexpr (DT == kFp16)
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                         __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

// K of a 16-token sub-tile: as loaded (lane l holds dims 8*(l%16)..+7 of row
// 4j + l/16, like V), or, after k_operand, in the A-operand layout of the four
// score MFMAs (lane i+16j holds dims 8*(4kk+j)..+7 of token i for MFMA kk).
struct KOp {
    u32x4 k[4];
};
// V rows of a sub-tile as loaded: lane l holds dims 8*(l%16).. of row 4j + l/16.
struct VRows {
    u32x4 v[4];
};

// Buffer resources over the rows of a 16-token sub-tile that hold tokens of the
// item (block tb/BS holds all 16 rows).  Rows past the context length lie
// outside the range: their loads return zeros and fetch nothing.
struct SubRsrc {
    __amdgpu_buffer_rsrc_t k, v;
};

// `t_load` is the end of the rows to fetch: the context end, or one less when the
// last row is the token being appended (it is then taken from the new rows).
template <int BS>
__device__ __forceinline__ SubRsrc sub_rsrc(int32_t phys, const uint16_t *kp, const uint16_t *vp,
                                            int tb, int t_load, int64_t head_off,
                                            int64_t blk_elems)
{
    const int64_t base = (int64_t)phys * blk_elems + head_off + (int64_t)(tb % BS) * kHeadDim;
    const int bytes = __builtin_amdgcn_readfirstlane(min(max(t_load - tb, 0), kSub) * kHeadDim * 2);
    SubRsrc r;
    r.k = make_rsrc(kp + base, bytes);
    r.v = make_rsrc(vp + base, bytes);
    return r;
}

// Table entry of the sub-tile at token tb; the index is clamped to the row so
// that a lookahead past the last sub-tile reads a valid (unused) entry.
template <int BS>
__device__ __forceinline__ int32_t sub_phys(meta_ptr trow, int width, int tb)
{
    return trow[min(tb / BS, width - 1)];
}

// K rows are loaded like V rows, 1 KiB of contiguous memory per load
// instruction.  Loading them straight into the A-operand layout (each 16-lane
// group reading 64 bytes of 16 different rows) delivered a third of the rate:
// about 9.5 TB/s from L2 against 30 TB/s for contiguous loads, measured with a
// plain read probe on MI355X.
template <int CPOL = kLoadStream>
__device__ __forceinline__ void load_k(KOp &t, __amdgpu_buffer_rsrc_t r, int lane)
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
        t.k[j] = ldbuf<CPOL>(r, lane * 16 + j * 1024);
}

// The A operand of the score MFMAs from K rows as loaded: the rows go through
// this wave's LDS K tile (row-major, 288-byte stride) and come back with one
// 16-byte read per MFMA (lane i+16j: row i, dims 8*(4kk+j)..).
__device__ __forceinline__ KOp k_operand(const KOp &raw, uint16_t *klds, int lane)
{
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *(u32x4 *)(klds + (4 * j + grp) * kKStride + col * 8) = raw.k[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    KOp a;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        a.k[kk] = *(const u32x4 *)(klds + col * kKStride + (4 * kk + grp) * 8);
    // the next sub-tile's K writes must not pass these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return a;
}

template <int CPOL = kLoadStream>
__device__ __forceinline__ void load_v(VRows &t, __amdgpu_buffer_rsrc_t r, int lane)
{
#pragma unroll
    for (int j = 0; j < 4; ++j)
        t.v[j] = ldbuf<CPOL>(r, lane * 16 + j * 1024);
}

struct GqaState {
    float m;        // reference max of this lane's query row (uniform over the 4 lane
                    // groups; lags the running max by at most kRescaleSlack)
    float l;        // this lane's share of the running sum
    f32x4 acc[8];   // O^T rows 16*jj + 4*(lane/16) + r, column = query row lane%16
};

// Scores of the sub-tile, online-softmax update of (m, l); returns the
// probabilities packed as the B operand of P.V and the rescale factor of acc.
// Scores of the sub-tile and the online-softmax update of (m, l).  PARTIAL:
// mask tokens outside [t_beg, t_end) (the sub-tile straddles an end), and the
// whole column of a lane whose col_on is false (a query row the sub-tile does
// not belong to).  Returns
// whether the wave rescales its accumulators (alpha holds each lane's factor,
// 1 where the column's reference max did not move); pb receives the
// probabilities packed as the B operand of P.V.
template <int DT, bool PARTIAL>
__device__ __forceinline__ bool qk_softmax(GqaState &st, const KOp &K, const u32x4 *qop, int tb,
                                           int t_beg, int t_end, int lane, float scale_log2,
                                           u32x2 &pb, float &alpha, bool col_on = true)
{
    const int grp = lane >> 4;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        s = mfma_qk<DT>(K.k[kk], qop[kk], s);
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        sc[r] = s[r] * scale_log2;
        const int t = tb + 4 * grp + r;
        if (PARTIAL && (t < t_beg || t >= t_end || !col_on))
            sc[r] = kNegInf;
    }
    float mt = vmax(vmax3(sc[0], sc[1], sc[2]), sc[3]);
    mt = pair_max32(pair_max16(mt));
    const bool grow = mt > st.m + kRescaleSlack;  // always true for the first scores
    const bool rescale = __ballot(grow) != 0;     // wave-uniform
    alpha = 1.f;
    if (rescale) {
        const float m_new = grow ? mt : st.m;
        alpha = fexp2(st.m - safe_ref(m_new));
        st.l *= alpha;
        st.m = m_new;
    }
    const float ref = safe_ref(st.m);
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        p[r] = fexp2(sc[r] - ref);
        psum += p[r];
    }
    st.l += psum;
    pb.x = (uint32_t)to_bits<DT>(p[0]) | ((uint32_t)to_bits<DT>(p[1]) << 16);
    pb.y = (uint32_t)to_bits<DT>(p[2]) | ((uint32_t)to_bits<DT>(p[3]) << 16);
    return rescale;
}

// Stage the V rows of the sub-tile, row-major, in this wave's LDS tile.
__device__ __forceinline__ void stage_v(const VRows &V, uint16_t *vlds, int lane)
{
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *(u32x4 *)(vlds + (4 * j + grp) * kVStride + col * 8) = V.v[j];
}

// acc = alpha * acc + V^T P^T.  The A operand of each 16x16x16 MFMA (lane l: dim
// 16jj + l%16 of tokens 4(l/16)..+3) comes from one transposing LDS read: lane j
// of each 16-lane group points at 4 consecutive elements of row 4(l/16) + j/4,
// column 16jj + 4(j%4), and the read hands lane i of the group element i%4 of the
// chunk addressed by lane 4e + i/4, for e = 0..3.  Rows past the context length
// were loaded as zeros (outside the buffer range), so their zero probabilities
// multiply zeros, never a stale NaN.
template <int DT>
__device__ __forceinline__ void pv_mma(GqaState &st, const uint16_t *vlds, const u32x2 &pb,
                                       bool rescale, float alpha, int lane)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int j = lane & 15, grp = lane >> 4;
    const uint16_t *base = vlds + (4 * grp + (j >> 2)) * kVStride + 4 * (j & 3);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (rescale) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st.acc[jj] *= alpha;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(base + 16 * jj));
        st.acc[jj] = mfma_pv<DT>(__builtin_bit_cast(u32x2, va), pb, st.acc[jj]);
    }
    // the next sub-tile's LDS writes must not pass these reads
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- sub-tiles staged in LDS by global-to-LDS loads ---------------------------
// The shared-prefix and slotted-tile kernels keep two sub-tiles per wave in
// flight without holding them in registers: gfx950's buffer loads can write
// straight to LDS (16 bytes per lane).  Such a load writes the 16 bytes of lane L
// at byte 16 L of its 1 KiB destination, and a lane outside the buffer's range
// writes zeros (both checked on the GPU with an in-bounds probe), so a masked row
// of a sub-tile is zero in LDS as it was in registers.
//
// A wave's staging area is two buffers, each a sub-tile's K rows then its V rows
// (16 rows x 256 bytes each, no padding).  Since the destination is lane-linear,
// the swizzle is applied on the global side: lane L of load i fetches chunk
// (L % 16) ^ swz(r) of row r = 4 i + L / 16, so chunk c of row r sits at position
// c ^ swz(r).  With swz(r) = (2 r + r / 8) % 16 the 16 lanes of a score-operand
// read (rows 0..15, one chunk) and the 32 lanes of a transposing V read (rows
// 0..7 or 8..15, two adjacent chunks) all fall on distinct banks.
//
// Ordering is explicit.  The compiler's own tracking of global-to-LDS loads is
// kept out (the destination address passes through an empty asm statement, so no
// LDS object is known to be written): it either waited for every such load in
// flight, or for none, depending on the loop's shape.  Instead each read of a
// buffer is preceded by a vector-memory wait whose count the caller derives from
// its own fixed issue order, and each refill of a buffer by a wait for the LDS
// reads of it.
constexpr int kDmaSubBytes = kSub * kHeadDim * 2;  // K (or V) of a sub-tile: 4 KiB
constexpr int kDmaBufBytes = 2 * kDmaSubBytes;     // K then V

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int dma_swz(int r) { return (2 * r + (r >> 3)) & 15; }

// Per-lane byte offsets of the staged layout (constant for the whole kernel).
struct DmaLanes {
    int src[4];  // row / chunk of the sub-tile that lane fetches in load i
    int ka[4];   // position of the A operand of score MFMA kk (row lane%16)
    int va[8];   // position of the transposing V^T read jj
};

__device__ __forceinline__ DmaLanes dma_lanes(int lane)
{
    DmaLanes d;
    const int col = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + grp;
        d.src[i] = r * 256 + ((col ^ dma_swz(r)) << 4);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        d.ka[kk] = col * 256 + (((4 * kk + grp) ^ dma_swz(col)) << 4);
    const int rv = 4 * grp + (col >> 2);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        d.va[jj] = rv * 256 + (((2 * jj + ((col & 3) >> 1)) ^ dma_swz(rv)) << 4) + (col & 1) * 8;
    return d;
}

// Issue the global-to-LDS loads of a sub-tile (K into buf, V into buf + 4 KiB):
// 8 vector-memory operations.  `buf` must be wave-uniform.
template <int CPOL = kLoadReuse>
__device__ __forceinline__ void dma_sub(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                        char *buf, const DmaLanes &d)
{
    // the LDS byte address, hidden from the compiler's alias analysis
    uint32_t base = (uint32_t)(uintptr_t)(lds_void *)buf;
    asm volatile("" : "+s"(base));
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(uintptr_t)(base + i * 1024), 16,
                                                 d.src[i], 0, 0, CPOL);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (lds_void *)(uintptr_t)(base + kDmaSubBytes + i * 1024), 16, d.src[i], 0, 0,
            CPOL);
}

// The score A operand and the P.V A operand (V^T) of a staged sub-tile.
__device__ __forceinline__ KOp dma_read_k(const char *buf, const DmaLanes &d)
{
    KOp a;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        a.k[kk] = *(const u32x4 *)(buf + d.ka[kk]);
    return a;
}

__device__ __forceinline__ void dma_read_v(i16x4 (&va)[8], const char *buf, const DmaLanes &d)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        va[jj] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4 *)(buf + kDmaSubBytes + d.va[jj]));
}

// acc = alpha * acc + V^T P^T for the halves that are live this sub-tile, from a
// V^T operand already in registers.
template <int DT, int NH>
__device__ __forceinline__ void pv_mma_regs(GqaState (&st)[NH], const i16x4 (&va)[8],
                                            const u32x2 (&pb)[NH], const bool (&rescale)[NH],
                                            const float (&alpha)[NH], const bool (&live)[NH])
{
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        if (!live[h])
            continue;  // wave-uniform: a half with no active column this sub-tile
        if (rescale[h]) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                st[h].acc[jj] *= alpha[h];
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st[h].acc[jj] = mfma_pv<DT>(__builtin_bit_cast(u32x2, va[jj]), pb[h], st[h].acc[jj]);
    }
}

// s_waitcnt encodings (gfx9 family): wait until at most N vector-memory
// operations are outstanding; until no LDS (or scalar) operation is.
#define PKV_WAIT_VMCNT(N) __builtin_amdgcn_s_waitcnt(0x0F70 | ((N) & 15) | (((N) >> 4) << 14))
#define PKV_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// A work-group barrier for data exchanged through LDS by ordinary LDS writes:
// the wave's LDS (and scalar) operations complete first, and vector-memory
// operations, global-to-LDS loads included, stay in flight (a fenced barrier
// waits for every one of them).  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work modes of the decode kernel.
constexpr int kModeSingle = 0;  // one pass over positions 0 .. n-1, writes `out`
constexpr int kModeSplit = 1;   // partitions of the context, writes part_o / part_lse
constexpr int kModeSuffix = 2;  // shared-prefix mode: positions prefix_len .. n-1, then
                                // merged with the prefix partials, writes `out`
constexpr int kModeMerge = 3;   // split mode whose last work-group per item merges the
                                // partials into `out` (a context of one partition is
                                // written to `out` directly)
constexpr int kModeSuffixSplit = 4;  // shared-prefix mode with the positions after the
                                     // prefix cut into partitions; the last work-group
                                     // per item merges prefix and suffix partials

// MODE kModeSplit / kModeMerge / kModeSuffixSplit run a partition loop; the other
// modes one pass, with the loop folded away at compile time.
// The register budget is capped so that 4 waves (single pass) or PKV_SPLIT_OCC
// waves (split modes, which keep two sub-tiles in registers and more state live
// across their partition loop) fit on each SIMD without spilling.
#ifndef PKV_SPLIT_OCC
#define PKV_SPLIT_OCC 2
#endif
template <int DT, int BS, int WAVES, int MODE>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(MODE == kModeSplit || MODE == kModeMerge ||
                                           MODE == kModeSuffixSplit
                                       ? PKV_SPLIT_OCC
                                       : 4)))
void decode_mfma_kernel(DecodeArgs a)
{
    constexpr bool SUFFIX = MODE == kModeSuffix || MODE == kModeSuffixSplit;
    constexpr bool MERGE = MODE == kModeMerge || MODE == kModeSuffixSplit;
    constexpr bool SPLIT = MODE == kModeSplit || MERGE;
    // V staging during the token loop; the cross-wave merge afterwards
    __shared__ __attribute__((aligned(16))) union {
        uint16_t v[WAVES][kStageElems];
        float o[WAVES][16][kOStride];
    } sm;
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    // fused append: the new K and V rows, parked by the wave that owns position
    // n-1 until its last sub-tile (registers would be held across the whole loop)
    __shared__ u32x4 s_new[2][kHeadDim / 8];
    __shared__ int32_t s_last;  // merged split mode: this work-group arrived last

    // sequence-major work items (see the MHA kernel): the KV heads of a sequence
    // are neighbours in dispatch order
    const int item = blockIdx.x;
    const int parts = SPLIT ? a.parts_per_item : 1;
    const int px0 = item % parts;
    const int rest = item / parts;
    const int g = rest % a.num_kv_heads;  // kv head
    const int s = ordered_seq(a, rest / a.num_kv_heads);
    const int G = a.num_q_heads / a.num_kv_heads;
    const int tid = threadIdx.x;
    // wave index, made explicitly uniform so that tile indices and table lookups
    // stay in SGPRs (scalar loads of the table entries)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const meta_ptr trow = as_meta(a.tables) + (int64_t)s * a.width;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)g * BS * kHeadDim;
    const int P = SPLIT ? a.partition_size : 0;
    // shared-prefix mode: this pass covers the positions after the group's prefix
    const int start = SUFFIX
                          ? as_meta(a.prefix_lens)[group_of(as_meta(a.group_cu), a.num_groups, s)]
                          : 0;
    const int start_sub = start & ~(kSub - 1);  // sub-tiles stay aligned to 16 positions
    // partitions start at position `base` (the suffix's first sub-tile, or 0)
    const int base = SUFFIX ? start_sub : 0;

    // The first sub-tile's table entry (and the next one's) do not depend on the
    // context length: request them together with it, so the two scalar-load
    // latencies overlap instead of chaining.
    const int tb_first = base + (P > 0 ? px0 * P : 0) + w * kSub;
    const int32_t e_first = sub_phys<BS>(trow, a.width, tb_first);
    const int32_t e_next = sub_phys<BS>(trow, a.width, tb_first + WAVES * kSub);
    const int n = as_meta(a.lens)[s];
    const bool fused = a.k_new != nullptr;
    if (fused && n <= 0 && px0 == 0 && g == 0 && tid == 0 && a.slot_out)
        a.slot_out[s] = -1;  // padding sequence: nothing appended

    // B operand of the score MFMAs: Q^T, query row `col` of the group (zero padding)
    u32x4 qop[4];
    {
        const uint16_t *qrow = (const uint16_t *)a.q +
                               ((int64_t)s * a.num_q_heads + (int64_t)g * G + col) * kHeadDim +
                               grp * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[kk] = col < G ? *(const u32x4 *)(qrow + kk * 32) : (u32x4){0u, 0u, 0u, 0u};
    }
    uint16_t *vlds = sm.v[w];
    uint16_t *klds = vlds + kSub * kVStride;
    const int64_t row0 = (int64_t)s * a.num_q_heads + (int64_t)g * G;

    // Shared-prefix mode: the first prefix partition's partials of the elements
    // this thread merges at the end (element e = (query row e/32, dims 4(e%32)..))
    // are requested now, so their latency overlaps the token loop.
    // Two rounds cover a group (G <= 16: 512 elements, 256 threads).  The merge's
    // loop counts rounds at run time, so the two are held as named values and
    // picked by select (an array indexed by the round would live in scratch).
    constexpr int kPre = 2;
    static_assert(kPre * WAVES * 64 >= 16 * 32, "two rounds cover a group of 16 heads");
    f32x4 pre_o0 = {0.f, 0.f, 0.f, 0.f}, pre_o1 = {0.f, 0.f, 0.f, 0.f};
    float pre_l0 = 0.f, pre_l1 = 0.f;
    if (SUFFIX) {
        const int e0 = tid, e1 = tid + WAVES * 64;
        if (e0 < G * 32) {
            const int64_t row = row0 + (e0 >> 5);
            pre_l0 = a.part_lse[row * a.max_partitions];
            pre_o0 = *(const f32x4 *)(a.part_o + row * a.max_partitions * kHeadDim + (e0 & 31) * 4);
        }
        if (e1 < G * 32) {
            const int64_t row = row0 + (e1 >> 5);
            pre_l1 = a.part_lse[row * a.max_partitions];
            pre_o1 = *(const f32x4 *)(a.part_o + row * a.max_partitions * kHeadDim + (e1 & 31) * 4);
        }
    }

    // Partitions px0, px0 + parts_per_item, ... of the item belong to this
    // work-group (the grid is sized from the batch, not from the table width).
    // Single pass: one iteration over the whole context (zeros when n = 0).
    // Merged split mode: a context of at most one partition is handled like a
    // single pass by the item's first work-group, which writes `out` itself.
    // Suffix split mode: the positions base .. n-1 are cut into partitions, whose
    // partials are kept after the group's prefix partials (index np_pre + p).
    const int np = SPLIT ? (max(n - base, 0) + P - 1) / P : 1;
    const bool direct = MERGE && np <= 1;
    const int np_loop = direct ? (px0 == 0 ? 1 : 0) : np;
    const int np_pre = SUFFIX && a.prefix_part > 0
                           ? min((start + a.prefix_part - 1) / a.prefix_part, a.max_partitions)
                           : 0;
    for (int px = px0; px < np_loop; px += parts) {
        if (px != px0)
            __syncthreads();  // the previous partition's merge is done with LDS
        const int t0 = P > 0 ? base + px * P : start_sub;
        const int t1 = P > 0 ? min(n, t0 + P) : n;
        const int t_beg = SUFFIX ? start : t0;  // positions below are masked
        // With a fused append, position n-1 (in the item's last sub-tile) is not
        // read from the pool: it holds stale data until this kernel writes it.
        const bool owns_new = fused && t1 == n;
        const int t_load = owns_new ? n - 1 : t1;

        GqaState st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st.acc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};

        const int nsub = t1 > t0 ? (t1 - t0 + kSub - 1) / kSub : 0;
        // the wave holding position n-1 (the item's last sub-tile) fetches the new
        // rows and their block id up front, so that the latency overlaps its loop:
        // knew[kk] is the A-operand chunk of the new key (dims 8*(4kk + lane/16)..),
        // vnew the 16-byte chunk lane%16 of the new value row
        const bool new_here = owns_new && nsub > 0 && w == (nsub - 1) % WAVES;
        u32x4 knew[4] = {}, vnew = {0u, 0u, 0u, 0u};
        const int64_t phys_n = new_here ? (int64_t)trow[(n - 1) / BS] : 0;  // block of n-1
        if (new_here) {
            const int64_t off = ((int64_t)s * a.num_kv_heads + g) * kHeadDim;
            const uint16_t *kq = (const uint16_t *)a.k_new + off;
            const uint16_t *vq = (const uint16_t *)a.v_new + off;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                knew[kk] = *(const u32x4 *)(kq + 32 * kk + 8 * grp);
            vnew = *(const u32x4 *)(vq + 8 * col);
        }
        const int T = nsub > w ? (nsub - w + WAVES - 1) / WAVES : 0;
        if (T > 0) {
            int tb = t0 + w * kSub;
            const int step = WAVES * kSub;
            const bool first = px == px0;
            // write the new rows to their slot once the first loads are out:
            // stores share the in-order vmcnt counter with loads, so issuing them
            // here lets their latency overlap the loop instead of the end of the
            // work-group
            auto store_new = [&]() {
                const int tn = n - 1;
                const int64_t dst =
                    phys_n * blk_elems + head_off + (int64_t)(tn % BS) * kHeadDim;
                if (col == (tn & 15)) {
                    // the four lanes of the new row's A-operand slot hold the key
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        *(u32x4 *)((uint16_t *)a.k_pool + dst + 32 * kk + 8 * grp) = knew[kk];
                }
                if (col == 0) {
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        s_new[0][4 * kk + grp] = knew[kk];
                }
                if (lane < 16) {
                    *(u32x4 *)((uint16_t *)a.v_pool + dst + lane * 8) = vnew;
                    s_new[1][lane] = vnew;
                }
                if (g == 0 && lane == 0 && a.slot_out)
                    a.slot_out[s] = phys_n * BS + tn % BS;
            };
            u32x2 pb;
            float alpha;
            bool rs;
            // The last sub-tile: position n-1, if it lies here, takes the new rows in
            // place of the (unfetched) pool row; a partial sub-tile is masked.
            auto last_step = [&](KOp &K, VRows &V) {
                const bool here = new_here && tb + kSub >= n;
                const int row = n - 1 - tb;  // 0..15 when `here`
                KOp KA = k_operand(K, klds, lane);
                if (here && (lane & 15) == row) {
                    // the four lanes of row `row` take the new key into the A operand
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
                        KA.k[kk] = s_new[0][4 * kk + grp];
                }
                if (tb + kSub <= t1)
                    rs = qk_softmax<DT, SUFFIX>(st, KA, qop, tb, t_beg, t1, lane, a.scale_log2,
                                                pb, alpha);
                else
                    rs = qk_softmax<DT, true>(st, KA, qop, tb, t_beg, t1, lane, a.scale_log2,
                                              pb, alpha);
                stage_v(V, vlds, lane);
                if (here && lane < 16)
                    *(u32x4 *)(vlds + row * kVStride + lane * 8) = s_new[1][lane];
                pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
            };
            // A full sub-tile, consumed from (K, V); the loads of the sub-tile `ahead`
            // steps later (table entry pn) go into the same registers once they are
            // free: the K loads once the scores' operand is staged, the V loads once
            // the V rows are, so they overlap softmax and P.V.
            auto full_step = [&](KOp &K, VRows &V, int32_t pn, int ahead) {
                const SubRsrc rn =
                    sub_rsrc<BS>(pn, kp, vp, tb + ahead * step, t_load, head_off, blk_elems);
                const KOp KA = k_operand(K, klds, lane);
                __builtin_amdgcn_sched_barrier(0);
                load_k(K, rn.k, lane);  // the raw registers are free once staged
                __builtin_amdgcn_sched_barrier(0);
                rs = qk_softmax<DT, SUFFIX>(st, KA, qop, tb, t_beg, t1, lane, a.scale_log2, pb,
                                            alpha);
                __builtin_amdgcn_sched_barrier(0);
                stage_v(V, vlds, lane);
                __builtin_amdgcn_sched_barrier(0);
                load_v(V, rn.v, lane);
                __builtin_amdgcn_sched_barrier(0);
                pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
                __builtin_amdgcn_sched_barrier(0);
                tb += step;
            };
            if constexpr (SPLIT) {
                // Split modes (3 waves per SIMD, registers to spare): two register
                // buffers, so the loads of the next two sub-tiles are in flight
                // behind the current one.  Step j consumes buffer j % 2 and refills
                // it with sub-tile j + 2; sub-tiles past the wave's last one have an
                // empty buffer range (zeros, no fetch).  Table entries are looked up
                // a step before the loads that use them.
                KOp K0, K1;
                VRows V0, V1;
                {
                    const int32_t ef = first ? e_first : sub_phys<BS>(trow, a.width, tb);
                    const int32_t en = first ? e_next : sub_phys<BS>(trow, a.width, tb + step);
                    const SubRsrc r0 = sub_rsrc<BS>(ef, kp, vp, tb, t_load, head_off, blk_elems);
                    const SubRsrc r1 =
                        sub_rsrc<BS>(en, kp, vp, tb + step, t_load, head_off, blk_elems);
                    load_k(K0, r0.k, lane);
                    load_v(V0, r0.v, lane);
                    load_k(K1, r1.k, lane);
                    load_v(V1, r1.v, lane);
                }
                if (new_here)
                    store_new();
                int32_t pa = sub_phys<BS>(trow, a.width, tb + 2 * step);
                int j = 0;
                for (; j + 2 < T; j += 2) {  // steps j and j + 1 are full
                    const int32_t pb2 = sub_phys<BS>(trow, a.width, tb + 3 * step);
                    full_step(K0, V0, pa, 2);
                    pa = sub_phys<BS>(trow, a.width, tb + 3 * step);
                    full_step(K1, V1, pb2, 2);
                }
                if (j + 1 < T) {
                    full_step(K0, V0, pa, 2);
                    last_step(K1, V1);
                } else {
                    last_step(K0, V0);
                }
            } else {
                // Single pass: one register buffer per operand (4 waves per SIMD).
                KOp K;
                VRows V;
                {
                    const int32_t ef = first ? e_first : sub_phys<BS>(trow, a.width, tb);
                    const SubRsrc r = sub_rsrc<BS>(ef, kp, vp, tb, t_load, head_off, blk_elems);
                    load_k(K, r.k, lane);
                    load_v(V, r.v, lane);
                }
                if (new_here)
                    store_new();
                // table entries are looked up one sub-tile ahead of the loads that use them
                int32_t pn = first ? e_next : sub_phys<BS>(trow, a.width, tb + step);
                for (int j = 0; j + 1 < T; ++j) {  // every sub-tile here is full
                    const int32_t pn2 = sub_phys<BS>(trow, a.width, tb + 2 * step);
                    full_step(K, V, pn, 1);
                    pn = pn2;
                }
                last_step(K, V);
            }
        }

        // sum of the four lane groups' shares of l (m is already uniform across them)
        st.l = pair_sum32(pair_sum16(st.l));

        __syncthreads();  // all waves are done with their V staging area
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            *(f32x4 *)&sm.o[w][col][16 * jj + 4 * grp] = st.acc[jj];
        if (grp == 0) {
            s_m[w][col] = st.m;
            s_l[w][col] = st.l;
        }
        __syncthreads();

        // element e: query row qi = e/32 of the group, dims d0 .. d0+3
        for (int e = tid, k = 0; e < G * 32; e += WAVES * 64, ++k) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            float M = s_m[0][qi];
#pragma unroll
            for (int i = 1; i < WAVES; ++i)
                M = fmaxf(M, s_m[i][qi]);
            const float ref = safe_ref(M);
            float L = 0.f;
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < WAVES; ++i) {
                const float wgt = fexp2(s_m[i][qi] - ref);
                L += s_l[i][qi] * wgt;
                O += *(const f32x4 *)&sm.o[i][qi][d0] * wgt;
            }
            const int64_t row = row0 + qi;
            if (MODE == kModeSuffix || P == 0 || direct) {
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
                if (SUFFIX) {
                    // merge with the prefix partitions (normalised o, natural-log lse)
                    const float *lse = a.part_lse + row * a.max_partitions;
                    const float *po = a.part_o + row * a.max_partitions * kHeadDim + d0;
                    float X = L > 0.f ? ref : kNegInf;
                    for (int p = 0; p < np_pre; ++p)
                        X = fmaxf(X, (p == 0 && k < kPre ? (k == 0 ? pre_l0 : pre_l1) : lse[p]) * kLog2e);
                    float den = 0.f;
                    f32x4 num = {0.f, 0.f, 0.f, 0.f};
                    if (X != kNegInf) {
                        if (L > 0.f) {
                            const float ws = fexp2(ref - X);
                            num = O * ws;
                            den = L * ws;
                        }
                        for (int p = 0; p < np_pre; ++p) {
                            const bool pf = p == 0 && k < kPre;
                            const float lp = (pf ? (k == 0 ? pre_l0 : pre_l1) : lse[p]) * kLog2e;
                            if (lp != kNegInf) {
                                const float wp = fexp2(lp - X);
                                num += (pf ? (k == 0 ? pre_o0 : pre_o1) : *(const f32x4 *)(po + p * kHeadDim)) * wp;
                                den += wp;
                            }
                        }
                    }
                    if (den > 0.f)
                        o = num / den;
                } else if (L > 0.f) {
                    o = O / L;
                }
                u32x2 packed;
                packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
                packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
                *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
            } else {
                float *po = a.part_o + (row * a.max_partitions + px) * kHeadDim + d0;
                const f32x4 ov = O / L;
                const float lse = (ref + flog2(L)) * kLn2;
                if constexpr (MERGE) {
                    // read by another work-group of the item (see arrive_last); suffix
                    // partitions follow the prefix partitions
                    const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
                    const int pi = np_pre + px;
                    st_ws4(ws.o, (int)((row * a.max_partitions + pi) * kHeadDim + d0) * 4, ov);
                    if (d0 == 0)
                        st_ws1(ws.lse, (int)(row * a.max_partitions + pi) * 4, lse);
                } else {
                    *(f32x4 *)po = ov;
                    if (d0 == 0)
                        a.part_lse[row * a.max_partitions + px] = lse;
                }
            }
        }
    }

    if constexpr (MERGE) {
        // the work-groups that wrote partials arrive; the last one merges them
        if (direct || px0 >= np)
            return;
        if (!arrive_last(a.counters + rest, min(np, parts), &s_last))
            return;
        const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
        for (int e = tid; e < G * 32; e += WAVES * 64) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            const int64_t row = row0 + qi;
            const f32x4 o = merge_partials4(ws, (int)(row * a.max_partitions) * 4,
                                            (int)(row * a.max_partitions * kHeadDim + d0) * 4,
                                            np_pre + np);
            u32x2 packed;
            packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
            packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
            *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
        }
    }
}

// Cache policy of the prefix pass's K/V loads: each shared block is re-read by
// every query tile of its group, so the loads keep the default policy (L2 hits).
#ifndef PKV_PREFIX_CPOL
#define PKV_PREFIX_CPOL kLoadReuse
#endif

// Shared-prefix pass.  The sequences of a group share the K/V of their first
// prefix_len positions (the same physical blocks: page "端侧 SLM 显存保活术：在 4GB
// 内存板卡上实现轻量 PagedAttention 与 KV 缓存分块", pwwt.cn, section "共享前缀块
// （Prefix Caching）"; blog.llmgo.top page, §四, concurrent reads of blocks whose
// reference count exceeds 1).  One work-group takes a 16-row query tile made of
// the G query heads of floor(16/G) consecutive sequences, one KV head and one
// prefix partition, so each K/V sub-tile it fetches feeds the score and P.V
// matrix-core tiles of all those sequences at once (the decode kernel pads a
// single sequence's G rows to 16 instead).  It writes each row's fp32 partial
// (normalised o and natural-log lse) of prefix partition pp to
// part_o / part_lse[row][pp]; partitions past the prefix are not written.  A
// tile whose sequences span several groups handles each group in turn.
template <int DT, int BS, int WAVES>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(4)))
void prefix_mfma_kernel(DecodeArgs a)
{
    __shared__ __attribute__((aligned(16))) union {
        uint16_t v[WAVES][kStageElems];
        float o[WAVES][16][kOStride];
    } sm;
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    __shared__ int64_t s_row[16];  // output row of each query column, -1 if inactive

    // items: (tile, KV head, partition), partition fastest, then KV head; the
    // partials' row stride is max_partitions
    const int item = blockIdx.x;
    const int npp = a.parts_per_item;
    const int pp = item % npp;
    const int g = (item / npp) % a.num_kv_heads;
    const int tile = item / (npp * a.num_kv_heads);
    const int G = a.num_q_heads / a.num_kv_heads;
    const int spt = a.seqs_per_tile;
    const int s0 = tile * spt;
    const int s_end = min(a.num_seqs, s0 + spt);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int PP = a.prefix_part;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)g * BS * kHeadDim;
    uint16_t *vlds = sm.v[w];
    uint16_t *klds = vlds + kSub * kVStride;
    // query column -> (sequence, query head) of the tile
    const int cs = s0 + col / G;
    const int ch = g * G + col % G;

    int k = group_of(as_meta(a.group_cu), a.num_groups, s0);
    for (bool more = true; more; ++k) {
        const int ga = as_meta(a.group_cu)[k], gb = as_meta(a.group_cu)[k + 1];
        more = gb < s_end;
        const int plen = as_meta(a.prefix_lens)[k];
        const int t0 = pp * PP;
        if (ga == gb || t0 >= plen)
            continue;  // uniform: an empty group, or no prefix in this partition
        const int t1 = min(plen, t0 + PP);
        const meta_ptr trow = as_meta(a.tables) + (int64_t)ga * a.width;
        const bool active = col < spt * G && cs < s_end && cs >= ga && cs < gb;

        u32x4 qop[4];
        {
            const uint16_t *qrow = (const uint16_t *)a.q +
                                   ((int64_t)cs * a.num_q_heads + ch) * kHeadDim + grp * 8;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qop[kk] = active ? *(const u32x4 *)(qrow + kk * 32) : (u32x4){0u, 0u, 0u, 0u};
        }
        GqaState st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st.acc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};

        const int nsub = (t1 - t0 + kSub - 1) / kSub;
        const int T = nsub > w ? (nsub - w + WAVES - 1) / WAVES : 0;
        if (T > 0) {
            int tb = t0 + w * kSub;
            const int step = WAVES * kSub;
            KOp K;
            VRows V;
            {
                const SubRsrc r = sub_rsrc<BS>(sub_phys<BS>(trow, a.width, tb), kp, vp, tb, t1,
                                               head_off, blk_elems);
                load_k<PKV_PREFIX_CPOL>(K, r.k, lane);
                load_v<PKV_PREFIX_CPOL>(V, r.v, lane);
            }
            int32_t pn = sub_phys<BS>(trow, a.width, tb + step);
            u32x2 pb;
            float alpha;
            bool rs;
            for (int j = 0; j + 1 < T; ++j) {
                const int32_t pn2 = sub_phys<BS>(trow, a.width, tb + 2 * step);
                const SubRsrc rn = sub_rsrc<BS>(pn, kp, vp, tb + step, t1, head_off, blk_elems);
                const KOp KA = k_operand(K, klds, lane);
                __builtin_amdgcn_sched_barrier(0);
                load_k<PKV_PREFIX_CPOL>(K, rn.k, lane);
                __builtin_amdgcn_sched_barrier(0);
                rs = qk_softmax<DT, false>(st, KA, qop, tb, t0, t1, lane, a.scale_log2, pb, alpha);
                __builtin_amdgcn_sched_barrier(0);
                stage_v(V, vlds, lane);
                __builtin_amdgcn_sched_barrier(0);
                load_v<PKV_PREFIX_CPOL>(V, rn.v, lane);
                __builtin_amdgcn_sched_barrier(0);
                pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
                __builtin_amdgcn_sched_barrier(0);
                pn = pn2;
                tb += step;
            }
            const KOp KA = k_operand(K, klds, lane);
            if (tb + kSub <= t1)
                rs = qk_softmax<DT, false>(st, KA, qop, tb, t0, t1, lane, a.scale_log2, pb, alpha);
            else
                rs = qk_softmax<DT, true>(st, KA, qop, tb, t0, t1, lane, a.scale_log2, pb, alpha);
            stage_v(V, vlds, lane);
            pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
        }
        st.l = pair_sum32(pair_sum16(st.l));

        __syncthreads();  // all waves are done with their V staging area
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            *(f32x4 *)&sm.o[w][col][16 * jj + 4 * grp] = st.acc[jj];
        if (grp == 0) {
            s_m[w][col] = st.m;
            s_l[w][col] = st.l;
        }
        if (tid < 16)
            s_row[tid] = active ? (int64_t)cs * a.num_q_heads + ch : -1;
        __syncthreads();
        // element e: query column qi = e/32, dims d0 .. d0+3
        for (int e = tid; e < 16 * 32; e += WAVES * 64) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            const int64_t row = s_row[qi];
            if (row < 0)
                continue;
            float M = s_m[0][qi];
#pragma unroll
            for (int i = 1; i < WAVES; ++i)
                M = fmaxf(M, s_m[i][qi]);
            const float ref = safe_ref(M);
            float L = 0.f;
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < WAVES; ++i) {
                const float wgt = fexp2(s_m[i][qi] - ref);
                L += s_l[i][qi] * wgt;
                O += *(const f32x4 *)&sm.o[i][qi][d0] * wgt;
            }
            *(f32x4 *)(a.part_o + (row * a.max_partitions + pp) * kHeadDim + d0) = O / L;
            if (d0 == 0)
                a.part_lse[row * a.max_partitions + pp] = (ref + flog2(L)) * kLn2;
        }
        __syncthreads();  // LDS is reused by the next group of the tile
    }
}

// Slotted segments.  A short radix-tree node is packed as a slot of a shared
// block and addressed by a (block id, slot offset, length) triple (mhpq.cn page
// on Radix-Tree fragmentation, sections "Slotted Block 分槽与微块共享架构" and
// "核心设计原则"); a sequence is the concatenation of its segments.  One
// work-group per (sequence, KV head): per round of up to 64 segments, the first
// wave turns them into sub-tile descriptors (block, first row, row count <= 16;
// a segment of L rows gives ceil(L/16) of them) with a wave prefix sum and parks
// them in LDS; then every wave streams its share of the sub-tiles through the
// same score / softmax / P.V path as the decode kernel.  Each sub-tile's buffer
// range covers only its segment's rows, so rows of other slots in the block are
// never fetched (their loads return zeros) and are masked out of the softmax.
constexpr int kSegRound = 64;
constexpr int kMaxRoundSubs = kSegRound * 16;  // a 256-row segment gives 16 sub-tiles

// Fused append for slotted segments, one whole wave per sequence: sequence s's new
// K and V rows of KV head g go to its position n-1, which is the last row of its
// last non-empty segment (lengths clamped to the block, as the decode reads
// them); with head 0 the wave also writes the slot id, or -1 when n = 0.  Split
// in two so that a wave can have the loads of several sequences in flight at
// once: slot_append_load issues every load (the segment count, lane k's segment
// k < 64, and lanes 0-31's 16 bytes of the new K (lanes 0-15) or V row), none
// depending on another; slot_append_store finds the row (a longer list's later
// segments are read there) and writes it.  The caller's next fenced barrier
// (workgroup-scope release and acquire) orders the stores before every later
// load of the work-group's waves.
struct SlotAppend {
    int nseg;           // segment count as passed
    int32_t blk, off, len;  // this lane's segment of the first 64
    u32x4 val;          // lanes 0-31: their 16 bytes of the new rows
};

__device__ __forceinline__ SlotAppend slot_append_load(const DecodeArgs &a, int s, int g,
                                                       int lane)
{
    SlotAppend r;
    const int32_t *seg =
        a.segments + ((int64_t)s * a.max_segments + min(lane, a.max_segments - 1)) * 3;
    r.nseg = a.num_segments[s];
    r.blk = seg[0];
    r.off = seg[1];
    r.len = seg[2];
    const int kv = (lane >> 4) & 1, c = lane & 15;
    r.val = *(const u32x4 *)((const uint16_t *)(kv ? a.v_new : a.k_new) +
                             ((int64_t)s * a.num_kv_heads + g) * kHeadDim + 8 * c);
    return r;
}

template <int BS>
__device__ __forceinline__ void slot_append_store(const DecodeArgs &a, const SlotAppend &r, int s,
                                                  int g, int lane)
{
    const int nseg = min(max(r.nseg, 0), a.max_segments);
    int last = -1, lblk = 0, lrow = 0;  // this lane's last non-empty segment
    auto take = [&](int i, int32_t blk, int off, int len) {
        off = min(max(off, 0), BS);
        len = min(max(len, 0), BS - off);
        if (len > 0) {
            last = i;
            lblk = blk;
            lrow = off + len - 1;
        }
    };
    if (lane < nseg)
        take(lane, r.blk, r.off, r.len);
    const int32_t *segs = a.segments + (int64_t)s * a.max_segments * 3;
    for (int i = 64 + lane; i < nseg; i += 64)
        take(i, segs[3 * i], segs[3 * i + 1], segs[3 * i + 2]);
    int best = last;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        best = max(best, __shfl_xor(best, d, 64));
    if (best < 0) {
        if (g == 0 && lane == 0 && a.slot_out)
            a.slot_out[s] = -1;
        return;
    }
    const int blk = __shfl(lblk, best & 63, 64), row = __shfl(lrow, best & 63, 64);
    const int64_t dst = ((int64_t)blk * a.num_kv_heads + g) * BS * kHeadDim +
                        (int64_t)row * kHeadDim;
    if (lane < 32)
        *(u32x4 *)((uint16_t *)(lane >> 4 ? a.v_pool : a.k_pool) + dst + 8 * (lane & 15)) = r.val;
    if (g == 0 && lane == 0 && a.slot_out)
        a.slot_out[s] = (int64_t)blk * BS + row;
}

// Buffer resources of slotted sub-tile jx: its block, first row and row count
// come from the LDS descriptors (made uniform for the scalar descriptor).
__device__ __forceinline__ SubRsrc slot_rsrc(const int32_t *s_phys, const int32_t *s_rows, int jx,
                                             const uint16_t *kp, const uint16_t *vp,
                                             int64_t head_off, int64_t blk_elems)
{
    const int32_t phys = __builtin_amdgcn_readfirstlane(s_phys[jx]);
    const int32_t rc = __builtin_amdgcn_readfirstlane(s_rows[jx]);
    const int64_t b = (int64_t)phys * blk_elems + head_off + (int64_t)(rc >> 8) * kHeadDim;
    SubRsrc r;
    r.k = make_rsrc(kp + b, (rc & 0xff) * kHeadDim * 2);
    r.v = make_rsrc(vp + b, (rc & 0xff) * kHeadDim * 2);
    return r;
}

// SPLIT: split-context mode with the partitions merged in the launch.  The
// sequence's logical positions (the concatenation of its segments) are cut into
// partitions of partition_size tokens; work-group px of an item takes
// partitions px, px + parts_per_item, ...  Each round's segments are clipped to
// the partition's positions before they become sub-tiles, so a segment that
// straddles a partition boundary is split between two partitions.  Partials and
// the arrival of the work-groups follow the merged split decode (arrive_last); a
// sequence of at most one partition is written to `out` directly.
template <int DT, int BS, int WAVES, bool SPLIT = false>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(3)))
void slotted_mfma_kernel(DecodeArgs a)
{
    __shared__ __attribute__((aligned(16))) union {
        uint16_t v[WAVES][kStageElems];
        float o[WAVES][16][kOStride];
    } sm;
    __shared__ float s_m[WAVES][16], s_l[WAVES][16];
    __shared__ int32_t s_phys[kMaxRoundSubs];
    __shared__ int32_t s_rows[kMaxRoundSubs];  // first row << 8 | row count
    __shared__ int32_t s_total;
    __shared__ int32_t s_run;   // positions covered by the rounds so far (see below)
    __shared__ int32_t s_last;  // split mode: this work-group arrived last

    const int item = blockIdx.x;
    const int parts = SPLIT ? a.parts_per_item : 1;
    const int px0 = item % parts;
    const int rest = item / parts;
    const int g = rest % a.num_kv_heads;
    const int s = rest / a.num_kv_heads;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)g * BS * kHeadDim;
    const int32_t *__restrict__ segs = a.segments + (int64_t)s * a.max_segments * 3;
    const int nseg = min(max(a.num_segments[s], 0), a.max_segments);  // never past the row
    uint16_t *vlds = sm.v[w];
    uint16_t *klds = vlds + kSub * kVStride;
    const int64_t row0 = (int64_t)s * a.num_q_heads + (int64_t)g * G;

    // a segment never reaches outside its block, whatever the caller passed
    auto clamped = [&](int i, int32_t &blk, int &off, int &len) {
        blk = segs[3 * i];
        off = min(max(segs[3 * i + 1], 0), BS);
        len = min(max(segs[3 * i + 2], 0), BS - off);
    };

    // split mode: the sequence length n (the clamped lengths' sum, every wave)
    int n = 0;
    if constexpr (SPLIT) {
        for (int base = 0; base < nseg; base += kSegRound) {
            int32_t blk;
            int off, len = 0;
            if (base + lane < nseg)
                clamped(base + lane, blk, off, len);
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1)
                len += __shfl_xor(len, d, 64);
            n += len;
        }
        n = __builtin_amdgcn_readfirstlane(n);
    }
    const int P = SPLIT ? a.partition_size : 0;
    const int np = SPLIT ? (n + P - 1) / P : 1;
    const bool direct = !SPLIT || np <= 1;
    const int np_loop = direct ? (px0 == 0 ? 1 : 0) : np;

    // fused append: wave 0 of the work-group that takes the partition holding
    // position n-1 (the only one that reads it) issues its loads with the query's
    // and writes the new rows before the partition loop; the round's first
    // barrier orders the stores before any wave's sub-tile loads
    SlotAppend ap;
    const bool appends = a.k_new && w == 0 && px0 == (direct ? 0 : (np - 1) % parts);
    if (appends)
        ap = slot_append_load(a, s, g, lane);
    u32x4 qop[4];
    {
        const uint16_t *qrow = (const uint16_t *)a.q +
                               ((int64_t)s * a.num_q_heads + (int64_t)g * G + col) * kHeadDim +
                               grp * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            qop[kk] = col < G ? *(const u32x4 *)(qrow + kk * 32) : (u32x4){0u, 0u, 0u, 0u};
    }

    if (appends)
        slot_append_store<BS>(a, ap, s, g, lane);

    for (int px = px0; px < np_loop; px += parts) {
        // positions [t0, t1) of this partition (the whole sequence in one pass)
        const int t0 = direct ? 0 : px * P;
        const int t1 = direct ? INT32_MAX : min(n, t0 + P);
        GqaState st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st.acc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (px != px0)
            __syncthreads();  // the previous partition's merge is done with LDS

        // `run` (positions covered by the earlier rounds) is the same register
        // value in every wave: wave 0 publishes the next one in s_run before the
        // round's first barrier, and every wave reads it back after that barrier
        // (s_run is rewritten only after the round's second barrier)
        int run = 0;
        for (int base = 0; base < nseg && run < t1; base += kSegRound) {
            if (w == 0) {
                const int i = base + lane;
                int32_t blk = 0;
                int off = 0, len = 0;
                if (i < nseg)
                    clamped(i, blk, off, len);
                // running start of this segment among the sequence's positions
                int incl_len = len;
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int up = __shfl_up(incl_len, d, 64);
                    if (lane >= d)
                        incl_len += up;
                }
                const int start = run + incl_len - len;
                // the part of the segment inside [t0, t1)
                const int lo = max(start, t0), hi = min(start + len, t1);
                const int rows = max(hi - lo, 0);
                const int first = off + (lo - start);
                const int c = (rows + kSub - 1) / kSub;
                int incl = c;  // inclusive prefix sum over the wave
#pragma unroll
                for (int d = 1; d < 64; d <<= 1) {
                    const int up = __shfl_up(incl, d, 64);
                    if (lane >= d)
                        incl += up;
                }
                for (int k = 0; k < c; ++k) {
                    s_phys[incl - c + k] = blk;
                    s_rows[incl - c + k] = ((first + kSub * k) << 8) | min(kSub, rows - kSub * k);
                }
                if (lane == 63) {
                    s_total = incl;
                    s_run = run + incl_len;
                }
            }
            __syncthreads();
            const int total = s_total;
            run = __builtin_amdgcn_readfirstlane(s_run);
            const int T = total > w ? (total - w + WAVES - 1) / WAVES : 0;
            if (T > 0) {
                int j = w;
                KOp K;
                VRows V;
                {
                    const SubRsrc r = slot_rsrc(s_phys, s_rows, j, kp, vp, head_off, blk_elems);
                    load_k(K, r.k, lane);
                    load_v(V, r.v, lane);
                }
                u32x2 pb;
                float alpha;
                bool rs;
                for (int it = 0; it + 1 < T; ++it) {
                    const int cnt = __builtin_amdgcn_readfirstlane(s_rows[j]) & 0xff;
                    const SubRsrc rn =
                        slot_rsrc(s_phys, s_rows, j + WAVES, kp, vp, head_off, blk_elems);
                    const KOp KA = k_operand(K, klds, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    load_k(K, rn.k, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    rs = qk_softmax<DT, true>(st, KA, qop, 0, 0, cnt, lane, a.scale_log2, pb,
                                              alpha);
                    __builtin_amdgcn_sched_barrier(0);
                    stage_v(V, vlds, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    load_v(V, rn.v, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
                    __builtin_amdgcn_sched_barrier(0);
                    j += WAVES;
                }
                const int cnt = __builtin_amdgcn_readfirstlane(s_rows[j]) & 0xff;
                const KOp KA = k_operand(K, klds, lane);
                rs = qk_softmax<DT, true>(st, KA, qop, 0, 0, cnt, lane, a.scale_log2, pb, alpha);
                stage_v(V, vlds, lane);
                pv_mma<DT>(st, vlds, pb, rs, alpha, lane);
            }
            __syncthreads();  // the descriptors of this round are no longer read
        }
        st.l = pair_sum32(pair_sum16(st.l));

#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            *(f32x4 *)&sm.o[w][col][16 * jj + 4 * grp] = st.acc[jj];
        if (grp == 0) {
            s_m[w][col] = st.m;
            s_l[w][col] = st.l;
        }
        __syncthreads();
        for (int e = tid; e < G * 32; e += WAVES * 64) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            float M = s_m[0][qi];
#pragma unroll
            for (int i = 1; i < WAVES; ++i)
                M = fmaxf(M, s_m[i][qi]);
            const float ref = safe_ref(M);
            float L = 0.f;
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < WAVES; ++i) {
                const float wgt = fexp2(s_m[i][qi] - ref);
                L += s_l[i][qi] * wgt;
                O += *(const f32x4 *)&sm.o[i][qi][d0] * wgt;
            }
            const int64_t row = row0 + qi;
            if (direct) {
                f32x4 o = {0.f, 0.f, 0.f, 0.f};
                if (L > 0.f)
                    o = O / L;
                u32x2 packed;
                packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
                packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
                *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
            } else {
                // read by another work-group of the item (see arrive_last)
                const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
                st_ws4(ws.o, (int)((row * a.max_partitions + px) * kHeadDim + d0) * 4, O / L);
                if (d0 == 0)
                    st_ws1(ws.lse, (int)(row * a.max_partitions + px) * 4,
                           (ref + flog2(L)) * kLn2);
            }
        }
    }

    if constexpr (SPLIT) {
        // the work-groups that wrote partials arrive; the last one merges them
        if (direct || px0 >= np)
            return;
        if (!arrive_last(a.counters + rest, min(np, parts), &s_last))
            return;
        const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
        for (int e = tid; e < G * 32; e += WAVES * 64) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            const int64_t row = row0 + qi;
            const f32x4 o = merge_partials4(ws, (int)(row * a.max_partitions) * 4,
                                            (int)(row * a.max_partitions * kHeadDim + d0) * 4, np);
            u32x2 packed;
            packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
            packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
            *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
        }
    }
}

// Shared-prefix decode in one pass.  One work-group per (query tile, KV head).  A
// tile is NH halves of 16 MFMA columns; each half holds the G query heads of
// floor(16/G) consecutive member sequences of a group.  The work-group's
// sub-tiles are the group's prefix (positions 0 .. prefix_len-1, read once
// through the first member's table with every member's columns active) followed
// by each member's own positions (prefix_len .. n-1, read through its own table
// with only its G columns active: the other columns score -inf and keep their
// state).  The waves take the concatenated list round-robin with the decode
// kernel's score / softmax / P.V code, so every column ends with attention over
// exactly its sequence's n positions.  The optional append is written to the pool
// in the prologue, before a barrier, so the new rows are then read like any
// other.  No partials leave the work-group.
//
// The prefix is re-read from L2 by every tile of the group, and L2-to-CU
// delivery (about 12 TB/s for this access pattern on MI355X, measured with a
// plain read probe), not HBM, bounds the kernel.  Two halves per tile (NH = 2)
// halve the prefix re-reads: each K/V sub-tile feeds 32 columns, at the cost of
// twice the score and P.V work per prefix sub-tile.
template <int DT, int BS, int WAVES, int NH>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(NH == 1 ? 4 : 2)))
void prefix_fused_mfma_kernel(DecodeArgs a)
{
    constexpr int kCols = 16 * NH;   // query columns of a tile
    constexpr int kMembers = kCols;  // most member sequences of a tile (G = 1)
    // Each wave stages its sub-tiles in two buffers, one in each of two LDS arrays
    // (even steps in stage_a, odd ones in stage_b): the compiler tracks the
    // global-to-LDS loads into distinct arrays separately, so a read of one buffer
    // waits only for that buffer's loads.  The cross-wave merge reuses both arrays
    // (wave i's fp32 outputs [kCols][128] in stage_a for i < WAVES/2, else stage_b).
    __shared__ __attribute__((aligned(16))) char stage_a[WAVES][kDmaBufBytes];
    __shared__ __attribute__((aligned(16))) char stage_b[WAVES][kDmaBufBytes];
    static_assert(kCols * kHeadDim * 4 * (WAVES / 2) <= WAVES * kDmaBufBytes,
                  "the merge fits the staging arrays");
    __shared__ float s_m[WAVES][kCols], s_l[WAVES][kCols];
    __shared__ float s_wgt[WAVES][kCols];    // merge weight of wave i's partial of a column
    __shared__ int64_t s_row[kCols];         // output row of each query column, -1 if inactive
    __shared__ int32_t s_cum[kMembers + 1];  // sub-tiles before member i's own ones (s_cum[0]: prefix)
    __shared__ int32_t s_len[kMembers];      // context length of member i (0 outside the group)

    const int item = blockIdx.x;
    const int g = item % a.num_kv_heads;
    const int tile = item / a.num_kv_heads;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int spt = a.seqs_per_tile;  // NH * floor(16 / G)
    const int sph = spt / NH;         // member sequences per half
    const int s0 = tile * spt;
    const int s_end = min(a.num_seqs, s0 + spt);
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const bool fused = a.k_new != nullptr;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const meta_ptr tabs = as_meta(a.tables);
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)g * BS * kHeadDim;
    const int ch = g * G + col % G;  // query head of this lane's column
    int cm[NH];                      // member of this lane's column in each half
#pragma unroll
    for (int h = 0; h < NH; ++h)
        cm[h] = h * sph + col / G;

    // The query rows are requested first, before anything they do not depend on
    // (each lane loads a valid row: a column outside the tile reads a neighbour's).
    u32x4 qop[NH][4];
    auto load_q = [&]() {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const uint16_t *qrow =
                (const uint16_t *)a.q +
                ((int64_t)min(s0 + cm[h], s_end - 1) * a.num_q_heads + ch) * kHeadDim + grp * 8;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qop[h][kk] = *(const u32x4 *)(qrow + kk * 32);
        }
    };
    load_q();

    // A sub-tile of the work-group's list: its member (-1 for the prefix), first
    // token, the positions it covers and the rows it loads, and its block.
    struct Sub {
        int seg, tb, t_beg, t_end, t_load;
        int32_t phys;
    };
    // Each sub-tile goes global -> LDS into one of the wave's two staging
    // buffers: 8 vector-memory operations.  Prefix sub-tiles load with the
    // default cache policy, which keeps the prefix in L2 for the group's other
    // tiles; a member's own rows are read once and stream past the caches
    // (nontemporal), so they do not evict it: 23.7-24.1 against 26.0-26.4 us per
    // launch on 256 sequences sharing 512 tokens.
    const DmaLanes dl = dma_lanes(lane);
    char *const buf_a = stage_a[w];
    char *const buf_b = stage_b[w];
    auto dma = [&](const Sub &d, char *buf) {
        const SubRsrc r = sub_rsrc<BS>(d.phys, kp, vp, d.tb, d.t_load, head_off, blk_elems);
        if (d.seg >= 0)
            dma_sub<kLoadStream>(r.k, r.v, buf, dl);  // a member's own rows: read once
        else
            dma_sub(r.k, r.v, buf, dl);
    };

    int k = group_of(as_meta(a.group_cu), a.num_groups, s0);
    for (bool more = true, first = true; more; ++k) {
        const int ga = as_meta(a.group_cu)[k], gb = as_meta(a.group_cu)[k + 1];
        more = gb < s_end;
        if (ga == gb)
            continue;  // an empty group (uniform)
        const int plen = as_meta(a.prefix_lens)[k];
        const int start_sub = plen & ~(kSub - 1);
        bool active[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int cs = s0 + cm[h];
            active[h] = col < sph * G && cs < s_end && cs >= ga && cs < gb;
        }

        // The list opens with a head of the first min(P, 2 WAVES) prefix sub-tiles.
        // When the head holds both of each wave's first sub-tiles, their loads
        // are issued here, before the members' set-up: they depend on the group's
        // first row and prefix length only, and no appended row lies in the prefix
        // (a member appends at its own position n - 1 >= prefix length).
        const int n_pre = (plen + kSub - 1) / kSub;
        const int head = min(n_pre, 2 * WAVES);
        const bool early = n_pre >= 2 * WAVES;  // uniform
        auto prefix_sub = [&](int j) {
            Sub d;
            d.seg = -1;
            d.tb = j * kSub;
            d.t_beg = 0;
            d.t_end = plen;
            d.t_load = plen;
            d.phys = max(tabs[(int64_t)ga * a.width + min(d.tb / BS, a.width - 1)], 0);
            return d;
        };
        // wave 0 requests the members' lengths first: the set-up below waits for
        // them, and vector-memory results are counted in issue order
        const int s_m0 = s0 + lane;
        const bool in_m = w == 0 && lane < kMembers && lane < spt && s_m0 < s_end &&
                          s_m0 >= ga && s_m0 < gb;
        const int n_m = in_m ? a.lens[s_m0] : 0;
        __builtin_amdgcn_sched_barrier(0);
        // Without a long enough head the two loads are issued empty (zero-byte
        // ranges), so that the count of loads in flight is the same on both paths;
        // the real ones follow after the set-up.
        Sub cur = prefix_sub(w), nxt = prefix_sub(w + WAVES);
        if (!early) {
            cur.t_load = 0;
            nxt.t_load = 0;
        }
        dma(cur, buf_a);
        dma(nxt, buf_b);
        __builtin_amdgcn_sched_barrier(0);

        // per-member lengths and the cumulative sub-tile counts: lane i of wave 0
        // takes member i, and a wave prefix sum gives the running counts
        if (w == 0) {
            const int n = n_m;
            if (in_m && fused && g == 0 && n <= 0 && a.slot_out)
                a.slot_out[s_m0] = -1;  // padding sequence: nothing appended
            int incl = n > start_sub ? (n - start_sub + kSub - 1) / kSub : 0;
#pragma unroll
            for (int d = 1; d < kMembers; d <<= 1) {
                const int up = __shfl_up(incl, d, 64);
                incl += lane >= d ? up : 0;
            }
            const int base = n_pre;
            if (lane < kMembers) {
                s_len[lane] = n;
                s_cum[lane + 1] = base + incl;
            }
            if (lane == 0)
                s_cum[0] = base;
        }
        lds_barrier();  // the global-to-LDS loads above stay in flight
        const int total = __builtin_amdgcn_readfirstlane(s_cum[kMembers]);

        // a column outside this group scores zeros (a later group of the tile
        // reloads the rows zeroed by an earlier one)
        if (!first)
            load_q();
        first = false;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                qop[h][kk] = active[h] ? qop[h][kk] : (u32x4){0u, 0u, 0u, 0u};
        }
        GqaState st[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            st[h].m = kNegInf;
            st[h].l = 0.f;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                st[h].acc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }

        // Sub-tile j of the work-group's list: after the head, the list interleaves
        // the remaining prefix sub-tiles (seg -1, read from L2 after their first
        // use) evenly with the members' own ones (seg >= 0, mostly HBM reads), so
        // that HBM is busy through the whole loop instead of only once the prefix
        // is done.  With P' prefix sub-tiles among the T' positions after a head of
        // H, position H + j is prefix sub-tile H + pi, pi = floor(j P' / T'), when
        // floor((j+1) P' / T') exceeds pi, else the members' sub-tile j - pi,
        // counted member after member.
        //
        // A wave takes positions w, w + WAVES, ...  Its lanes describe the next 64
        // of them at once, each lane one position with its table entry, so the
        // table reads of 64 steps cost one round trip; a step then takes its
        // descriptor from the lanes with uniform lane reads.  A position past the
        // list describes an empty sub-tile (seg -2, a zero-byte buffer range).
        const int rest_pre = n_pre - head;
        const int rest = max(total - head, 1);  // positions after the head (none: 1)
        int d_seg, d_tb;                // this lane's position: member (or -1, -2), first token
        int32_t d_phys;                 // and its table entry
        auto describe_lanes = [&](int i0) {
            const int j = w + (i0 + lane) * WAVES;
            int row = ga;
            d_seg = -2;
            d_tb = 0;
            if (j < head) {
                d_seg = -1;
                d_tb = j * kSub;
            } else if (j < total) {
                const int64_t jp = (int64_t)(j - head) * rest_pre;
                const int pi = (int)(jp / rest), pi1 = (int)((jp + rest_pre) / rest);
                if (pi1 > pi) {
                    d_seg = -1;
                    d_tb = (head + pi) * kSub;
                } else {
                    const int jm = n_pre + (j - head) - pi;  // s_cum coordinate of a member sub-tile
                    int seg = 0;
#pragma unroll
                    for (int i = 1; i < kMembers; ++i)
                        seg += s_cum[i] <= jm ? 1 : 0;
                    d_seg = seg;
                    d_tb = start_sub + (jm - s_cum[seg]) * kSub;
                    row = s0 + seg;
                }
            }
            d_phys = 0;
            if (j < total)
                d_phys = a.tables[(int64_t)row * a.width + min(d_tb / BS, a.width - 1)];
        };
        // the descriptor of the wave's position i (i % 64 is the lane holding it)
        auto take = [&](int i) {
            const int l = i & 63;
            Sub d;
            d.seg = __builtin_amdgcn_readlane(d_seg, l);
            d.tb = __builtin_amdgcn_readlane(d_tb, l);
            d.phys = __builtin_amdgcn_readlane(d_phys, l);
            const bool own = d.seg >= 0;
            const int n = own ? __builtin_amdgcn_readfirstlane(s_len[own ? d.seg : 0]) : plen;
            d.t_beg = own ? plen : 0;
            d.t_end = n;
            d.t_load = d.seg == -2 ? 0 : n;
            d.seg = max(d.seg, -1);
            return d;
        };
        // The wave's k-th sub-tile is staged in buffer k % 2 (stage_a, stage_b).
        // Step k reads both operands of sub-tile k from its buffer into registers,
        // computes the scores and softmax, refills the buffer with sub-tile k + 2,
        // and then runs P.V, so the loads of two sub-tiles are in flight behind the
        // current one's work.  Steps -2 and -1 only issue the loads of sub-tiles 0
        // and 1 (issued above already when the head holds them).  The loop is
        // unrolled by two so that each step names its buffer.
        //
        // Vector-memory operations are issued in this order only (the scheduling
        // barriers keep the compiler from moving them): step k issues the 8 loads
        // of sub-tile k + 2, preceded every 64 steps by the table reads of the next
        // 64 positions.  When step k reads sub-tile k, at least the 8 loads of
        // sub-tile k + 1 were issued after that sub-tile's loads: waiting until at
        // most 8 operations are outstanding covers it.
        constexpr int kReadWait = 8;
        auto step = [&](auto parity, auto run, Sub &cur, Sub &nxt, int k) {
            constexpr bool RUN = decltype(run)::value;
            char *const buf = decltype(parity)::value ? buf_b : buf_a;
            i16x4 va[8];
            u32x2 pb[NH];
            float alpha[NH];
            bool rs[NH];
            // A member's own sub-tile has active columns only in the half holding
            // the member: the other half's scores, softmax and P.V are skipped
            // (wave-uniform), leaving its state as it was.
            bool live[NH];
#pragma unroll
            for (int h = 0; h < NH; ++h)
                live[h] = RUN && (cur.seg < 0 || (cur.seg >= h * sph && cur.seg < (h + 1) * sph));
            if constexpr (RUN) {
                __builtin_amdgcn_sched_barrier(0);
                PKV_WAIT_VMCNT(kReadWait);  // this buffer's loads have landed
                __builtin_amdgcn_sched_barrier(0);
                const KOp KA = dma_read_k(buf, dl);
                dma_read_v(va, buf, dl);
                // a prefix sub-tile that the prefix fills needs no mask: its
                // positions are all in range, and a column outside the tile only
                // updates a state that is never written out
                if (cur.seg < 0 && cur.tb + kSub <= cur.t_end) {
#pragma unroll
                    for (int h = 0; h < NH; ++h)
                        rs[h] = qk_softmax<DT, false>(st[h], KA, qop[h], cur.tb, 0, cur.t_end,
                                                      lane, a.scale_log2, pb[h], alpha[h]);
                } else {
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        rs[h] = false;
                        if (live[h]) {
                            const bool on =
                                cur.seg < 0 ? active[h] : (active[h] && cm[h] == cur.seg);
                            rs[h] = qk_softmax<DT, true>(st[h], KA, qop[h], cur.tb, cur.t_beg,
                                                         cur.t_end, lane, a.scale_log2, pb[h],
                                                         alpha[h], on);
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                PKV_WAIT_LGKM0();  // this buffer's reads are done: refill it
            }
            __builtin_amdgcn_sched_barrier(0);
            if (((k + 2) & 63) == 0 && k + 2 > 0)
                describe_lanes(k + 2);
            const Sub nxt2 = take(k + 2);
            dma(nxt2, buf);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (RUN)
                pv_mma_regs<DT, NH>(st, va, pb, rs, alpha, live);
            __builtin_amdgcn_sched_barrier(0);
            cur = nxt;
            nxt = nxt2;
        };
        // the descriptors' table reads go out before the append, whose latency
        // they share
        if (w < total)
            describe_lanes(0);
        // Fused append, spread over the work-group: each thread moves one 16-byte
        // chunk of a member's new K or V row to its slot.  The barrier below makes
        // the rows visible to the whole work-group, so the member's last sub-tile
        // then reads position n-1 from the pool like any other row (substituting
        // the rows in registers instead cost about 50 registers per lane).
        if (fused) {
            for (int e = tid; e < spt * 32; e += WAVES * 64) {
                const int i = e >> 5, kv = (e >> 4) & 1, c = e & 15;
                const int n = s_len[i];
                if (n <= plen)
                    continue;  // not in the group, or nothing to append past the prefix
                const int s = s0 + i;
                const int tn = n - 1;
                const int64_t phys_n = tabs[(int64_t)s * a.width + tn / BS];
                const int64_t src = ((int64_t)s * a.num_kv_heads + g) * kHeadDim + 8 * c;
                const u32x4 val =
                    *(const u32x4 *)((const uint16_t *)(kv ? a.v_new : a.k_new) + src);
                const int64_t dst =
                    phys_n * blk_elems + head_off + (int64_t)(tn % BS) * kHeadDim + 8 * c;
                *(u32x4 *)((uint16_t *)(kv ? a.v_pool : a.k_pool) + dst) = val;
                if (g == 0 && kv == 0 && c == 0 && a.slot_out)
                    a.slot_out[s] = phys_n * BS + tn % BS;
            }
        }
        __syncthreads();

        if (w < total) {
            using even = std::integral_constant<int, 0>;
            using odd = std::integral_constant<int, 1>;
            using warm = std::false_type;
            using full = std::true_type;
            if (!early) {
                step(even(), warm(), cur, nxt, -2);
                step(odd(), warm(), cur, nxt, -1);
            }
            const int steps = (total - w + WAVES - 1) / WAVES;
            for (int k = 0;;) {
                step(even(), full(), cur, nxt, k);
                if (++k >= steps)
                    break;
                step(odd(), full(), cur, nxt, k);
                if (++k >= steps)
                    break;
            }
        }
        // the loads of the sub-tiles past the list still write this wave's buffers
        PKV_WAIT_VMCNT(0);
#pragma unroll
        for (int h = 0; h < NH; ++h)
            st[h].l = pair_sum32(pair_sum16(st[h].l));

        __syncthreads();  // every wave is done with its staging buffers
        // wave i's outputs: 16-byte chunk q of column r at chunk q ^ (r % 16) of
        // the column's 512-byte row, so that the 16 columns one write (or read)
        // instruction covers fall in different banks
        auto o_area = [&](int i) -> float * {
            char *const base = i < WAVES / 2 ? &stage_a[0][0] : &stage_b[0][0];
            return (float *)base + (i % (WAVES / 2)) * (kCols * kHeadDim);
        };
        {
            float *const ow = o_area(w);
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const int r = 16 * h + col;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    *(f32x4 *)&ow[r * kHeadDim + 4 * ((4 * jj + grp) ^ (r & 15))] = st[h].acc[jj];
            }
        }
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            if (grp == 0) {
                s_m[w][16 * h + col] = st[h].m;
                s_l[w][16 * h + col] = st[h].l;
            }
        }
        if (tid < kCols) {
            const int h = tid / 16, c = tid % 16;
            const int mi = h * sph + c / G, cs = s0 + mi;
            const bool act = c < sph * G && cs < s_end && cs >= ga && cs < gb;
            s_row[tid] = act ? (int64_t)cs * a.num_q_heads + g * G + c % G : -1;
        }
        __syncthreads();
        // the weight of wave i's partial of column qi: exp2(m_i - M) / L, with M
        // the column's largest reference max and L its merged denominator (0 for
        // an empty column)
        if (tid < WAVES * kCols) {
            const int i = tid / kCols, qi = tid % kCols;
            float M = s_m[0][qi];
#pragma unroll
            for (int v = 1; v < WAVES; ++v)
                M = fmaxf(M, s_m[v][qi]);
            const float ref = safe_ref(M);
            float L = 0.f;
#pragma unroll
            for (int v = 0; v < WAVES; ++v)
                L += s_l[v][qi] * fexp2(s_m[v][qi] - ref);
            s_wgt[i][qi] = L > 0.f ? fexp2(s_m[i][qi] - ref) / L : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < kCols * 32; e += WAVES * 64) {
            const int qi = e >> 5, d0 = (e & 31) * 4;
            const int64_t row = s_row[qi];
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < WAVES; ++i)
                o += *(const f32x4 *)&o_area(i)[qi * kHeadDim + 4 * ((d0 / 4) ^ (qi & 15))] *
                     s_wgt[i][qi];
            if (row < 0)
                continue;
            u32x2 packed;
            packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
            packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
            *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
        }
        if (more)
            __syncthreads();  // LDS is reused by the next group of the tile
    }
}

// Slotted decode in tiles of sequences.  One work-group per (query tile, KV head),
// with the tile of the one-pass shared-prefix kernel: NH halves of 16 MFMA
// columns, each holding the G query heads of floor(16/G) consecutive sequences.
// A radix-tree batch lists each sequence as the path of nodes from the root, so
// consecutive sequences start with the same segments.  The tile's common segments
// -- the leading triples that every member lists identically, found by comparing
// the first kCommonScan of them -- become sub-tiles read once for the whole tile
// with every column active.  Of the remaining segments, one that a run of
// consecutive members lists at the same index (a node under the common path that
// part of the tile shares; in a batch in tree order, the sequences under one node
// are neighbours) becomes sub-tiles read once for the run, with the run's columns
// active; the others, sub-tiles of one member (the other columns score -inf and
// keep their state).  The whole list of descriptors sits in LDS: the host takes
// this path only when a tile's sub-tiles fit (members x max_segments x ceil(B/16)
// <= kTileSubs).  The waves take the list round-robin with the common sub-tiles
// spread evenly among the members' ones, as in the shared-prefix kernel.
constexpr int kTileSubs = kSlottedTileSubs;  // descriptor capacity of one tile's list
constexpr int kCommonScan = 64;              // leading segments compared across a tile

__device__ __forceinline__ int wave_sum_i(int x)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
        x += __shfl_xor(x, d, 64);
    return x;
}

// Sub-tile descriptor: physical block, and first row | row count << 8 | lo << 16 |
// hi << 21: the sub-tile belongs to members lo..hi of the tile (0..31 for a common
// sub-tile).
__device__ __forceinline__ int32_t slot_desc(int first_row, int rows, int lo, int hi)
{
    return first_row | (rows << 8) | (lo << 16) | (hi << 21);
}

template <int DT, int BS, int WAVES, int NH>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void slotted_tiled_mfma_kernel(DecodeArgs a)
{
    constexpr int kCols = 16 * NH;   // query columns of a tile
    constexpr int kMembers = kCols;  // most member sequences of a tile (G = 1)
    // two staging buffers per wave in two LDS arrays, as in the one-pass
    // shared-prefix kernel; the cross-wave merge reuses them
    __shared__ __attribute__((aligned(16))) char stage_a[WAVES][kDmaBufBytes];
    __shared__ __attribute__((aligned(16))) char stage_b[WAVES][kDmaBufBytes];
    static_assert(kCols * kHeadDim * 4 * (WAVES / 2) <= WAVES * kDmaBufBytes,
                  "the merge fits the staging arrays");
    __shared__ float s_m[WAVES][kCols], s_l[WAVES][kCols];
    __shared__ int32_t s_phys[kTileSubs];
    __shared__ int32_t s_desc[kTileSubs];
    __shared__ uint64_t s_diff[WAVES];  // per wave: segment indices where a member differs
    __shared__ uint64_t s_same[kMembers];  // member i: segment indices equal to member i-1's
    __shared__ int32_t s_cnt[kMembers];  // each member's own sub-tiles
    __shared__ int32_t s_ncom;          // common sub-tiles

    const int item = blockIdx.x;
    const int g = item % a.num_kv_heads;
    const int tile = item / a.num_kv_heads;
    const int G = a.num_q_heads / a.num_kv_heads;
    const int spt = a.seqs_per_tile;  // NH * floor(16 / G)
    const int sph = spt / NH;         // member sequences per half
    const int s0 = tile * spt;
    const int m = min(a.num_seqs - s0, spt);  // members of this tile, >= 1
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int col = lane & 15, grp = lane >> 4;
    const int ms = a.max_segments;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)g * BS * kHeadDim;
    // segments of member i, and how many are in use (clamped to the row)
    auto seg_row = [&](int i) { return a.segments + (int64_t)(s0 + i) * ms * 3; };
    auto seg_count = [&](int i) { return min(max(a.num_segments[s0 + i], 0), ms); };
    // a segment never reaches outside its block, whatever the caller passed
    auto clamp_seg = [&](int &off, int &len) {
        off = min(max(off, 0), BS);
        len = min(max(len, 0), BS - off);
    };

    const int ch = g * G + col % G;  // query head of this lane's column
    int cm[NH];                      // member of this lane's column in each half
    bool active[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        cm[h] = h * sph + col / G;
        active[h] = col < sph * G && cm[h] < m;
    }
    // every lane loads a valid query row (inactive columns read a neighbour's and
    // zero it): no load sits under a lane-dependent branch.  The rows are
    // requested first, so that they have landed long before the loop starts.
    u32x4 qop[NH][4];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const uint16_t *qrow = (const uint16_t *)a.q +
                               ((int64_t)(s0 + min(cm[h], m - 1)) * a.num_q_heads + ch) *
                                   kHeadDim +
                               grp * 8;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const u32x4 v = *(const u32x4 *)(qrow + kk * 32);
            qop[h][kk] = active[h] ? v : (u32x4){0u, 0u, 0u, 0u};
        }
    }
    // 0. Fused append: each wave takes members w, w + WAVES, ...; their loads are
    // in flight with step 1's, the stores go out after step 1's barrier, and the
    // barriers that follow order them before any wave's sub-tile loads
    constexpr int kPer = (kMembers + WAVES - 1) / WAVES;
    SlotAppend ap[kPer];
    if (a.k_new) {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (w + j * WAVES < m)
                ap[j] = slot_append_load(a, s0 + w + j * WAVES, g, lane);
    }

    // 1. Lane k compares segment k (k < 64) of every member with member 0's (the
    // segments common to the tile) and with the previous member's (runs of
    // members that share a segment, such as a node under the tile's common path);
    // each wave takes members w, w + WAVES, ...  Every lane reads an entry of its
    // own row (segment min(k, max_segments - 1)), so the segment loads go out with
    // the counts' instead of after them; the counts mask the comparisons.
    const int kseg = min(lane, ms - 1);
    const int n0 = seg_count(0);
    const int32_t *r0 = seg_row(0) + 3 * kseg;
    const int b0 = r0[0], o0 = r0[1], l0 = r0[2];  // used for lanes below n0 only
    {
        bool diff = lane >= n0;
        for (int i = w; i < m; i += WAVES) {
            if (i == 0)
                continue;
            const int ni = seg_count(i), np = seg_count(i - 1);
            const int32_t *r = seg_row(i) + 3 * kseg, *rp = seg_row(i - 1) + 3 * kseg;
            const int bi = r[0], oi = r[1], li = r[2];
            diff |= lane >= ni || bi != b0 || oi != o0 || li != l0;
            const bool same = lane < ni && lane < np && bi == rp[0] && oi == rp[1] && li == rp[2];
            const uint64_t sm = __ballot(same);
            if (lane == 0)
                s_same[i] = sm;
        }
        if (w == 0 && lane == 0)
            s_same[0] = 0;
        const uint64_t d = __ballot(diff);
        if (lane == 0)
            s_diff[w] = d;
    }
    __syncthreads();
    int ncom;
    {
        uint64_t d = 0;
#pragma unroll
        for (int i = 0; i < WAVES; ++i)
            d |= s_diff[i];
        ncom = d ? __builtin_ctzll(d) : kCommonScan;
    }
    if (a.k_new) {
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            if (w + j * WAVES < m)
                slot_append_store<BS>(a, ap[j], s0 + w + j * WAVES, g, lane);
    }

    // 2. The common sub-tiles (wave 0, from member 0's segments) at the head of
    // the list, and each member's count of the other sub-tiles it starts: those
    // of its segments that do not repeat the previous member's
    if (w == 0) {
        int off = o0, len = l0;
        clamp_seg(off, len);
        const int c = lane < ncom ? (len + kSub - 1) / kSub : 0;
        int incl = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int up = __shfl_up(incl, d, 64);
            incl += lane >= d ? up : 0;
        }
        for (int k = 0; k < c; ++k) {
            s_phys[incl - c + k] = b0;
            s_desc[incl - c + k] =
                slot_desc(off + kSub * k, min(kSub, len - kSub * k), 0, kMembers - 1);
        }
        if (lane == 63)
            s_ncom = incl;
    }
    for (int i = w; i < m; i += WAVES) {
        const int ni = seg_count(i);
        const int32_t *r = seg_row(i);
        const uint64_t same = s_same[i];
        int cnt = 0;
        for (int base = ncom; base < ni; base += 64) {
            const int k = base + lane;
            int c = 0;
            if (k < ni && !(k < 64 && ((same >> k) & 1))) {
                int off = r[3 * k + 1], len = r[3 * k + 2];
                clamp_seg(off, len);
                c = (len + kSub - 1) / kSub;
            }
            cnt += wave_sum_i(c);
        }
        if (lane == 0)
            s_cnt[i] = cnt;
    }
    __syncthreads();

    // 3. The sub-tiles each member starts, member after member, after the common
    // ones; a segment shared by members i..j (each repeating the previous one's)
    // is read once, for all of them
    const int n_pre = __builtin_amdgcn_readfirstlane(s_ncom);
    int total = n_pre;
    for (int i = 0; i < m; ++i)
        total += __builtin_amdgcn_readfirstlane(s_cnt[i]);
    for (int i = w; i < m; i += WAVES) {
        int pos = n_pre;
        for (int k = 0; k < i; ++k)
            pos += __builtin_amdgcn_readfirstlane(s_cnt[k]);
        const int ni = seg_count(i);
        const int32_t *r = seg_row(i);
        const uint64_t same = s_same[i];
        for (int base = ncom; base < ni; base += 64) {
            const int kk = base + lane;
            int blk = 0, off = 0, len = 0, c = 0, hi = i;
            if (kk < ni && !(kk < 64 && ((same >> kk) & 1))) {
                blk = r[3 * kk];
                off = r[3 * kk + 1];
                len = r[3 * kk + 2];
                clamp_seg(off, len);
                c = (len + kSub - 1) / kSub;
                // the run of following members that repeat this segment
                if (kk < 64)
                    while (hi + 1 < m && ((s_same[hi + 1] >> kk) & 1))
                        ++hi;
            }
            int incl = c;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int up = __shfl_up(incl, d, 64);
                incl += lane >= d ? up : 0;
            }
            for (int k = 0; k < c; ++k) {
                s_phys[pos + incl - c + k] = blk;
                s_desc[pos + incl - c + k] =
                    slot_desc(off + kSub * k, min(kSub, len - kSub * k), i, hi);
            }
            pos += __builtin_amdgcn_readlane(incl, 63);
        }
    }
    __syncthreads();

    GqaState st[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        st[h].m = kNegInf;
        st[h].l = 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            st[h].acc[jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    // Position j of the list is common sub-tile pi = floor(j P / T) when
    // floor((j+1) P / T) exceeds pi, else the members' sub-tile j - pi (entry
    // P + j - pi).  A j past the list describes an empty sub-tile (zero rows, so
    // its buffer range is empty and nothing is fetched), so every step issues its
    // loads the same way.  A wave takes positions w, w + WAVES, ...: its lanes
    // hold the descriptors of the next 64 of them (lane l: the wave's position
    // i0 + l), read from the LDS list once per 64 steps, and a step takes its own
    // with two lane reads.  The list holds at most kTileSubs entries, so j P fits
    // in 32 bits.
    struct Sub {
        int32_t phys, desc;
    };
    static_assert((int64_t)kTileSubs * kTileSubs < ((int64_t)1 << 31), "32-bit quotients");
    const int tot = max(total, 1);
    int d_phys = 0, d_desc = 0;  // this lane's position of the wave's current 64
    auto describe_lanes = [&](int i0) {
        const int j = w + (i0 + lane) * WAVES;
        int idx = 0;
        const bool past = j >= total;
        if (!past) {
            const int pi = j * n_pre / tot, pi1 = (j + 1) * n_pre / tot;
            idx = pi1 > pi ? pi : n_pre + j - pi;
        }
        d_phys = s_phys[idx];
        d_desc = past ? 0 : s_desc[idx];
    };
    // the descriptor of the wave's position i (i % 64 is the lane holding it)
    auto take = [&](int i) {
        Sub d;
        d.phys = __builtin_amdgcn_readlane(d_phys, i & 63);
        d.desc = __builtin_amdgcn_readlane(d_desc, i & 63);
        return d;
    };
    // Sub-tile k of the wave goes global -> LDS into buffer k % 2 (stage_a,
    // stage_b): 8 vector-memory operations.  Step k reads sub-tile k's operands,
    // computes its scores and softmax, refills the buffer with sub-tile k + 2 and
    // runs P.V; steps -2 and -1 only issue the first two sub-tiles' loads.  The
    // loop issues no other vector-memory operation (the descriptors come from
    // LDS), so when step k reads, the 8 loads of sub-tile k + 1 were issued after
    // sub-tile k's: waiting until at most 8 are outstanding covers them.  Segments
    // common to the whole tile load with the default cache policy (other tiles of
    // the batch read them too); member and run sub-tiles, read once, stream past
    // the caches (27.1-27.4 against 28.1-28.4 us on the radix batch).
    const DmaLanes dl = dma_lanes(lane);
    char *const buf_a = stage_a[w];
    char *const buf_b = stage_b[w];
    auto dma = [&](const Sub &d, char *buf) {
        const int64_t b = (int64_t)d.phys * blk_elems + head_off +
                          (int64_t)(d.desc & 0xff) * kHeadDim;
        const int bytes = ((d.desc >> 8) & 0xff) * kHeadDim * 2;
        const int lo = (d.desc >> 16) & 31, hi = (d.desc >> 21) & 31;
        if (lo == 0 && hi >= m - 1)  // a segment of the whole tile: other tiles read it too
            dma_sub(make_rsrc(kp + b, bytes), make_rsrc(vp + b, bytes), buf, dl);
        else
            dma_sub<kLoadStream>(make_rsrc(kp + b, bytes), make_rsrc(vp + b, bytes), buf, dl);
    };
    constexpr int kReadWait = 8;
    auto step = [&](auto parity, auto run, Sub &cur, Sub &nxt, int kn) {
        constexpr bool RUN = decltype(run)::value;
        char *const buf = decltype(parity)::value ? buf_b : buf_a;
        if (kn > 0 && (kn & 63) == 0)
            describe_lanes(kn);
        const Sub nxt2 = take(kn);
        i16x4 va[8];
        u32x2 pb[NH];
        float alpha[NH];
        bool rs[NH];
        const int rows = (cur.desc >> 8) & 0xff;
        const int lo = (cur.desc >> 16) & 31, hi = (cur.desc >> 21) & 31;  // its members
        // a half that holds none of the sub-tile's members skips its scores,
        // softmax and P.V (uniform)
        bool live[NH];
#pragma unroll
        for (int h = 0; h < NH; ++h)
            live[h] = RUN && hi >= h * sph && lo < (h + 1) * sph;
        if constexpr (RUN) {
            __builtin_amdgcn_sched_barrier(0);
            PKV_WAIT_VMCNT(kReadWait);  // this buffer's loads have landed
            __builtin_amdgcn_sched_barrier(0);
            const KOp KA = dma_read_k(buf, dl);
            dma_read_v(va, buf, dl);
            // a full sub-tile of every member needs no mask: a column outside the
            // tile only updates a state that is never written out
            if (lo == 0 && hi >= m - 1 && rows == kSub) {
#pragma unroll
                for (int h = 0; h < NH; ++h)
                    rs[h] = qk_softmax<DT, false>(st[h], KA, qop[h], 0, 0, kSub, lane,
                                                  a.scale_log2, pb[h], alpha[h]);
            } else {
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    rs[h] = false;
                    if (live[h]) {
                        const bool on = active[h] && cm[h] >= lo && cm[h] <= hi;
                        rs[h] = qk_softmax<DT, true>(st[h], KA, qop[h], 0, 0, rows, lane,
                                                     a.scale_log2, pb[h], alpha[h], on);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            PKV_WAIT_LGKM0();  // this buffer's reads are done: refill it
        }
        __builtin_amdgcn_sched_barrier(0);
        dma(nxt2, buf);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (RUN)
            pv_mma_regs<DT, NH>(st, va, pb, rs, alpha, live);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
        nxt = nxt2;
    };
    if (w < total) {
        using even = std::integral_constant<int, 0>;
        using odd = std::integral_constant<int, 1>;
        Sub cur{}, nxt{};
        describe_lanes(0);
        step(even(), std::false_type(), cur, nxt, 0);
        step(odd(), std::false_type(), cur, nxt, 1);
        // step k consumes the wave's sub-tile k (position w + k WAVES) and issues
        // the loads of sub-tile k + 2
        for (int k = 0;;) {
            step(even(), std::true_type(), cur, nxt, k + 2);
            if (w + ++k * WAVES >= total)
                break;
            step(odd(), std::true_type(), cur, nxt, k + 2);
            if (w + ++k * WAVES >= total)
                break;
        }
    }
    // the loads of the sub-tiles past the list still write this wave's buffers
    PKV_WAIT_VMCNT(0);
#pragma unroll
    for (int h = 0; h < NH; ++h)
        st[h].l = pair_sum32(pair_sum16(st[h].l));

    __syncthreads();  // every wave is done with its staging buffers
    // wave i's outputs: 16-byte chunk q of column r at chunk q ^ (r % 16) of the
    // column's 512-byte row
    auto o_area = [&](int i) -> float * {
        char *const base = i < WAVES / 2 ? &stage_a[0][0] : &stage_b[0][0];
        return (float *)base + (i % (WAVES / 2)) * (kCols * kHeadDim);
    };
    {
        float *const ow = o_area(w);
#pragma unroll
        for (int h = 0; h < NH; ++h) {
            const int r = 16 * h + col;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                *(f32x4 *)&ow[r * kHeadDim + 4 * ((4 * jj + grp) ^ (r & 15))] = st[h].acc[jj];
        }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        if (grp == 0) {
            s_m[w][16 * h + col] = st[h].m;
            s_l[w][16 * h + col] = st[h].l;
        }
    }
    __syncthreads();
    for (int e = tid; e < kCols * 32; e += WAVES * 64) {
        const int qi = e >> 5, d0 = (e & 31) * 4;
        const int h = qi / 16, c = qi % 16;
        const int mi = h * sph + c / G;
        if (c >= sph * G || mi >= m)
            continue;
        const int64_t row = (int64_t)(s0 + mi) * a.num_q_heads + g * G + c % G;
        float M = s_m[0][qi];
#pragma unroll
        for (int i = 1; i < WAVES; ++i)
            M = fmaxf(M, s_m[i][qi]);
        const float ref = safe_ref(M);
        float L = 0.f;
        f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < WAVES; ++i) {
            const float wgt = fexp2(s_m[i][qi] - ref);
            L += s_l[i][qi] * wgt;
            O += *(const f32x4 *)&o_area(i)[qi * kHeadDim + 4 * ((d0 / 4) ^ (qi & 15))] * wgt;
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
        if (L > 0.f)
            o = O / L;
        u32x2 packed;
        packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
        packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
        *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
    }
}

}  // namespace

// Waves per work-group (tuning knobs): the decode kernel, its suffix pass in
// shared-prefix mode, and the prefix pass.
#ifndef PKV_MFMA_WAVES
#define PKV_MFMA_WAVES 4
#endif
#ifndef PKV_SUFFIX_WAVES
#define PKV_SUFFIX_WAVES 4
#endif
#ifndef PKV_PREFIX_WAVES
#define PKV_PREFIX_WAVES 4
#endif
// one-pass shared-prefix kernel (8 waves measured faster than 4 with two halves
// per tile; its LDS merge area allows at most 8)
#ifndef PKV_PFX_FUSED_WAVES
#define PKV_PFX_FUSED_WAVES 8
#endif

template <int DT, int BS>
static hipError_t launch_mfma_t(const DecodeArgs &a, hipStream_t stream)
{
    constexpr int W = PKV_MFMA_WAVES;
    constexpr int WS = PKV_SUFFIX_WAVES;
    if (a.group_cu && a.counters)
        hipLaunchKernelGGL((decode_mfma_kernel<DT, BS, WS, kModeSuffixSplit>), dim3(a.n_items),
                           dim3(WS * 64), 0, stream, a);
    else if (a.group_cu)
        hipLaunchKernelGGL((decode_mfma_kernel<DT, BS, WS, kModeSuffix>), dim3(a.n_items),
                           dim3(WS * 64), 0, stream, a);
    else if (a.partition_size > 0 && a.counters)
        hipLaunchKernelGGL((decode_mfma_kernel<DT, BS, W, kModeMerge>), dim3(a.n_items),
                           dim3(W * 64), 0, stream, a);
    else if (a.partition_size > 0)
        hipLaunchKernelGGL((decode_mfma_kernel<DT, BS, W, kModeSplit>), dim3(a.n_items),
                           dim3(W * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<DT, BS, W, kModeSingle>), dim3(a.n_items),
                           dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DT, int BS>
static hipError_t launch_prefix_t(const DecodeArgs &a, int n_items, hipStream_t stream)
{
    constexpr int W = PKV_PREFIX_WAVES;
    hipLaunchKernelGGL((prefix_mfma_kernel<DT, BS, W>), dim3(n_items), dim3(W * 64), 0, stream,
                       a);
    return hipGetLastError();
}

template <int DT, int BS>
static hipError_t launch_prefix_fused_t(const DecodeArgs &a, int n_items, hipStream_t stream)
{
    constexpr int W = PKV_PFX_FUSED_WAVES;
    hipLaunchKernelGGL((prefix_fused_mfma_kernel<DT, BS, W, kPrefixHalves>), dim3(n_items),
                       dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_prefix_fused_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                                    hipStream_t stream)
{
#define PKV_PX_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_prefix_fused_t<kFp16, BSV>(a, n_items, stream)    \
                              : launch_prefix_fused_t<kBf16, BSV>(a, n_items, stream);
    switch (block_size) {
        PKV_PX_CASE(16)
        PKV_PX_CASE(32)
        PKV_PX_CASE(64)
        PKV_PX_CASE(128)
        PKV_PX_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_PX_CASE
}

hipError_t launch_prefix_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                              hipStream_t stream)
{
#define PKV_PF_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_prefix_t<kFp16, BSV>(a, n_items, stream)          \
                              : launch_prefix_t<kBf16, BSV>(a, n_items, stream);
    switch (block_size) {
        PKV_PF_CASE(16)
        PKV_PF_CASE(32)
        PKV_PF_CASE(64)
        PKV_PF_CASE(128)
        PKV_PF_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_PF_CASE
}

template <int DT, int BS>
static hipError_t launch_slotted_t(const DecodeArgs &a, hipStream_t stream)
{
    constexpr int W = PKV_MFMA_WAVES;
    if (a.partition_size > 0)
        hipLaunchKernelGGL((slotted_mfma_kernel<DT, BS, W, true>), dim3(a.n_items), dim3(W * 64),
                           0, stream, a);
    else
        hipLaunchKernelGGL((slotted_mfma_kernel<DT, BS, W>), dim3(a.n_items), dim3(W * 64), 0,
                           stream, a);
    return hipGetLastError();
}

template <int DT, int BS>
static hipError_t launch_slotted_tiled_t(const DecodeArgs &a, int n_items, hipStream_t stream)
{
    constexpr int W = PKV_PFX_FUSED_WAVES;
    hipLaunchKernelGGL((slotted_tiled_mfma_kernel<DT, BS, W, kPrefixHalves>), dim3(n_items),
                       dim3(W * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_slotted_tiled_mfma(const DecodeArgs &a, int n_items, int dtype, int block_size,
                                     hipStream_t stream)
{
#define PKV_ST_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_slotted_tiled_t<kFp16, BSV>(a, n_items, stream)   \
                              : launch_slotted_tiled_t<kBf16, BSV>(a, n_items, stream);
    switch (block_size) {
        PKV_ST_CASE(16)
        PKV_ST_CASE(32)
        PKV_ST_CASE(64)
        PKV_ST_CASE(128)
        PKV_ST_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_ST_CASE
}

hipError_t launch_slotted_mfma(const DecodeArgs &a, int dtype, int block_size, hipStream_t stream)
{
#define PKV_SL_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_slotted_t<kFp16, BSV>(a, stream)                  \
                              : launch_slotted_t<kBf16, BSV>(a, stream);
    switch (block_size) {
        PKV_SL_CASE(16)
        PKV_SL_CASE(32)
        PKV_SL_CASE(64)
        PKV_SL_CASE(128)
        PKV_SL_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_SL_CASE
}

hipError_t launch_decode_mfma(const DecodeArgs &a, int dtype, int block_size, hipStream_t stream)
{
#define PKV_MF_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_mfma_t<kFp16, BSV>(a, stream)                     \
                              : launch_mfma_t<kBf16, BSV>(a, stream);
    switch (block_size) {
        PKV_MF_CASE(16)
        PKV_MF_CASE(32)
        PKV_MF_CASE(64)
        PKV_MF_CASE(128)
        PKV_MF_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_MF_CASE
}

}  // namespace pkv
