// decode_g1.hip -- paged decode attention for one query head per KV head (MHA).
//
// What it computes: for sequence s and head h, softmax(scale * q.K^T) V over the
// logical tokens of the work item, each token fetched through the block table
// (page "显存虚拟化革命：PagedAttention 内存池管理与显存碎片终结", blog.llmgo.top,
// §五.1: loop over logical blocks, look up the physical block, load its K/V tile,
// QK^T with running softmax scaling, normalise, store).
//
// gfx950 design.  With one query row per KV head each K/V element is used by
// exactly one multiply-add, so this path is HBM-bound with no reuse to exploit:
// MFMA would only pad a vector product to a 16-row tile.  The kernel therefore
// streams K/V straight into VGPRs with 16-byte loads and reduces on the VALU:
//   * a work-group is 4 wave64s; one work-group per (sequence, head[, partition]);
//   * tokens are processed in tiles of 32; the waves of a work-group take tiles
//     round-robin and double-buffer them in registers (the loads of tile k+4 are
//     in flight while tile k is computed);
//   * lane l = 16*r + c owns dims 8c..8c+7 of token 4i+r of the tile (i = 0..7):
//     every load instruction of the wave covers 4 consecutive token rows = 1 KiB
//     of contiguous memory, and the same mapping serves K and V;
//   * q.k partial dots use v_dot2_f32_{f16,bf16}; the 16 lanes of a row are summed
//     with four DPP row operations, leaving the score in all 16 lanes;
//   * each 16-lane row keeps its own running max / sum / accumulator over its
//     tokens (4i+r), so the per-tile softmax needs no cross-row traffic; rows,
//     then waves (through LDS) are merged once at the end with the log-sum-exp
//     rule.
// Reduction order depends only on logical token positions, so the result is
// bitwise invariant under any relabelling of physical blocks.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;
constexpr int kTile = 32;  // tokens per tile

template <int DT, int BS>
struct G1Tile {
    u32x4 k[8];
    u32x4 v[8];
};

// Issue the 16 loads of tile `tb` (first token of the tile).  Every address is
// inside a block that holds tokens of the item: for BS >= 32 the whole tile sits
// in block tb/BS; for BS == 16 the second half uses block tb/16+1 only when it
// holds tokens, else it re-reads the first block (those rows are masked).
template <int DT, int BS>
__device__ __forceinline__ void load_tile(G1Tile<DT, BS> &t, const uint16_t *__restrict__ kp,
                                          const uint16_t *__restrict__ vp,
                                          const int32_t *__restrict__ trow, int tb, int t_end,
                                          int64_t head_off, int64_t blk_elems, int lane_off)
{
    if constexpr (BS >= kTile) {
        const int64_t phys = trow[tb / BS];
        const int64_t base = phys * blk_elems + head_off + (int64_t)(tb % BS) * kHeadDim;
        const uint16_t *kb = kp + base + lane_off;
        const uint16_t *vb = vp + base + lane_off;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.k[i] = *(const u32x4 *)(kb + i * 4 * kHeadDim);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.v[i] = *(const u32x4 *)(vb + i * 4 * kHeadDim);
        }
    } else {
        static_assert(BS == 16, "block sizes below 32 other than 16 are not built");
        const int blk = tb / 16;
        const int64_t p0 = trow[blk];
        const int64_t p1 = (tb + 16 < t_end) ? (int64_t)trow[blk + 1] : p0;
        const uint16_t *k0 = kp + p0 * blk_elems + head_off + lane_off;
        const uint16_t *k1 = kp + p1 * blk_elems + head_off + lane_off;
        const uint16_t *v0 = vp + p0 * blk_elems + head_off + lane_off;
        const uint16_t *v1 = vp + p1 * blk_elems + head_off + lane_off;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.k[i] = *(const u32x4 *)((i < 4 ? k0 : k1) + (i & 3) * 4 * kHeadDim);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            t.v[i] = *(const u32x4 *)((i < 4 ? v0 : v1) + (i & 3) * 4 * kHeadDim);
        }
    }
}

template <int DT>
struct RowState {
    float m;       // running max of scaled (log2-domain) scores of this row's tokens
    float l;       // running sum of exp2(score - m)
    float acc[8];  // running sum of exp2(score - m) * v[dims 8c..8c+7]
};

template <int DT, int BS, bool PARTIAL>
__device__ __forceinline__ void compute_tile(RowState<DT> &st, const G1Tile<DT, BS> &t,
                                             const u32x4 &q, int tb, int t_end, int r,
                                             float scale_log2)
{
    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float d = dot2<DT>(q.x, t.k[i].x, 0.f);
        d = dot2<DT>(q.y, t.k[i].y, d);
        d = dot2<DT>(q.z, t.k[i].z, d);
        d = dot2<DT>(q.w, t.k[i].w, d);
        sc[i] = row_sum16(d) * scale_log2;
        if (PARTIAL && tb + 4 * i + r >= t_end)
            sc[i] = kNegInf;
    }
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        mt = fmaxf(mt, sc[i]);
    const float m_new = fmaxf(st.m, mt);
    const float ref = safe_ref(m_new);
    const float alpha = fexp2(st.m - ref);
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        st.acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float p = fexp2(sc[i] - ref);
        u32x4 v = t.v[i];
        if (PARTIAL && tb + 4 * i + r >= t_end) {
            p = 0.f;
            v = (u32x4){0u, 0u, 0u, 0u};
        }
        st.l += p;
        st.acc[0] += p * lo_f32<DT>(v.x);
        st.acc[1] += p * hi_f32<DT>(v.x);
        st.acc[2] += p * lo_f32<DT>(v.y);
        st.acc[3] += p * hi_f32<DT>(v.y);
        st.acc[4] += p * lo_f32<DT>(v.z);
        st.acc[5] += p * hi_f32<DT>(v.z);
        st.acc[6] += p * lo_f32<DT>(v.w);
        st.acc[7] += p * hi_f32<DT>(v.w);
    }
    st.m = m_new;
}

template <int DT, int BS>
__device__ __forceinline__ void compute_any(RowState<DT> &st, const G1Tile<DT, BS> &t,
                                            const u32x4 &q, int tb, int t_end, int r,
                                            float scale_log2)
{
    if (tb + kTile <= t_end)
        compute_tile<DT, BS, false>(st, t, q, tb, t_end, r, scale_log2);
    else
        compute_tile<DT, BS, true>(st, t, q, tb, t_end, r, scale_log2);
}

// Merge the running state of the lane `mask` lanes away into this lane's.
template <int DT>
__device__ __forceinline__ void merge_xor(RowState<DT> &st, int mask)
{
    const float mo = xor_lane(st.m, mask);
    const float lo = xor_lane(st.l, mask);
    const float M = fmaxf(st.m, mo);
    const float ref = safe_ref(M);
    const float a = fexp2(st.m - ref), b = fexp2(mo - ref);
    st.l = st.l * a + lo * b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float ao = xor_lane(st.acc[j], mask);
        st.acc[j] = st.acc[j] * a + ao * b;
    }
    st.m = M;
}

template <int DT, int BS>
__global__ __launch_bounds__(kWaves * 64) void decode_g1_kernel(DecodeArgs a)
{
    __shared__ float s_acc[kWaves][kHeadDim];
    __shared__ float s_m[kWaves], s_l[kWaves];

    const int item = xcd_item(blockIdx.x, a.n_items);
    const int px = item % a.parts_per_item;
    const int rest = item / a.parts_per_item;
    const int s = rest % a.num_seqs;
    const int h = rest / a.num_seqs;  // query head == kv head
    const int n = a.lens[s];

    int t0 = 0, t1 = n;
    if (a.partition_size > 0) {
        t0 = px * a.partition_size;
        if (t0 >= n)
            return;  // partition holds no token: nothing is written
        t1 = min(n, t0 + a.partition_size);
    }

    const int tid = threadIdx.x;
    // wave index, made explicitly uniform so that tile indices and table lookups
    // stay in SGPRs (scalar loads of the table entries)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const int32_t *__restrict__ trow = a.tables + (int64_t)s * a.width;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)h * BS * kHeadDim;
    const int lane_off = r * kHeadDim + c * 8;

    const u32x4 q = *(const u32x4 *)((const uint16_t *)a.q +
                                     ((int64_t)s * a.num_q_heads + h) * kHeadDim + c * 8);

    RowState<DT> st;
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        st.acc[j] = 0.f;

    const int ntiles = (t1 - t0 + kTile - 1) / kTile;
    const int T = ntiles > w ? (ntiles - w + kWaves - 1) / kWaves : 0;  // tiles of this wave
    if (T > 0) {
        G1Tile<DT, BS> A, B;
        int tb = t0 + w * kTile;
        const int step = kWaves * kTile;
        load_tile<DT, BS>(A, kp, vp, trow, tb, t1, head_off, blk_elems, lane_off);
        int j = 0;
        for (; j + 2 < T; j += 2) {
            load_tile<DT, BS>(B, kp, vp, trow, tb + step, t1, head_off, blk_elems, lane_off);
            compute_any<DT, BS>(st, A, q, tb, t1, r, a.scale_log2);
            load_tile<DT, BS>(A, kp, vp, trow, tb + 2 * step, t1, head_off, blk_elems,
                              lane_off);
            compute_any<DT, BS>(st, B, q, tb + step, t1, r, a.scale_log2);
            tb += 2 * step;
        }
        if (j + 1 < T) {
            load_tile<DT, BS>(B, kp, vp, trow, tb + step, t1, head_off, blk_elems, lane_off);
            compute_any<DT, BS>(st, A, q, tb, t1, r, a.scale_log2);
            compute_any<DT, BS>(st, B, q, tb + step, t1, r, a.scale_log2);
        } else {
            compute_any<DT, BS>(st, A, q, tb, t1, r, a.scale_log2);
        }
    }

    // rows of the wave -> one state per wave (identical in every lane)
    merge_xor<DT>(st, 16);
    merge_xor<DT>(st, 32);
    if (r == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            s_acc[w][c * 8 + j] = st.acc[j];
    }
    if (lane == 0) {
        s_m[w] = st.m;
        s_l[w] = st.l;
    }
    __syncthreads();

    if (tid < kHeadDim) {
        const int d = tid;
        float M = s_m[0];
#pragma unroll
        for (int i = 1; i < kWaves; ++i)
            M = fmaxf(M, s_m[i]);
        const float ref = safe_ref(M);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            const float wgt = fexp2(s_m[i] - ref);
            L += s_l[i] * wgt;
            O += s_acc[i][d] * wgt;
        }
        const int64_t row = (int64_t)s * a.num_q_heads + h;
        if (a.partition_size == 0) {
            const float o = L > 0.f ? O / L : 0.f;
            ((uint16_t *)a.out)[row * kHeadDim + d] = to_bits<DT>(o);
        } else {
            a.part_o[(row * a.max_partitions + px) * kHeadDim + d] = O / L;
            if (d == 0)
                a.part_lse[row * a.max_partitions + px] = (ref + flog2(L)) * kLn2;
        }
    }
}

}  // namespace

template <int DT, int BS>
static hipError_t launch_g1_t(const DecodeArgs &a, hipStream_t stream)
{
    hipLaunchKernelGGL((decode_g1_kernel<DT, BS>), dim3(a.n_items), dim3(kWaves * 64), 0, stream,
                       a);
    return hipGetLastError();
}

hipError_t launch_decode_g1(const DecodeArgs &a, int dtype, int block_size, hipStream_t stream)
{
#define PKV_G1_CASE(BSV)                                                                  \
    case BSV:                                                                             \
        return dtype == kFp16 ? launch_g1_t<kFp16, BSV>(a, stream)                       \
                              : launch_g1_t<kBf16, BSV>(a, stream);
    switch (block_size) {
        PKV_G1_CASE(16)
        PKV_G1_CASE(32)
        PKV_G1_CASE(64)
        PKV_G1_CASE(128)
        PKV_G1_CASE(256)
    default:
        return hipErrorInvalidValue;
    }
#undef PKV_G1_CASE
}

}  // namespace pkv
