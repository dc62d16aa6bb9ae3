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
//   * a work-group is 8 wave64s; one work-group per (sequence, head[, partition]);
//   * tokens are processed in tiles of 32; the waves of a work-group take tiles
//     round-robin, with the next tile's K and V loads in flight while the current
//     tile is computed (one register buffer per half, see the loop);
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

// Tokens per tile (tuning knob).  16-token tiles take 75 registers instead of 113
// and fit 3 work-groups per CU instead of 2, but each wave then has half the bytes
// in flight: measured 3.6 % slower on the 7B-shaped batch.
#ifndef PKV_G1_TILE
#define PKV_G1_TILE 32
#endif
constexpr int kTile = PKV_G1_TILE;  // tokens per tile (16 or 32)
static_assert(kTile == 16 || kTile == 32, "tiles of 16 or 32 tokens");
constexpr int kRows = kTile / 4;  // token rows of a tile per lane

// Physical blocks of the two 16-token halves of the tile starting at token tb.
// For BS >= 32 the whole tile sits in block tb/BS.  For BS == 16 the second half
// uses block tb/16+1 only when it holds tokens of the item, else the first block
// again (its rows are then masked), so every K/V address stays inside a block of
// the sequence.  Table indices are clamped to the row so that a lookahead for a
// tile that does not exist reads a valid entry (whose value is then unused).
struct TilePhys {
    int32_t p0, p1;
};

// Raw table entries of the tile at token tb (the second one is only used for
// BS == 16).  Reading them does not depend on the context length, so they can
// be requested before it is known.
template <int BS>
__device__ __forceinline__ TilePhys tile_entries(meta_ptr trow, int width,
                                                 int tb)
{
    TilePhys p;
    if constexpr (BS >= kTile) {
        p.p0 = trow[min(tb / BS, width - 1)];
        p.p1 = p.p0;
    } else {
        static_assert(BS == 16, "block sizes below 32 other than 16 are not built");
        p.p0 = trow[min(tb / 16, width - 1)];
        p.p1 = trow[min(tb / 16 + 1, width - 1)];
    }
    return p;
}

template <int BS>
__device__ __forceinline__ TilePhys tile_select(TilePhys p, int tb, int t_end)
{
    if constexpr (BS < kTile)
        p.p1 = (tb + 16 < t_end) ? p.p1 : p.p0;
    return p;
}

template <int BS>
__device__ __forceinline__ TilePhys tile_phys(meta_ptr trow, int width, int tb,
                                              int t_end)
{
    return tile_select<BS>(tile_entries<BS>(trow, width, tb), tb, t_end);
}

// Buffer resources of the two 16-token halves of a tile in the K and V pools.
// Each covers only the rows that hold tokens of the item, so loads of rows past
// the context length return zeros and fetch nothing from HBM.
struct TileRsrc {
    __amdgpu_buffer_rsrc_t k0, k1, v0, v1;
};

// `t_load` is the end of the rows to fetch: the context end, or one less when the
// last row is the token being appended (it is then taken from the new rows).
template <int BS>
__device__ __forceinline__ TileRsrc tile_rsrc(const TilePhys &p, const uint16_t *kp,
                                              const uint16_t *vp, int tb, int t_load,
                                              int64_t head_off, int64_t blk_elems)
{
    int64_t b0, b1;
    if constexpr (BS >= kTile) {
        b0 = (int64_t)p.p0 * blk_elems + head_off + (int64_t)(tb % BS) * kHeadDim;
        b1 = b0 + 16 * kHeadDim;
    } else {
        b0 = (int64_t)p.p0 * blk_elems + head_off;
        b1 = (int64_t)p.p1 * blk_elems + head_off;
    }
    const int valid = t_load - tb;
    // readfirstlane keeps the ranges in SGPRs (the clamp would otherwise be
    // selected as a VALU med3, making the descriptor look divergent)
    const int n0 = __builtin_amdgcn_readfirstlane(min(max(valid, 0), 16) * kHeadDim * 2);
    const int n1 = kTile > 16
                       ? __builtin_amdgcn_readfirstlane(min(max(valid - 16, 0), 16) * kHeadDim * 2)
                       : 0;
    TileRsrc t;
    t.k0 = make_rsrc(kp + b0, n0);
    t.k1 = make_rsrc(kp + b1, n1);
    t.v0 = make_rsrc(vp + b0, n0);
    t.v1 = make_rsrc(vp + b1, n1);
    return t;
}

// kRows 16-byte loads: rows 4i + lane/16 of the tile, dims 8*(lane%16)..+7.
struct Half {
    u32x4 x[kRows];
};

__device__ __forceinline__ void load_half(Half &h, __amdgpu_buffer_rsrc_t r0,
                                          __amdgpu_buffer_rsrc_t r1, int lane_byte)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        h.x[i] = ldbuf(r0, lane_byte + i * 4 * kHeadDim * 2);
    if constexpr (kRows > 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            h.x[4 + i] = ldbuf(r1, lane_byte + i * 4 * kHeadDim * 2);
    }
}

template <int DT>
struct RowState {
    float m;       // running max of scaled (log2-domain) scores of this row's tokens
    float l;       // running sum of exp2(score - m)
    float acc[8];  // running sum of exp2(score - m) * v[dims 8c..8c+7]
};

// Scores of the row's kRows tokens of a tile (log2 domain); masked tokens get -inf.
template <int DT, bool PARTIAL>
__device__ __forceinline__ void scores(float (&sc)[kRows], const Half &K, const u32x4 &q, int tb,
                                       int t_end, int r, float scale_log2)
{
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        float d = dot2<DT>(q.x, K.x[i].x, 0.f);
        d = dot2<DT>(q.y, K.x[i].y, d);
        d = dot2<DT>(q.z, K.x[i].z, d);
        d = dot2<DT>(q.w, K.x[i].w, d);
        sc[i] = row_sum16(d) * scale_log2;
        if (PARTIAL && tb + 4 * i + r >= t_end)
            sc[i] = kNegInf;
    }
}

// Online-softmax update of the row state with a tile's scores and V rows.
template <int DT, bool PARTIAL>
__device__ __forceinline__ void accumulate(RowState<DT> &st, const float (&sc)[kRows],
                                           const Half &V, int tb, int t_end, int r)
{
    float mt = sc[0];
#pragma unroll
    for (int i = 1; i < kRows; ++i)
        mt = fmaxf(mt, sc[i]);
    const float m_new = fmaxf(st.m, mt);
    const float ref = safe_ref(m_new);
    const float alpha = fexp2(st.m - ref);
    st.l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        st.acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
        float p = fexp2(sc[i] - ref);
        u32x4 v = V.x[i];
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

// Swap helpers for the row merges: both values of the lane pair (l, l^16) or
// (l, l^32), the even-row / lower-half lane's first (gfx950 lane-swap
// instructions; lane layout checked on the GPU with an in-bounds probe).
template <int SPAN>
__device__ __forceinline__ void swap_pair(float x, float &lo, float &hi)
{
    const unsigned u = __float_as_uint(x);
    const auto t = SPAN == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                              : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    lo = __uint_as_float(t[0]);
    hi = __uint_as_float(t[1]);
}

// Merge the running states of lanes l and l^SPAN; both lanes end with the same
// state (the lower lane's terms first, as a shuffle-based merge computes it in
// the lanes that write the result).
template <int DT, int SPAN>
__device__ __forceinline__ void merge_pair(RowState<DT> &st)
{
    float m0, m1, l0, l1;
    swap_pair<SPAN>(st.m, m0, m1);
    swap_pair<SPAN>(st.l, l0, l1);
    const float M = fmaxf(m0, m1);
    const float ref = safe_ref(M);
    const float a = fexp2(m0 - ref), b = fexp2(m1 - ref);
    st.l = l0 * a + l1 * b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float x0, x1;
        swap_pair<SPAN>(st.acc[j], x0, x1);
        st.acc[j] = x0 * a + x1 * b;
    }
    st.m = M;
}

// SPLIT: split-context mode (partition loop); otherwise one pass over the
// whole context, with the loop folded away at compile time.  MERGE (with SPLIT):
// the last work-group of an item to finish merges the item's partials into `out`,
// and a context of one partition is written to `out` directly.
// The register budget is capped so that 4 waves fit on each SIMD (the
// split variant would otherwise be allocated past that occupancy).
#ifndef PKV_G1_OCCUPANCY
#define PKV_G1_OCCUPANCY 4  // waves per SIMD the register budget is capped for
#endif
template <int DT, int BS, int WAVES, bool SPLIT, bool MERGE = false>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(PKV_G1_OCCUPANCY)))
void decode_g1_kernel(DecodeArgs a)
{
    static_assert(SPLIT || !MERGE, "the merged mode is a split mode");
    __shared__ float s_acc[WAVES][kHeadDim];
    __shared__ float s_m[WAVES], s_l[WAVES];
    __shared__ int32_t s_last;

    // Work items are ordered sequence-major: the KV heads of one sequence are
    // neighbours in dispatch order, so the concurrently running work-groups read
    // all heads of the same blocks (whole contiguous slabs of the pool) rather
    // than one head's slice of many blocks.  Measured faster on MI355X than the
    // KV-head-major order.
    const int item = blockIdx.x;
    const int parts = SPLIT ? a.parts_per_item : 1;
    const int px0 = item % parts;
    const int rest = item / parts;
    const int h = rest % a.num_kv_heads;  // query head == kv head
    const int s = ordered_seq(a, rest / a.num_kv_heads);

    const int tid = threadIdx.x;
    // wave index, made explicitly uniform so that tile indices and table lookups
    // stay in SGPRs (scalar loads of the table entries)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int r = lane >> 4, c = lane & 15;

    const uint16_t *__restrict__ kp = (const uint16_t *)a.k_pool;
    const uint16_t *__restrict__ vp = (const uint16_t *)a.v_pool;
    const meta_ptr trow = as_meta(a.tables) + (int64_t)s * a.width;
    const int64_t blk_elems = (int64_t)a.num_kv_heads * BS * kHeadDim;
    const int64_t head_off = (int64_t)h * BS * kHeadDim;
    const int lane_byte = (r * kHeadDim + c * 8) * 2;
    const int P = SPLIT ? a.partition_size : 0;

    // The first tile's table entries (and the next tile's) do not depend on the
    // context length: request them together with it, so the two scalar-load
    // latencies overlap instead of chaining.
    const int tb_first = (P > 0 ? px0 * P : 0) + w * kTile;
    const TilePhys e_first = tile_entries<BS>(trow, a.width, tb_first);
    const TilePhys e_next = tile_entries<BS>(trow, a.width, tb_first + WAVES * kTile);
    const int n = as_meta(a.lens)[s];
    const bool fused = a.k_new != nullptr;
    if (fused && n <= 0 && px0 == 0 && h == 0 && tid == 0 && a.slot_out)
        a.slot_out[s] = -1;  // padding sequence: nothing appended

    const u32x4 q = *(const u32x4 *)((const uint16_t *)a.q +
                                     ((int64_t)s * a.num_q_heads + h) * kHeadDim + c * 8);

    // Partitions px0, px0 + parts_per_item, ... of the item belong to this
    // work-group (the grid is sized from the batch, not from the table width, so
    // short sequences do not launch empty work-groups).  Single pass: px0 = 0,
    // one iteration over the whole context (which also writes zeros when n = 0).
    const int np = SPLIT ? (n + P - 1) / P : 1;
    const bool direct = MERGE && np <= 1;
    const int np_loop = direct ? (px0 == 0 ? 1 : 0) : np;
    for (int px = px0; px < np_loop; px += parts) {
        if (px != px0)
            __syncthreads();  // the previous partition's merge is done with LDS
        const int t0 = P > 0 ? px * P : 0;
        const int t1 = P > 0 ? min(n, t0 + P) : n;
        // With a fused append, position n-1 (in the item's last tile) is not read
        // from the pool: it holds stale data until this kernel writes the new row.
        const bool owns_new = fused && t1 == n;
        const int t_load = owns_new ? n - 1 : t1;
        const int ntiles = (t1 - t0 + kTile - 1) / kTile;
        // the wave holding position n-1 (the item's last tile) fetches the new
        // rows and their block id up front, so that the latency overlaps its loop
        const bool new_here = owns_new && ntiles > 0 && w == (ntiles - 1) % WAVES;
        u32x4 kn = {0u, 0u, 0u, 0u}, vn = {0u, 0u, 0u, 0u};
        const int64_t phys_n = new_here ? (int64_t)trow[(n - 1) / BS] : 0;  // block of n-1
        if (new_here) {
            const int64_t off = ((int64_t)s * a.num_kv_heads + h) * kHeadDim + c * 8;
            kn = *(const u32x4 *)((const uint16_t *)a.k_new + off);
            vn = *(const u32x4 *)((const uint16_t *)a.v_new + off);
        }

        RowState<DT> st;
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            st.acc[j] = 0.f;

        // Tiles w, w+WAVES, ... of the partition belong to this wave.  The K and V
        // halves are pipelined separately: the next tile's K loads are issued as
        // soon as the current scores are computed, its V loads as soon as the
        // current V rows are consumed, so one tile stays in flight with a single
        // register buffer per half.
        const int T = ntiles > w ? (ntiles - w + WAVES - 1) / WAVES : 0;
        if (T > 0) {
            const int step = WAVES * kTile;
            int tb = t0 + w * kTile;
            const bool first = px == px0;
            Half K, V;
            {
                const TilePhys ef = first ? e_first : tile_entries<BS>(trow, a.width, tb);
                const TileRsrc rs = tile_rsrc<BS>(tile_select<BS>(ef, tb, t1), kp, vp, tb,
                                                  t_load, head_off, blk_elems);
                load_half(K, rs.k0, rs.k1, lane_byte);
                load_half(V, rs.v0, rs.v1, lane_byte);
            }
            if (new_here) {
                // write the new rows to their slot now: stores share the in-order
                // vmcnt counter with loads, so issuing them here lets their latency
                // overlap the loop instead of the end of the work-group
                const int tn = n - 1;
                const int64_t dst =
                    phys_n * blk_elems + head_off + (int64_t)(tn % BS) * kHeadDim + c * 8;
                if (r == 0)
                    *(u32x4 *)((uint16_t *)a.k_pool + dst) = kn;
                else if (r == 1)
                    *(u32x4 *)((uint16_t *)a.v_pool + dst) = vn;
                if (h == 0 && lane == 0 && a.slot_out)
                    a.slot_out[s] = phys_n * BS + tn % BS;
            }
            // table entries are looked up one tile ahead of the loads that use them
            const TilePhys en = first ? e_next : tile_entries<BS>(trow, a.width, tb + step);
            TilePhys pn = tile_select<BS>(en, tb + step, t1);
            float sc[kRows];
            for (int j = 0; j + 1 < T; ++j) {  // every tile here is full
                const TilePhys pn2 = tile_phys<BS>(trow, a.width, tb + 2 * step, t1);
                const TileRsrc rn =
                    tile_rsrc<BS>(pn, kp, vp, tb + step, t_load, head_off, blk_elems);
                scores<DT, false>(sc, K, q, tb, t1, r, a.scale_log2);
                // keep the scheduler from sinking the prefetches below the math they
                // are meant to overlap
                __builtin_amdgcn_sched_barrier(0);
                load_half(K, rn.k0, rn.k1, lane_byte);
                __builtin_amdgcn_sched_barrier(0);
                accumulate<DT, false>(st, sc, V, tb, t1, r);
                __builtin_amdgcn_sched_barrier(0);
                load_half(V, rn.v0, rn.v1, lane_byte);
                __builtin_amdgcn_sched_barrier(0);
                pn = pn2;
                tb += step;
            }
            if (new_here && tb + kTile >= n) {
                // this tile holds position n-1: put the new rows in place of the
                // (unfetched) pool row
                const int row = n - 1 - tb;  // 0 .. kTile-1
#pragma unroll
                for (int i = 0; i < kRows; ++i) {
                    if (row == 4 * i + r) {
                        K.x[i] = kn;
                        V.x[i] = vn;
                    }
                }
            }
            if (tb + kTile <= t1) {
                scores<DT, false>(sc, K, q, tb, t1, r, a.scale_log2);
                accumulate<DT, false>(st, sc, V, tb, t1, r);
            } else {
                scores<DT, true>(sc, K, q, tb, t1, r, a.scale_log2);
                accumulate<DT, true>(st, sc, V, tb, t1, r);
            }
        }

        // rows of the wave -> one state per wave (identical in every lane)
        merge_pair<DT, 16>(st);
        merge_pair<DT, 32>(st);
        const int64_t row = (int64_t)s * a.num_q_heads + h;
        if (WAVES == 1) {
            if (r == 0) {
                const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
                if (P == 0 || direct) {
                    u32x4 o;
                    o.x = (uint32_t)to_bits<DT>(st.acc[0] * inv) |
                          ((uint32_t)to_bits<DT>(st.acc[1] * inv) << 16);
                    o.y = (uint32_t)to_bits<DT>(st.acc[2] * inv) |
                          ((uint32_t)to_bits<DT>(st.acc[3] * inv) << 16);
                    o.z = (uint32_t)to_bits<DT>(st.acc[4] * inv) |
                          ((uint32_t)to_bits<DT>(st.acc[5] * inv) << 16);
                    o.w = (uint32_t)to_bits<DT>(st.acc[6] * inv) |
                          ((uint32_t)to_bits<DT>(st.acc[7] * inv) << 16);
                    *(u32x4 *)((uint16_t *)a.out + row * kHeadDim + c * 8) = o;
                } else {
                    float *po = a.part_o + (row * a.max_partitions + px) * kHeadDim + c * 8;
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        po[j] = st.acc[j] * inv;
                    if (c == 0)
                        a.part_lse[row * a.max_partitions + px] =
                            (safe_ref(st.m) + flog2(st.l)) * kLn2;
                }
            }
            continue;
        }
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
            for (int i = 1; i < WAVES; ++i)
                M = fmaxf(M, s_m[i]);
            const float ref = safe_ref(M);
            float L = 0.f, O = 0.f;
#pragma unroll
            for (int i = 0; i < WAVES; ++i) {
                const float wgt = fexp2(s_m[i] - ref);
                L += s_l[i] * wgt;
                O += s_acc[i][d] * wgt;
            }
            if (P == 0 || direct) {
                const float o = L > 0.f ? O / L : 0.f;
                ((uint16_t *)a.out)[row * kHeadDim + d] = to_bits<DT>(o);
            } else {
                float *po = a.part_o + (row * a.max_partitions + px) * kHeadDim + d;
                float *pl = a.part_lse + row * a.max_partitions + px;
                const float lse = (ref + flog2(L)) * kLn2;
                if constexpr (MERGE) {
                    // read by another work-group of the item (see arrive_last)
                    const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
                    st_ws1(ws.o, (int)(po - a.part_o) * 4, O / L);
                    if (d == 0)
                        st_ws1(ws.lse, (int)(pl - a.part_lse) * 4, lse);
                } else {
                    *po = O / L;
                    if (d == 0)
                        *pl = lse;
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
        if (tid < kHeadDim / 4) {
            const int64_t row = (int64_t)s * a.num_q_heads + h;
            const int d0 = tid * 4;
            const Workspace ws = workspace_rsrc(a, (int64_t)a.num_seqs * a.num_q_heads);
            const f32x4 o = merge_partials4(ws, (int)(row * a.max_partitions) * 4,
                                            (int)(row * a.max_partitions * kHeadDim + d0) * 4, np);
            u32x2 packed;
            packed.x = (uint32_t)to_bits<DT>(o[0]) | ((uint32_t)to_bits<DT>(o[1]) << 16);
            packed.y = (uint32_t)to_bits<DT>(o[2]) | ((uint32_t)to_bits<DT>(o[3]) << 16);
            *(u32x2 *)((uint16_t *)a.out + row * kHeadDim + d0) = packed;
        }
    }
}

}  // namespace

// Waves per work-group (tuning knob; 8 measured best for the 7B-shaped batch).
#ifndef PKV_G1_WAVES
#define PKV_G1_WAVES 8
#endif

template <int DT, int BS>
static hipError_t launch_g1_t(const DecodeArgs &a, hipStream_t stream)
{
    constexpr int W = PKV_G1_WAVES;
    if (a.partition_size > 0 && a.counters)
        hipLaunchKernelGGL((decode_g1_kernel<DT, BS, W, true, true>), dim3(a.n_items),
                           dim3(W * 64), 0, stream, a);
    else if (a.partition_size > 0)
        hipLaunchKernelGGL((decode_g1_kernel<DT, BS, W, true>), dim3(a.n_items), dim3(W * 64), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_g1_kernel<DT, BS, W, false>), dim3(a.n_items), dim3(W * 64), 0,
                           stream, a);
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
