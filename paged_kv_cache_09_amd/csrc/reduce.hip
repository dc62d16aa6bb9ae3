// reduce.hip -- log-sum-exp merge of split-context partitions.
//
// Split-context decoding gives long sequences more parallelism than one work-group
// per (sequence, head): each partition of P tokens produces its normalised
// attention output o_p and the log-sum-exp lse_p of its scaled scores.  The exact
// result over the whole context is the lse-weighted mean
//     out = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M),  M = max_p lse_p.
// The pages describe no partitioning; this is the algebraic identity that makes
// the split exact.  One wave64 per (sequence, query head); each lane owns two of
// the 128 dims, so reads of a partition row are one coalesced 512-byte access.
#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

struct ReduceArgs {
    void *out;
    const float *part_o;
    const float *part_lse;
    const int32_t *lens;
    int num_seqs, num_q_heads, partition_size, max_partitions;
};

// Max over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1)
        x = fmaxf(x, xor_lane(x, m));
    return x;
}

// Partitions whose rows are requested before the context length is known.
constexpr int kEarly = 8;

template <int DT>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a)
{
    // the wave index is uniform: the length and the partition count come from
    // scalar loads, and every loop below is wave-uniform
    const int wave = __builtin_amdgcn_readfirstlane((blockIdx.x * 256 + threadIdx.x) >> 6);
    const int lane = threadIdx.x & 63;
    if (wave >= a.num_seqs * a.num_q_heads)
        return;
    const int s = wave / a.num_q_heads;
    const int64_t row = wave;
    const int MP = a.max_partitions;
    const float *lse = a.part_lse + row * MP;
    const float *po = a.part_o + row * MP * kHeadDim + 2 * lane;

    // The loads of the first 64 lse values and of the first kEarly partition rows
    // do not depend on the context length: they are issued together with its load,
    // so the three latencies overlap instead of chaining.  Entries of partitions
    // the decode did not write (p >= np) are read but never used: every use below
    // is guarded by p < np, a wave-uniform condition, so their contents (arbitrary
    // bits, possibly NaN) cannot reach the result.
    const float lse0 = lane < MP ? lse[lane] : kNegInf;
    float2 early[kEarly];
#pragma unroll
    for (int i = 0; i < kEarly; ++i)
        if (i < MP)
            early[i] = *(const float2 *)(po + (int64_t)i * kHeadDim);
    const int n = as_meta(a.lens)[s];
    // a length needing more partitions than the workspace holds is a caller error;
    // only the partitions the workspace holds are read
    const int np = n > 0 ? min((n + a.partition_size - 1) / a.partition_size, MP) : 0;

    // partition p's lse is read by lane p % 64 (one load for up to 64 partitions)
    float M = lane < np ? lse0 : kNegInf;
    for (int p0 = 64; p0 < np; p0 += 64) {
        const int p = p0 + lane;
        M = fmaxf(M, p < np ? lse[p] : kNegInf);
    }
    M = wave_max(M);
    const float ref = safe_ref(M);
    float W = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p0 = 0; p0 < np; p0 += 64) {
        const int p = p0 + lane;
        const float lp = p0 == 0 ? lse0 : (p < np ? lse[p] : kNegInf);
        const float wl = p < np ? fexp2((lp - ref) * kLog2e) : 0.f;
        const int cnt = min(64, np - p0);
        int i = 0;
        if (p0 == 0) {
            // the rows requested up front
#pragma unroll
            for (int u = 0; u < kEarly; ++u) {
                if (u < cnt) {
                    const float wgt =
                        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), u));
                    W += wgt;
                    o0 += wgt * early[u].x;
                    o1 += wgt * early[u].y;
                }
            }
            i = min(cnt, kEarly);
        }
        // the remaining partition rows are independent loads: four are in flight
        // together
        for (; i + 4 <= cnt; i += 4) {
            float2 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = *(const float2 *)(po + (int64_t)(p0 + i + u) * kHeadDim);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float wgt =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i + u));
                W += wgt;
                o0 += wgt * v[u].x;
                o1 += wgt * v[u].y;
            }
        }
        for (; i < cnt; ++i) {
            const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), i));
            const float2 v = *(const float2 *)(po + (int64_t)(p0 + i) * kHeadDim);
            W += wgt;
            o0 += wgt * v.x;
            o1 += wgt * v.y;
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    const uint32_t packed = (uint32_t)to_bits<DT>(o0 * inv) | ((uint32_t)to_bits<DT>(o1 * inv) << 16);
    ((uint32_t *)a.out)[row * (kHeadDim / 2) + lane] = packed;
}

}  // namespace

hipError_t launch_reduce(void *out, const float *part_o, const float *part_lse,
                         const int32_t *lens, int num_seqs, int num_q_heads, int partition_size,
                         int max_partitions, int dtype, hipStream_t stream)
{
    ReduceArgs a{out, part_o, part_lse, lens, num_seqs, num_q_heads, partition_size,
                 max_partitions};
    const int64_t waves = (int64_t)num_seqs * num_q_heads;
    const dim3 grid((unsigned)((waves + 3) / 4));
    if (dtype == kFp16)
        hipLaunchKernelGGL(reduce_kernel<kFp16>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(reduce_kernel<kBf16>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace pkv
