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

template <int DT>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a)
{
    const int wave = (blockIdx.x * 256 + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (wave >= a.num_seqs * a.num_q_heads)
        return;
    const int s = wave / a.num_q_heads;
    const int n = a.lens[s];
    const int np = n > 0 ? (n + a.partition_size - 1) / a.partition_size : 0;
    const int64_t row = wave;
    const float *lse = a.part_lse + row * a.max_partitions;
    const float *po = a.part_o + row * a.max_partitions * kHeadDim + 2 * lane;

    float M = kNegInf;
    for (int p = 0; p < np; ++p)
        M = fmaxf(M, lse[p]);
    const float ref = safe_ref(M);
    float W = 0.f, o0 = 0.f, o1 = 0.f;
    for (int p = 0; p < np; ++p) {
        const float wgt = fexp2((lse[p] - ref) * kLog2e);
        const float2 v = *(const float2 *)(po + (int64_t)p * kHeadDim);
        W += wgt;
        o0 += wgt * v.x;
        o1 += wgt * v.y;
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
