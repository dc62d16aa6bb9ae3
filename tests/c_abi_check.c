/*
 * c_abi_check.c -- drives libpagedkv through include/paged_kv.h alone: plain C,
 * device memory from the HIP runtime, no Python and no torch.  Built next to the
 * library by the package's build step; run by tests/test_gpu_c_abi.py.
 *
 * Checks, each against a result that needs no reference implementation:
 *   1. a context of one token: softmax over one score is exactly 1, so the output
 *      of every query head equals the value row just appended (bit for bit), and
 *      that row sits in the pool at (block table[0], offset 0);
 *   2. scale 0: every score is 0, so the output is the plain mean of the n value
 *      rows of the sequence (walked through its block table), within 1e-2;
 *   3. the same one-token case through slotted segments: each sequence's one
 *      segment (block, offset, length 1) is the slot the fused append writes,
 *      and the output equals that value row, bit for bit;
 *   4. argument errors come back as status codes without touching the device.
 * Prints one line per check and exits 0 when all pass.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "paged_kv.h"

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);  \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

enum { S = 4, HQ = 8, HKV = 2, D = 128, B = 16, W = 8, NB = 64 };

static uint64_t rng = 88172645463325252ull;
static uint32_t next_u32(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (uint32_t)(rng >> 32);
}

/* A finite binary16 value in +-[0.5, 2): random sign and mantissa, exponent 14 or 15. */
static uint16_t rand_half(void)
{
    const uint32_t r = next_u32();
    return (uint16_t)(((r & 1u) << 15) | ((14u + ((r >> 1) & 1u)) << 10) | ((r >> 2) & 0x3FFu));
}

static double half_to_double(uint16_t h)
{
    const int sign = h >> 15, exp = (h >> 10) & 0x1F, man = h & 0x3FF;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp(1.0 + man / 1024.0, exp - 15);
    return sign ? -v : v;
}

static void *dev_copy(const void *host, size_t bytes)
{
    void *d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes));
    CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

int main(void)
{
    const size_t pool_elems = (size_t)NB * HKV * B * D;
    uint16_t *k_pool_h = malloc(pool_elems * 2), *v_pool_h = malloc(pool_elems * 2);
    uint16_t q_h[S * HQ * D], kn_h[S * HKV * D], vn_h[S * HKV * D], out_h[S * HQ * D];
    int32_t tables_h[S * W], lens_h[S];
    int failures = 0;
    for (size_t i = 0; i < pool_elems; ++i) {
        k_pool_h[i] = rand_half();
        v_pool_h[i] = rand_half();
    }
    for (int i = 0; i < S * HQ * D; ++i)
        q_h[i] = rand_half();
    for (int i = 0; i < S * HKV * D; ++i) {
        kn_h[i] = rand_half();
        vn_h[i] = rand_half();
    }
    /* sequence s owns blocks 9s+3, 9s+4, ... (distinct, scattered through the pool) */
    for (int s = 0; s < S; ++s)
        for (int b = 0; b < W; ++b)
            tables_h[s * W + b] = (9 * s + 3 + 5 * b) % NB;

    void *k_pool = dev_copy(k_pool_h, pool_elems * 2), *v_pool = dev_copy(v_pool_h, pool_elems * 2);
    void *q = dev_copy(q_h, sizeof q_h), *kn = dev_copy(kn_h, sizeof kn_h),
         *vn = dev_copy(vn_h, sizeof vn_h);
    void *tables = dev_copy(tables_h, sizeof tables_h);
    void *out = NULL, *lens = NULL;
    CHECK_HIP(hipMalloc(&out, sizeof out_h));
    CHECK_HIP(hipMalloc(&lens, sizeof lens_h));
    const int G = HQ / HKV;

    /* 1. one-token contexts: output = appended value row, exactly */
    for (int s = 0; s < S; ++s)
        lens_h[s] = 1;
    CHECK_HIP(hipMemcpy(lens, lens_h, sizeof lens_h, hipMemcpyHostToDevice));
    int rc = paged_attention_append_decode(out, q, k_pool, v_pool, kn, vn, NULL, tables, lens, S,
                                           HQ, HKV, D, B, W, NB, 1.0f / sqrtf((float)D), 0, 0,
                                           NULL, NULL, PKV_FP16, NULL);
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out_h, out, sizeof out_h, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(v_pool_h, v_pool, pool_elems * 2, hipMemcpyDeviceToHost));
    int bad = rc != PKV_OK;
    for (int s = 0; s < S; ++s)
        for (int h = 0; h < HQ; ++h) {
            const uint16_t *vrow = vn_h + (s * HKV + h / G) * D;
            if (memcmp(out_h + (s * HQ + h) * D, vrow, D * 2) != 0)
                bad = 1;
        }
    for (int s = 0; s < S; ++s)
        for (int g = 0; g < HKV; ++g) {
            const size_t slot = (((size_t)tables_h[s * W] * HKV + g) * B + 0) * D;
            if (memcmp(v_pool_h + slot, vn_h + (s * HKV + g) * D, D * 2) != 0)
                bad = 1;
        }
    printf("one-token contexts: output equals the appended value row: %s\n", bad ? "FAIL" : "ok");
    failures += bad;

    /* 2. scale 0 over n tokens of history: output = mean of the sequence's value rows */
    const int n_h[S] = {1, 17, 40, 128};
    for (int s = 0; s < S; ++s)
        lens_h[s] = n_h[s];
    CHECK_HIP(hipMemcpy(lens, lens_h, sizeof lens_h, hipMemcpyHostToDevice));
    rc = paged_attention_decode(out, q, k_pool, v_pool, tables, lens, S, HQ, HKV, D, B, W, NB,
                                0.0f, 0, 0, NULL, NULL, PKV_FP16, NULL);
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(out_h, out, sizeof out_h, hipMemcpyDeviceToHost));
    bad = rc != PKV_OK;
    double max_err = 0.0;
    for (int s = 0; s < S; ++s)
        for (int h = 0; h < HQ; ++h)
            for (int d = 0; d < D; ++d) {
                double mean = 0.0;
                for (int t = 0; t < n_h[s]; ++t) {
                    const int phys = tables_h[s * W + t / B];
                    mean += half_to_double(
                        v_pool_h[(((size_t)phys * HKV + h / G) * B + t % B) * D + d]);
                }
                mean /= n_h[s];
                const double got = half_to_double(out_h[(s * HQ + h) * D + d]);
                const double err = fabs(got - mean);
                if (err > max_err)
                    max_err = err;
                if (!(err <= 1e-2 + 1e-2 * fabs(mean)))
                    bad = 1;
            }
    printf("scale 0: output equals the mean of the value rows (max abs err %.2e): %s\n", max_err,
           bad ? "FAIL" : "ok");
    failures += bad;

    /* 3. one-token slotted segments, fused append: output = appended value row */
    {
        int32_t segs_h[S * 3], nsegs_h[S];
        int64_t slots_h[S];
        for (int s = 0; s < S; ++s) {
            segs_h[3 * s] = (7 * s + 1) % NB; /* block */
            segs_h[3 * s + 1] = 2 * s + 1;    /* slot offset */
            segs_h[3 * s + 2] = 1;            /* length: the new token */
            nsegs_h[s] = 1;
        }
        void *segs = dev_copy(segs_h, sizeof segs_h), *nsegs = dev_copy(nsegs_h, sizeof nsegs_h);
        void *slots = NULL;
        CHECK_HIP(hipMalloc(&slots, sizeof slots_h));
        rc = paged_attention_append_decode_slotted(out, q, k_pool, v_pool, kn, vn, slots, segs,
                                                   nsegs, S, HQ, HKV, D, B, 1, NB,
                                                   PKV_DEFAULT_SCALE, PKV_FP16, NULL);
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(out_h, out, sizeof out_h, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(v_pool_h, v_pool, pool_elems * 2, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(slots_h, slots, sizeof slots_h, hipMemcpyDeviceToHost));
        bad = rc != PKV_OK;
        for (int s = 0; s < S; ++s) {
            if (slots_h[s] != (int64_t)segs_h[3 * s] * B + segs_h[3 * s + 1])
                bad = 1;
            for (int h = 0; h < HQ; ++h)
                if (memcmp(out_h + (s * HQ + h) * D, vn_h + (s * HKV + h / G) * D, D * 2) != 0)
                    bad = 1;
            for (int g = 0; g < HKV; ++g) {
                const size_t at = (((size_t)segs_h[3 * s] * HKV + g) * B + segs_h[3 * s + 1]) * D;
                if (memcmp(v_pool_h + at, vn_h + (s * HKV + g) * D, D * 2) != 0)
                    bad = 1;
            }
        }
        printf("one-token slotted segments: the row lands at the segment's slot and is the "
               "output: %s\n", bad ? "FAIL" : "ok");
        failures += bad;
        hipFree(segs);
        hipFree(nsegs);
        hipFree(slots);
    }

    /* 4. argument errors */
    bad = 0;
    if (paged_attention_decode(out, NULL, k_pool, v_pool, tables, lens, S, HQ, HKV, D, B, W, NB,
                               1.0f, 0, 0, NULL, NULL, PKV_FP16, NULL) != PKV_EINVAL)
        bad = 1;
    if (paged_attention_decode(out, q, k_pool, v_pool, tables, lens, S, HQ, HKV, 64, B, W, NB,
                               1.0f, 0, 0, NULL, NULL, PKV_FP16, NULL) != PKV_ENOTSUP)
        bad = 1;
    if (paged_attention_decode(out, q, k_pool, v_pool, tables, lens, S, HQ, HKV, D, B, W, NB,
                               1.0f, 64, 0, NULL, NULL, PKV_FP16, NULL) != PKV_EWORKSPACE)
        bad = 1;
    printf("argument errors: %s (%s)\n", bad ? "FAIL" : "ok", pkv_status_string(PKV_EWORKSPACE));
    failures += bad;

    hipFree(k_pool);
    hipFree(v_pool);
    hipFree(q);
    hipFree(kn);
    hipFree(vn);
    hipFree(tables);
    hipFree(out);
    hipFree(lens);
    free(k_pool_h);
    free(v_pool_h);
    return failures ? 1 : 0;
}
