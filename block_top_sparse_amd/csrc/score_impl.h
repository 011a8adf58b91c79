// score_impl.h -- device helpers of the block scoring: per-lane fp64 dot
// products over 8-channel slices of a summary row, the fixed butterfly that
// folds 16 lanes' partials for 4 blocks, the group query sum, and the
// newest-block summary.  Shared by the scoring kernels and the single-kernel
// decode step; the arithmetic of a block's score is the same in all of
// them, so identical summaries always give bit-identical scores.
#pragma once

#include "kin_internal.h"

namespace kin {

// Load the 8 channels of this lane's slice of summary row `row` (bf16: one
// 16 B load; fp32: two).
template <int DT>
__device__ __forceinline__ void load_row_slice(const void *S, size_t row, int sub, u32x4 &a,
                                               u32x4 &b) {
    if (DT == KIN_BF16) {
        a = ld_nt16(static_cast<const uint16_t *>(S) + row * kHeadDim + 8 * sub);
    } else {
        const float *p = static_cast<const float *>(S) + row * kHeadDim + 8 * sub;
        a = ld_nt16(p);
        b = ld_nt16(p + 4);
    }
}

// fp64 dot product of this lane's 8 channels with the group query sum, in
// channel order.
template <int DT>
__device__ __forceinline__ double slice_dot(const double (&qs)[8], const u32x4 &a,
                                            const u32x4 &b) {
    double acc = 0.0;
    if (DT == KIN_BF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fma(qs[2 * e], (double)bf16_lo(a[e]), acc);
            acc = fma(qs[2 * e + 1], (double)bf16_hi(a[e]), acc);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fma(qs[e], (double)__uint_as_float(a[e]), acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fma(qs[4 + e], (double)__uint_as_float(b[e]), acc);
    }
    return acc;
}

// A 64-bit value moved between lanes by a DPP pattern (both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF,
                                                              false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                              0xF, 0xF, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Fold the per-lane partials of 4 blocks (one per 16-lane row group slot u)
// over the 16 lanes of each row with DPP moves (no LDS traffic):
//   1. partner i^8 (row_ror:8): lanes 0-7 keep blocks 0,1, lanes 8-15 keep 2,3
//   2. partner 7-i inside each 8-lane half (row_half_mirror): one block each
//   3. partners i^1 then i^2 inside each quad (quad_perm)
// Returns the full sum of block u = 2*(lane&8 ? 1:0) + (lane&4 ? 1:0); all
// 4 lanes of a quad hold it.  Every block goes through the same pairing
// tree, so identical summaries give bit-identical scores.
__device__ __forceinline__ double fold4(const double (&part)[4], int lane) {
    const bool hi8 = (lane & 8) != 0, hi4 = (lane & 4) != 0;
    const double r0 = dpp_f64<0x128>(hi8 ? part[0] : part[2]);
    const double r1 = dpp_f64<0x128>(hi8 ? part[1] : part[3]);
    const double w0 = (hi8 ? part[2] : part[0]) + r0;
    const double w1 = (hi8 ? part[3] : part[1]) + r1;
    const double r2 = dpp_f64<0x141>(hi4 ? w0 : w1);
    double x = (hi4 ? w1 : w0) + r2;
    x += dpp_f64<0xB1>(x);  // quad_perm [1,0,3,2]
    x += dpp_f64<0x4E>(x);  // quad_perm [2,3,0,1]
    return x;
}

// (sum over the group's heads of q) for this lane's 8 channels, fp64
template <int DT>
__device__ __forceinline__ void group_query_sum(const void *qv, int b, int g, int hkv, int gqa,
                                                int sub, double (&qs)[8]) {
    const int hq = hkv * gqa;
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[e] = 0.0;
    for (int h = g * gqa; h < (g + 1) * gqa; ++h) {
        const size_t qo = ((size_t)b * hq + h) * kHeadDim + 8 * sub;
        if (DT == KIN_BF16) {
            const u32x4 w = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(qv) + qo);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qs[2 * e] += (double)bf16_lo(w[e]);
                qs[2 * e + 1] += (double)bf16_hi(w[e]);
            }
        } else {
            const float *p = static_cast<const float *>(qv) + qo;
            const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
            const u32x4 c = *reinterpret_cast<const u32x4 *>(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qs[e] += (double)__uint_as_float(a[e]);
                qs[4 + e] += (double)__uint_as_float(c[e]);
            }
        }
    }
}

__device__ __forceinline__ void store_score(double *scores, size_t at, double x) {
    if (x == 0.0) x = 0.0;  // one zero: -0.0 becomes +0.0
    scores[at] = x;
}

// Newest-block summary (one wave, lane = channels 2l, 2l+1): fp64 sum in
// ascending token order, fp64 division, fp64 -> fp32 -> (bf16) rounding.
// Writes the row to S (unless S is null) and, if row_lds is not null, to
// row_lds (the same 256 / 512 B row layout).
template <int DT>
__device__ void newest_summary(const void *K, void *S, size_t pair, int t_cap, int nb_cap,
                               int ctx_len, int block, uint32_t *row_lds, int lane) {
    const int j = (ctx_len - 1) / block;
    const int t0 = j * block;
    const int n = min(block, ctx_len - t0);
    double s0 = 0.0, s1 = 0.0;
    if (DT == KIN_BF16) {
        const uint32_t *k = static_cast<const uint32_t *>(K) +
                            (pair * (size_t)t_cap + (size_t)t0) * (kHeadDim / 2) + lane;
#pragma unroll 16
        for (int t = 0; t < n; ++t) {
            const uint32_t w = k[(size_t)t * (kHeadDim / 2)];
            s0 += (double)bf16_lo(w);
            s1 += (double)bf16_hi(w);
        }
    } else {
        const float2 *k = static_cast<const float2 *>(K) +
                          (pair * (size_t)t_cap + (size_t)t0) * (kHeadDim / 2) + lane;
#pragma unroll 16
        for (int t = 0; t < n; ++t) {
            const float2 v = k[(size_t)t * (kHeadDim / 2)];
            s0 += (double)v.x;
            s1 += (double)v.y;
        }
    }
    const double cnt = (double)n;
    const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
    const size_t o = (pair * (size_t)nb_cap + (size_t)j) * (kHeadDim / 2) + lane;
    if (DT == KIN_BF16) {
        const uint32_t w = f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
        if (S) static_cast<uint32_t *>(S)[o] = w;
        if (row_lds) row_lds[lane] = w;
    } else {
        if (S) static_cast<float2 *>(S)[o] = make_float2(m0, m1);
        if (row_lds) {
            row_lds[2 * lane] = __float_as_uint(m0);
            row_lds[2 * lane + 1] = __float_as_uint(m1);
        }
    }
}

}  // namespace kin
