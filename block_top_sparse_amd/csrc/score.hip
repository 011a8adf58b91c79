// score.hip -- K2: block scores.
//
// The group score of block j for (sequence b, KV head g) is
//     sigma_j = sum_{h : h / gqa == g} q_h . s_j = (sum_h q_h) . s_j
// (the page's "mean score per block" of BlockTopKAttention, skill summary
// "Kinetics: Memory-Aware Test-Time Scaling", Implementation, summed over
// the query heads that share the KV head).  The scale 1/sqrt(d) is left out:
// it does not change the order.  Arithmetic is fp64, so rounding cannot
// reorder two blocks whose scores differ by more than ~1e-15 relative.
//
// This kernel streams every summary row once, which is the part of a
// sparse step that still grows with the context length, so it is written
// as a pure HBM stream:
//   - 16 lanes own one block row, 8 channels (16 B of bf16 / 32 B of fp32)
//     per lane, so one wave load covers 4 whole consecutive rows (1 KiB of
//     bf16) and a wave keeps TPW x 4 such loads in flight;
//   - each lane forms its 8-term fp64 partial in a fixed order, and the 16
//     partials of 4 blocks are folded with a reduce-scatter butterfly
//     (xor 8, 4, 2, 1).  The summation tree is the same for every block, so
//     two blocks with identical summaries get bit-identical scores and a tie
//     between them is decided by index alone.
#include "kin_internal.h"

namespace kin {

template <int DT, int TPW>
__global__ __launch_bounds__(256) void k_block_score(const void *__restrict__ qv,
                                                     const void *__restrict__ Sv,
                                                     double *__restrict__ scores, int hkv,
                                                     int gqa, int nb_cap, int nb) {
    constexpr int kBlocksPerWave = 16 * TPW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane & 15;  // channel slice: channels 8*sub .. 8*sub+7
    const int grp = lane >> 4;  // which of the 4 rows of a wave load
    const int pair = blockIdx.y;
    const int b = pair / hkv, g = pair % hkv;
    const int hq = hkv * gqa;

    // (sum over the group's heads of q) for this lane's 8 channels, fp64
    double qs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[e] = 0.0;
    for (int h = g * gqa; h < (g + 1) * gqa; ++h) {
        const size_t qo = ((size_t)b * hq + h) * kHeadDim + 8 * sub;
        if (DT == KIN_BF16) {
            const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(qv) + qo);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qs[2 * e] += (double)bf16_lo(ww[e]);
                qs[2 * e + 1] += (double)bf16_hi(ww[e]);
            }
        } else {
            const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(qv) + qo);
            const float4 a = p[0], c = p[1];
            const float f[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) qs[e] += (double)f[e];
        }
    }

    const int wave_j0 = (blockIdx.x * 4 + wave) * kBlocksPerWave;
    if (wave_j0 >= nb) return;
    const size_t row0 = (size_t)pair * nb_cap;

#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        const int tile_j0 = wave_j0 + 16 * t;
        double part[4];
        // all 4 row loads of the tile are issued before any arithmetic
        if (DT == KIN_BF16) {
            u32x4 w[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = min(tile_j0 + 4 * u + grp, nb - 1);
                w[u] = ld_stream16(static_cast<const uint16_t *>(Sv) + (row0 + j) * kHeadDim +
                                   8 * sub);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t ww[4] = {w[u][0], w[u][1], w[u][2], w[u][3]};
                double acc = 0.0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc = fma(qs[2 * e], (double)bf16_lo(ww[e]), acc);
                    acc = fma(qs[2 * e + 1], (double)bf16_hi(ww[e]), acc);
                }
                part[u] = acc;
            }
        } else {
            u32x4 w[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = min(tile_j0 + 4 * u + grp, nb - 1);
                const float *p = static_cast<const float *>(Sv) + (row0 + j) * kHeadDim + 8 * sub;
                w[u][0] = ld_stream16(p);
                w[u][1] = ld_stream16(p + 4);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float f[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    f[e] = __uint_as_float(w[u][0][e]);
                    f[4 + e] = __uint_as_float(w[u][1][e]);
                }
                double acc = 0.0;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fma(qs[e], (double)f[e], acc);
                part[u] = acc;
            }
        }
        // reduce-scatter over the 16 lanes of a row: after xor 8 each lane
        // keeps 2 of the 4 blocks, after xor 4 one; xor 2 and xor 1 finish.
        const bool hi8 = (lane & 8) != 0, hi4 = (lane & 4) != 0;
        const double send0 = hi8 ? part[0] : part[2];
        const double send1 = hi8 ? part[1] : part[3];
        const double r0 = __shfl_xor(send0, 8);
        const double r1 = __shfl_xor(send1, 8);
        const double w0 = (hi8 ? part[2] : part[0]) + r0;
        const double w1 = (hi8 ? part[3] : part[1]) + r1;
        const double r2 = __shfl_xor(hi4 ? w0 : w1, 4);
        double x = (hi4 ? w1 : w0) + r2;
        x += __shfl_xor(x, 2);
        x += __shfl_xor(x, 1);
        // lane holds block u = 2*hi8 + hi4 of its row group
        const int u = (hi8 ? 2 : 0) + (hi4 ? 1 : 0);
        const int j = tile_j0 + 4 * u + grp;
        if ((lane & 3) == 0 && j < nb) {
            if (x == 0.0) x = 0.0;  // one zero: -0.0 becomes +0.0
            scores[row0 + j] = x;
        }
    }
}

template <int DT>
static hipError_t launch_tpw(const Geo &g, const void *q, const void *S, double *scores,
                             hipStream_t s) {
    // blocks per workgroup = 4 waves x 16 x TPW; keep >= ~4 workgroups per
    // CU-sized slice of the grid when the problem is small
    const long long total = (long long)g.pairs * g.nb;
    if (total >= 2048LL * 256) {
        dim3 grid((g.nb + 255) / 256, g.pairs);
        k_block_score<DT, 4><<<grid, 256, 0, s>>>(q, S, scores, g.hkv, g.gqa, g.nb_cap, g.nb);
    } else if (total >= 2048LL * 128) {
        dim3 grid((g.nb + 127) / 128, g.pairs);
        k_block_score<DT, 2><<<grid, 256, 0, s>>>(q, S, scores, g.hkv, g.gqa, g.nb_cap, g.nb);
    } else {
        dim3 grid((g.nb + 63) / 64, g.pairs);
        k_block_score<DT, 1><<<grid, 256, 0, s>>>(q, S, scores, g.hkv, g.gqa, g.nb_cap, g.nb);
    }
    return hipGetLastError();
}

hipError_t launch_block_score(const Geo &g, const void *q, const void *S, double *scores,
                              hipStream_t s) {
    return g.dtype == KIN_BF16 ? launch_tpw<KIN_BF16>(g, q, S, scores, s)
                               : launch_tpw<KIN_F32>(g, q, S, scores, s);
}

}  // namespace kin
