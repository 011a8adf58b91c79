// select_stream.h -- top-k selection for one pair by one workgroup when the
// keys do not fit in registers (token-level selection: one key per token,
// up to kStreamMaxRounds * NT of them).
//
// The kept set follows the same rule as select.h: the k largest fp64
// scores, ties to the lower index, indices written in ascending order,
// then -1 (token-level TopK is the block method with blocks of one token:
// rebuttal "Kinetics: Rethinking Test-Time Scaling Law", Q2, which compares
// TopK attention over single tokens with Block-TopK).
//
// Method: the same MSD radix select over order-preserving u64 keys, but
// every pass streams the scores from memory (coalesced: key j = r * NT +
// tid in round r) instead of keeping them in registers.  Pass 0 counts the
// sign/exponent bins (wave-aggregated LDS atomics), then 8-bit mantissa
// digits follow until the bin of the k-th key holds exactly the keys still
// needed (or all 64 bits are used: exact ties, lowest indices first).  The
// ordered compaction takes two more streams: per (round, wave) counts of
// the keys above the threshold and of the ties, an exclusive scan of those
// counts over the workgroup, then the writes.
#pragma once

#include "select.h"

namespace kin {

constexpr int kStreamMaxRounds = 512;
constexpr int kStreamBatch = 16;  // rounds whose loads are issued together

// The keys of rounds r0 .. r0 + kStreamBatch - 1 of this thread (slots past
// n re-read key 0; callers ignore them): one batch of independent loads, so
// a pass waits for memory once per batch, not once per round.
template <int NT>
__device__ __forceinline__ void load_keys(const double *__restrict__ sc, int n, int r0,
                                          uint64_t (&key)[kStreamBatch]) {
    double v[kStreamBatch];
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) {
        const int j = (r0 + u) * NT + (int)threadIdx.x;
        v[u] = sc[j < n ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) key[u] = order_key(v[u]);
}

template <int NT>
struct StreamSelectLds {
    uint32_t coarse[256];
    uint32_t fine[4096];
    uint32_t hist[3][256];
    uint32_t cnt[kStreamMaxRounds * (NT / 64)];      // keys above the threshold
    uint32_t cnt_tie[kStreamMaxRounds * (NT / 64)];  // keys equal to it
    uint32_t wsum[2][NT / 64];
};

// Exclusive prefix sums, in place, of a[0..n) and b[0..n) over the whole
// workgroup (each thread scans a contiguous segment).  Ends with a barrier.
template <int NT>
__device__ void block_exclusive_scan2(uint32_t *a, uint32_t *b, int n, uint32_t (&wsum)[2][NT / 64]) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = (n + NT - 1) / NT;
    const int s0 = min(tid * m, n), s1 = min(s0 + m, n);
    uint32_t sa = 0, sb = 0;
    for (int i = s0; i < s1; ++i) {
        sa += a[i];
        sb += b[i];
    }
    const uint32_t ia = wave_incl_scan(sa), ib = wave_incl_scan(sb);
    if (lane == 63) {
        wsum[0][wave] = ia;
        wsum[1][wave] = ib;
    }
    __syncthreads();
    uint32_t oa = ia - sa, ob = ib - sb;
    for (int w = 0; w < wave; ++w) {
        oa += wsum[0][w];
        ob += wsum[1][w];
    }
    for (int i = s0; i < s1; ++i) {
        const uint32_t va = a[i], vb = b[i];
        a[i] = oa;
        b[i] = ob;
        oa += va;
        ob += vb;
    }
    __syncthreads();
}

// Sign/exponent counts of a run of keys: 256 bins by bits 63..56, then 4096
// by bits 63..52 (kTableWords words per run).
constexpr int kTableWords = 256 + 4096;

// Write out[0..k): the min(k, n) largest of sc[0..n) (global memory), their
// indices ascending, then -1.  Every thread of the NT-thread workgroup calls
// this; it ends with a barrier after the last write of `out` (LDS or
// global).  tables: NULL, or ntables count tables (kTableWords each, written
// by an earlier kernel) that together count every key once; pass 0 is then
// skipped.  Requires 1 <= k and n <= kStreamMaxRounds * NT.
template <int NT>
__device__ void select_stream(const double *__restrict__ sc, int n, int k, int32_t *out,
                              StreamSelectLds<NT> &lds, const uint32_t *__restrict__ tables,
                              int ntables) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int keff = min(k, n);
    const int R = (n + NT - 1) / NT;

    for (int i = keff + tid; i < k; i += NT) out[i] = -1;
    if (keff == n) {  // every key is kept
        for (int i = tid; i < n; i += NT) out[i] = i;
        __syncthreads();
        return;
    }

    for (int i = tid; i < 256; i += NT) lds.hist[0][i] = 0u;
    if (tables) {
        // pass 0 from the count tables: the coarse sums now, the 16 fine
        // bins under the chosen coarse bin below
        for (int i = tid; i < 256; i += NT) {
            uint32_t c = 0;
            for (int t = 0; t < ntables; ++t) c += tables[(size_t)t * kTableWords + i];
            lds.coarse[i] = c;
        }
        __syncthreads();
    } else {
        for (int i = tid; i < 4096; i += NT) lds.fine[i] = 0u;
        __syncthreads();

        // pass 0: keys per sign/exponent bin
        for (int r0 = 0; r0 < R; r0 += kStreamBatch) {
            uint64_t key[kStreamBatch];
            load_keys<NT>(sc, n, r0, key);
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u)
                if (r0 + u < R)  // uniform over the workgroup
                    count_wave_aggregated(lds.fine, (uint32_t)(key[u] >> 52),
                                          (r0 + u) * NT + tid < n);
        }
        __syncthreads();
        for (int i = tid; i < 256; i += NT) {
            const uint32_t *f = lds.fine + 16 * i;
            uint32_t c = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) c += f[r];
            lds.coarse[i] = c;
        }
        __syncthreads();
    }

    uint32_t krem = (uint32_t)keff;
    uint64_t prefix, pmask = 0xFFFull << 52;
    uint32_t in_bin;
    {
        uint32_t c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = lds.coarse[255 - 4 * lane - r];
        const BinHit h1 = find_bin(c, krem, 255u, lane);
        krem -= h1.above;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int f = 16 * h1.digit + 15 - 4 * lane - r;
            uint32_t v = 0;
            if (lane < 4) {
                if (tables) {
                    for (int t = 0; t < ntables; ++t)
                        v += tables[(size_t)t * kTableWords + 256 + f];
                } else {
                    v = lds.fine[f];
                }
            }
            c[r] = v;
        }
        const BinHit h2 = find_bin(c, krem, 16u * h1.digit + 15u, lane);
        krem -= h2.above;
        prefix = (uint64_t)h2.digit << 52;
        in_bin = h2.in_bin;
    }
    bool resolved = in_bin == krem;

    // mantissa digits: bits 51..44, ..., 11..4, then 3..0
    int buf = 0, lo = 44, width = 8;
    while (!resolved) {
        uint32_t *h = lds.hist[buf];
        const int nbuf = buf == 2 ? 0 : buf + 1;
        const uint32_t dmask = (1u << width) - 1u;
        for (int r0 = 0; r0 < R; r0 += kStreamBatch) {
            uint64_t key[kStreamBatch];
            load_keys<NT>(sc, n, r0, key);
#pragma unroll
            for (int u = 0; u < kStreamBatch; ++u)
                if ((r0 + u) * NT + tid < n && (key[u] & pmask) == prefix)
                    atomicAdd(&h[(uint32_t)(key[u] >> lo) & dmask], 1u);
        }
        for (int i = tid; i < 256; i += NT) lds.hist[nbuf][i] = 0u;
        __syncthreads();
        uint32_t c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = h[255 - 4 * lane - r];
        const BinHit hb = find_bin(c, krem, 255u, lane);
        buf = nbuf;
        krem -= hb.above;
        prefix |= (uint64_t)hb.digit << lo;
        pmask |= (uint64_t)dmask << lo;
        if (hb.in_bin == krem) {
            resolved = true;
            break;
        }
        if (lo == 0) break;  // all 64 bits used: the rest are exact ties
        if (lo >= 8) {
            lo -= 8;
        } else {
            width = lo;
            lo = 0;
        }
    }

    // compaction: above = kept for sure; tie = equal to the exact k-th key
    // (only when not resolved), the first krem of them in index order kept
    for (int r0 = 0; r0 < R; r0 += kStreamBatch) {
        uint64_t key[kStreamBatch];
        load_keys<NT>(sc, n, r0, key);
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) {
            const int r = r0 + u;
            if (r >= R) break;  // uniform
            const bool on = r * NT + tid < n;
            const bool above = on && (resolved ? key[u] >= prefix : key[u] > prefix);
            const bool tie = on && !resolved && key[u] == prefix;
            const uint64_t ma = __ballot(above), mt = __ballot(tie);
            if (lane == 0) {
                lds.cnt[r * NW + wave] = (uint32_t)__popcll(ma);
                lds.cnt_tie[r * NW + wave] = (uint32_t)__popcll(mt);
            }
        }
    }
    __syncthreads();
    block_exclusive_scan2<NT>(lds.cnt, lds.cnt_tie, R * NW, lds.wsum);
    for (int r0 = 0; r0 < R; r0 += kStreamBatch) {
        uint64_t key[kStreamBatch];
        load_keys<NT>(sc, n, r0, key);
#pragma unroll
        for (int u = 0; u < kStreamBatch; ++u) {
            const int r = r0 + u;
            if (r >= R) break;  // uniform
            const int j = r * NT + tid;
            const bool above = j < n && (resolved ? key[u] >= prefix : key[u] > prefix);
            const bool tie = j < n && !resolved && key[u] == prefix;
            const uint64_t ma = __ballot(above), mt = __ballot(tie);
            const uint32_t gt_before = lds.cnt[r * NW + wave] + rank_below(ma);
            const uint32_t tie_before = lds.cnt_tie[r * NW + wave] + rank_below(mt);
            if (above || (tie && tie_before < krem)) out[gt_before + min(tie_before, krem)] = j;
        }
    }
    __syncthreads();
}

}  // namespace kin
