// topk.hip -- K3: per-(sequence, KV head) top-k block selection.
//
// The kept set is the k blocks with the largest group scores
// (torch.topk over the per-block mean scores in BlockTopKAttention, skill
// summary "Kinetics: Memory-Aware Test-Time Scaling", Implementation; k is
// counted in blocks, rebuttal "Kinetics: Rethinking Test-Time Scaling Law",
// Q4 "KV block size and grouping strategy").  Ties keep the lower block
// index, and the indices are written in ascending order (the order the
// attention kernel walks the cache).
//
// Method: one 512-thread workgroup per pair, the pair's scores held in
// registers (up to KPT per thread).  Each fp64 score maps to an unsigned
// 64-bit key with the same order (flip all bits of negatives, set the sign
// bit of the rest).  An MSD radix select over 8-bit digits finds the k-th
// largest key: per pass, an LDS histogram of the digit among the keys that
// still match the prefix (a wave whose candidates all share one digit adds
// its ballot count with a single atomic), then one wave scans the 256 bins
// from the top.  It stops as soon as the bin that holds the k-th key holds
// exactly the keys still needed.  If all 64 bits are used up, the remaining
// equal keys are exact ties and the lowest indices among them are kept.
// The kept flags are finally compacted in block order with ballot + mbcnt
// ranks and a scan of per-wave counts, which yields ascending indices.
#include "kin_internal.h"

namespace kin {

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;

__device__ __forceinline__ uint64_t order_key(double s) {
    if (s == 0.0) s = 0.0;  // -0.0 and +0.0 are one score
    const uint64_t u = (uint64_t)__double_as_longlong(s);
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ uint32_t rank_below(uint64_t mask) {
    // number of set bits of mask in lanes below this one
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Exclusive scan, in (e, wave) order, of cnt[e][wave] for e < kpt; in place.
// Called by every thread; uses wave 0 only.
__device__ void scan_counts(uint32_t *cnt, int n) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        uint32_t carry = 0;
        for (int base = 0; base < n; base += 64) {
            const int i = base + lane;
            const uint32_t v = i < n ? cnt[i] : 0u;
            uint32_t incl = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d);
                if (lane >= d) incl += o;
            }
            if (i < n) cnt[i] = carry + incl - v;
            carry += __shfl(incl, 63);
        }
    }
}

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void k_block_topk(const double *__restrict__ scores,
                                                             int32_t *__restrict__ idx,
                                                             int nb_cap, int nb, int k) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t cnt[KPT * kTopkWaves];
    __shared__ uint32_t s_digit, s_above, s_in_bin;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const size_t pair = blockIdx.x;
    const double *sc = scores + pair * (size_t)nb_cap;
    int32_t *out = idx + pair * (size_t)k;
    const int keff = min(k, nb);

    for (int i = keff + tid; i < k; i += kTopkThreads) out[i] = -1;
    if (keff == nb) {  // every block is kept
        for (int i = tid; i < nb; i += kTopkThreads) out[i] = i;
        return;
    }

    uint64_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int j = e * kTopkThreads + tid;
        key[e] = j < nb ? order_key(sc[j]) : 0ull;  // 0 is below every finite key
    }

    uint64_t prefix = 0, pmask = 0;
    uint32_t krem = (uint32_t)keff;
    bool resolved = false;  // true: every key matching `prefix` is kept
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const bool cand = (e * kTopkThreads + tid < nb) && ((key[e] & pmask) == prefix);
            const uint32_t dig = (uint32_t)(key[e] >> shift) & 255u;
            const uint64_t act = __ballot(cand);
            if (act == 0) continue;
            const int first = __builtin_ctzll(act);
            const uint32_t d0 = __shfl(dig, first);
            const uint64_t same = __ballot(cand && dig == d0);
            if (same == act) {
                if (lane == first) atomicAdd(&hist[d0], (uint32_t)__popcll(act));
            } else if (cand) {
                atomicAdd(&hist[dig], 1u);
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l (descending digits)
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                c[r] = hist[255 - 4 * lane - r];
                sum += c[r];
            }
            uint32_t incl = sum;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t o = __shfl_up(incl, d);
                if (lane >= d) incl += o;
            }
            const uint32_t excl = incl - sum;
            if (excl < krem && krem <= incl) {
                uint32_t run = excl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (run + c[r] >= krem) {
                        s_digit = 255u - 4u * lane - r;
                        s_above = run;
                        s_in_bin = c[r];
                        break;
                    }
                    run += c[r];
                }
            }
        }
        __syncthreads();
        const uint32_t dsel = s_digit, above = s_above, in_bin = s_in_bin;
        krem -= above;
        prefix |= (uint64_t)dsel << shift;
        pmask |= 0xFFull << shift;
        if (in_bin == krem) {
            resolved = true;
            break;
        }
    }

    // kept: key above the threshold prefix, or equal to it and (resolved, or
    // among the first krem equal keys in block order)
    bool keep[KPT];
    if (resolved) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) keep[e] = (e * kTopkThreads + tid < nb) && key[e] >= prefix;
    } else {
        // prefix is now the exact k-th key; rank the ties in block order
        bool tie[KPT];
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            tie[e] = (e * kTopkThreads + tid < nb) && key[e] == prefix;
            const uint64_t m = __ballot(tie[e]);
            if (lane == 0) cnt[e * kTopkWaves + wave] = (uint32_t)__popcll(m);
        }
        __syncthreads();
        scan_counts(cnt, KPT * kTopkWaves);
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const uint64_t m = __ballot(tie[e]);
            const uint32_t r = cnt[e * kTopkWaves + wave] + rank_below(m);
            keep[e] = (e * kTopkThreads + tid < nb) && (key[e] > prefix || (tie[e] && r < krem));
        }
        __syncthreads();  // cnt is reused below
    }

#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint64_t m = __ballot(keep[e]);
        if (lane == 0) cnt[e * kTopkWaves + wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    scan_counts(cnt, KPT * kTopkWaves);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint64_t m = __ballot(keep[e]);
        const uint32_t pos = cnt[e * kTopkWaves + wave] + rank_below(m);
        if (keep[e] && pos < (uint32_t)keff) out[pos] = e * kTopkThreads + tid;
    }
}

hipError_t launch_block_topk(const Geo &g, const double *scores, int k, int32_t *idx,
                             hipStream_t s) {
    const int kpt = (g.nb + kTopkThreads - 1) / kTopkThreads;
    dim3 grid(g.pairs);
    if (kpt <= 1)
        k_block_topk<1><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    else if (kpt <= 2)
        k_block_topk<2><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    else if (kpt <= 4)
        k_block_topk<4><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    else if (kpt <= 8)
        k_block_topk<8><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    else if (kpt <= 16)
        k_block_topk<16><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    else
        k_block_topk<32><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k);
    return hipGetLastError();
}

}  // namespace kin
