// select.h -- device-side top-k block selection for one (sequence, KV head)
// pair, run by one whole workgroup of NT threads.
//
// The kept set is the k blocks with the largest group scores
// (torch.topk over the per-block mean scores in BlockTopKAttention, skill
// summary "Kinetics: Memory-Aware Test-Time Scaling", Implementation; k is
// counted in blocks, rebuttal "Kinetics: Rethinking Test-Time Scaling Law",
// Q4 "KV block size and grouping strategy").  Ties keep the lower block
// index, and the indices are written in ascending order (the order the
// attention kernel walks the cache).
//
// Method: the pair's scores are held in registers (KPT per thread, block
// j = e * NT + tid).  Each fp64 score maps to an unsigned 64-bit key with
// the same order (flip all bits of negatives, set the sign bit of the
// rest).  An MSD radix select finds the k-th largest key.  Its top 12 bits
// (sign and exponent) come either from two count tables filled one atomic
// per key while the scores are computed (COUNTED: the fused decode step,
// where the atomics hide under HBM latency; by bits 63..56, 256 bins, and
// by bits 63..52, 4096 bins; every wave reads the 256 coarse bins, then the
// 16 fine bins under the chosen coarse one, with no barrier), or, when the
// scores arrive ready-made, from a search down from the largest bin: the
// keys of the 8 bins below it are counted with ballots per round (a pair's
// scores sit in a few neighbouring bins, and per-key LDS atomics on those
// few words would queue), falling back to the tables after two rounds.  The
// mantissa follows 8 bits at a time (the last 4): each pass builds an LDS
// histogram of the digit among the keys that still match the prefix (one
// LDS atomic per candidate), then EVERY wave scans the 256 bins itself
// (a DPP prefix sum, lane broadcasts by readlane), so a pass costs a single
// barrier: three histogram buffers rotate, and the buffer for pass p+1 is
// cleared during pass p (its last readers finished before the barrier of
// pass p-1).  The select stops as soon as the bin holding the k-th key
// holds exactly the keys still needed; if all 64 bits are used up, the
// remaining equal keys are exact ties and the lowest indices among them are
// kept.  The kept flags are compacted in block order with ballot + mbcnt
// ranks and a scan of the per-wave counts that every wave repeats (one
// barrier).
#pragma once

#include "kin_internal.h"

namespace kin {

template <int KPT, int NT>
struct SelectLds {
    uint32_t coarse[256];   // keys per value of bits 63..56
    uint32_t fine[4096];    // keys per value of bits 63..52 (sign, exponent)
    uint32_t hist[3][256];  // mantissa passes
    uint32_t cnt[KPT * (NT / 64)];
    uint32_t cnt_tie[KPT * (NT / 64)];
    uint32_t wtop[NT / 64];             // per wave: largest sign/exponent bin
    uint32_t wcnt[2][8 * (NT / 64)];    // per round, bin and wave: keys counted
    static_assert(NT / 64 <= 8, "the bin counts of all waves fit one wave");
};

__device__ __forceinline__ uint64_t order_key(double s) {
    if (s == 0.0) s = 0.0;  // -0.0 and +0.0 are one score
    const uint64_t u = (uint64_t)__double_as_longlong(s);
    return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Zero the count tables and the first mantissa histogram; every thread of
// the workgroup calls this, and a barrier must separate it from the first
// select_count or select_topk.
template <int KPT, int NT>
__device__ __forceinline__ void select_clear(SelectLds<KPT, NT> &lds) {
    for (int i = threadIdx.x; i < 4096; i += NT) lds.fine[i] = 0u;
    for (int i = threadIdx.x; i < 256; i += NT) {
        lds.coarse[i] = 0u;
        lds.hist[0][i] = 0u;
    }
}

// Count one score in the two exponent tables (each score exactly once).
template <int KPT, int NT>
__device__ __forceinline__ void select_count(SelectLds<KPT, NT> &lds, double s) {
    const uint64_t key = order_key(s);
    atomicAdd(&lds.coarse[key >> 56], 1u);
    atomicAdd(&lds.fine[key >> 52], 1u);
}

__device__ __forceinline__ uint32_t rank_below(uint64_t mask) {
    // number of set bits of mask in lanes below this one
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Value of v in lane `src` (src uniform across the wave): a scalar read of
// one lane, no LDS round trip.
__device__ __forceinline__ uint32_t lane_value(uint32_t v, int src) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, src);
}

// Inclusive prefix sum over the 64 lanes with DPP moves (row shifts inside
// each 16-lane row, then row broadcasts of lanes 15 and 31); lanes with no
// source add the 0 held in `old`.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return v;
}

// Largest value over the 64 lanes (DPP row shifts, then row broadcasts; the
// result is read from lane 63).
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return lane_value(v, 63);
}

// Every wave: the exclusive prefix, in (e, wave) order, of cnt[e * NW + w]
// at position (e, my_wave), for each e < KPT.  n = KPT * NW entries.
template <int KPT, int NW>
__device__ __forceinline__ void offsets_of(const uint32_t *cnt, int wave, int lane,
                                           uint32_t (&off)[KPT]) {
    constexpr int N = KPT * NW;
    uint32_t carry = 0;
#pragma unroll
    for (int base = 0; base < N; base += 64) {
        const int i = base + lane;
        const uint32_t v = i < N ? cnt[i] : 0u;
        const uint32_t incl = wave_incl_scan(v);
        const uint32_t excl = carry + incl - v;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int at = e * NW + wave;
            if (at >= base && at < base + 64) off[e] = lane_value(excl, at - base);
        }
        carry += lane_value(incl, 63);
    }
}

// table[bin] += 1 for every lane with `on`, one atomic per distinct bin of
// the wave instead of one per lane: the scores of a pair fall into a few
// sign/exponent bins, so per-lane atomics would queue on the same words.
// The first two distinct bins are added by their lowest lane with a
// population count; lanes with other bins add 1 each.
__device__ __forceinline__ void count_wave_aggregated(uint32_t *table, uint32_t bin, bool on) {
#pragma unroll
    for (int round = 0; round < 2; ++round) {
        const uint64_t act = __ballot(on);
        if (act == 0) return;
        const int src = __builtin_ctzll(act);
        const uint32_t lead = lane_value(bin, src);
        const uint64_t same = __ballot(on && bin == lead);
        if ((int)(threadIdx.x & 63) == src) atomicAdd(&table[lead], (uint32_t)__popcll(same));
        on = on && bin != lead;
    }
    if (on) atomicAdd(&table[bin], 1u);
}

// Every wave: the bin holding the krem-th largest key, given that lane l
// holds the counts c[0..3] of bins base - 4l .. base - 4l - 3 (descending
// digits).  Returns the digit, the keys in bins above it and in it.
struct BinHit {
    uint32_t digit, above, in_bin;
};

__device__ __forceinline__ BinHit find_bin(const uint32_t (&c)[4], uint32_t krem, uint32_t base,
                                           int lane) {
    const uint32_t sum = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(sum);
    const uint32_t excl = incl - sum;
    const uint64_t hit = __ballot(excl < krem && krem <= incl);
    const int src = __builtin_ctzll(hit);
    // bins are disjoint in the running sum: at most one r of the hit lane
    // brackets krem (selects, no branches)
    uint32_t run = excl, dsel = 0, above = 0, in_bin = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const uint32_t next = run + c[r];
        const bool here = run < krem && krem <= next;
        dsel = here ? base - 4u * lane - r : dsel;
        above = here ? run : above;
        in_bin = here ? c[r] : in_bin;
        run = next;
    }
    return BinHit{lane_value(dsel, src), lane_value(above, src), lane_value(in_bin, src)};
}

// The selection's hook once the sign/exponent bin of the k-th key is known
// from the count tables: early(key, bin), called by every thread with its
// keys (block e * NT + threadIdx.x in key[e]; 0 past nb) and the bin (top
// 12 bits of the k-th key); keys in higher bins are certainly kept.  This
// one does nothing.
struct NoEarly {
    template <int KPT>
    __device__ void operator()(const uint64_t (&)[KPT], uint32_t) const {}
};

// Write out[0..k): the min(k, nb) selected block indices ascending, then -1.
// sc: the pair's scores (nb entries; global memory or LDS).  Every thread of
// the workgroup calls this, after select_clear and a barrier; with COUNTED
// the caller has also passed every score to select_count (and synchronised
// since), and early (see NoEarly) runs between the count tables and the
// mantissa passes.  It ends without a barrier, so callers synchronise before
// other waves read `out`.  Requires 1 <= k and nb <= KPT * NT.
template <int KPT, int NT, bool COUNTED, class Early = NoEarly>
__device__ void select_topk(const double *__restrict__ sc, int nb, int k, int32_t *out,
                            SelectLds<KPT, NT> &lds, Early early = Early()) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int keff = min(k, nb);

    for (int i = keff + tid; i < k; i += NT) out[i] = -1;
    if (keff == nb) {  // every block is kept
        for (int i = tid; i < nb; i += NT) out[i] = i;
        return;
    }

    // all loads first (slots past nb re-read entry nb - 1), then the keys;
    // 0 is below every finite key
    double v[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) v[e] = sc[min(e * NT + tid, nb - 1)];
    uint64_t key[KPT];
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const int j = e * NT + tid;
        key[e] = order_key(v[e]) & (0ull - (uint64_t)(j < nb));  // a mask, not a branch
    }

    // sign and exponent of the k-th key
    uint32_t krem = (uint32_t)keff;
    uint64_t prefix = 0, pmask = 0xFFFull << 52;
    uint32_t in_bin = 0;
    bool have = COUNTED;  // COUNTED: read off the count tables below
    if (!COUNTED) {
        // Without count tables: the largest sign/exponent bin of the pair,
        // then the keys in the 8 bins below it counted with ballots (no
        // atomics; a pair's scores sit in a few neighbouring bins, so the
        // k-th key is almost always there), one barrier per round of 8.
        uint32_t top = 0;
#pragma unroll
        for (int e = 0; e < KPT; ++e) top = max(top, (uint32_t)(key[e] >> 52));  // invalid: 0
        top = wave_max(top);
        if (lane == 0) lds.wtop[wave] = top;
        __syncthreads();
        top = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) top = max(top, lds.wtop[w]);
        bool found = false;
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            if (found) break;
            const uint32_t base = 8u * round;
            // this lane's keys per bin q, two 16-bit counters per word
            // (a wave holds at most 64 * 32 keys, so the sums fit)
            uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const bool valid = e * NT + tid < nb;
                const uint32_t d = top - (uint32_t)(key[e] >> 52) - base;
                const uint32_t inc = (valid && d < 8u) ? 1u << (16 * (d & 1u)) : 0u;
#pragma unroll
                for (int h = 0; h < 4; ++h) c[h] += (d >> 1) == (uint32_t)h ? inc : 0u;
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) c[h] = wave_incl_scan(c[h]);  // lane 63: the wave's
            if (lane == 63) {
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    lds.wcnt[round][q * NW + wave] = (c[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
            }
            __syncthreads();
            // lane q * NW + w reads one count; bin q's total is the scan's
            // step over lanes q * NW .. q * NW + NW - 1
            const uint32_t mine = lane < 8 * NW ? lds.wcnt[round][lane] : 0u;
            const uint32_t incl = wave_incl_scan(mine);
            uint32_t run = 0;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t total = lane_value(incl, q * NW + NW - 1) - run;
                if (!found && run + total >= krem) {
                    found = true;
                    prefix = (uint64_t)(top - base - q) << 52;
                    krem -= run;
                    in_bin = total;
                }
                run += total;
            }
            if (!found) krem -= run;
        }
        if (!found) {
            // far below the top (e.g. across zero): the count tables after all
            krem = (uint32_t)keff;
#pragma unroll
            for (int e = 0; e < KPT; ++e)
                count_wave_aggregated(lds.fine, (uint32_t)(key[e] >> 52), e * NT + tid < nb);
            __syncthreads();
            for (int i = tid; i < 256; i += NT) {  // coarse = fine summed over 16 bins
                const uint32_t *f = lds.fine + 16 * i;
                uint32_t c = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) c += f[r];
                lds.coarse[i] = c;
            }
            __syncthreads();
        }
        have = !found;
    }
    if (have) {
        // from the count tables: the coarse bin, then the fine bin under it
        uint32_t c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = lds.coarse[255 - 4 * lane - r];
        const BinHit h1 = find_bin(c, krem, 255u, lane);
        krem -= h1.above;
        // lanes 0..3 hold the 16 fine bins of coarse bin h1.digit, descending
#pragma unroll
        for (int r = 0; r < 4; ++r)
            c[r] = lane < 4 ? lds.fine[16 * h1.digit + 15 - 4 * lane - r] : 0u;
        const BinHit h2 = find_bin(c, krem, 16u * h1.digit + 15u, lane);
        krem -= h2.above;
        prefix = (uint64_t)h2.digit << 52;
        in_bin = h2.in_bin;
        if (COUNTED) early(key, h2.digit);
    }
    bool resolved = in_bin == krem;  // true: every key matching `prefix` is kept

    // mantissa: bits 51..44, 43..36, ..., 11..4, then 3..0
    int buf = 0;
    int lo = 44, width = 8;  // bit range of the current digit: [lo, lo + width)
    while (!resolved) {
        uint32_t *h = lds.hist[buf];
        const int nbuf = buf == 2 ? 0 : buf + 1;
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const bool cand = (e * NT + tid < nb) && ((key[e] & pmask) == prefix);
            const uint32_t dig = (uint32_t)(key[e] >> lo) & ((1u << width) - 1u);
            if (cand) atomicAdd(&h[dig], 1u);
        }
        for (int i = tid; i < 256; i += NT) lds.hist[nbuf][i] = 0u;
        __syncthreads();
        // every wave: lane l holds bins 255-4l .. 252-4l (descending digits)
        uint32_t c[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = h[255 - 4 * lane - r];
        const BinHit hb = find_bin(c, krem, 255u, lane);
        buf = nbuf;
        krem -= hb.above;
        prefix |= (uint64_t)hb.digit << lo;
        pmask |= (uint64_t)((1u << width) - 1u) << lo;
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

    // kept: key above the threshold prefix, or equal to it and (resolved, or
    // among the first krem equal keys in block order)
    bool keep[KPT];
    if (resolved) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) keep[e] = (e * NT + tid < nb) && key[e] >= prefix;
    } else {
        // prefix is now the exact k-th key; rank the ties in block order
        bool tie[KPT];
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            tie[e] = (e * NT + tid < nb) && key[e] == prefix;
            const uint64_t m = __ballot(tie[e]);
            if (lane == 0) lds.cnt_tie[e * NW + wave] = (uint32_t)__popcll(m);
        }
        __syncthreads();
        uint32_t off[KPT];
        offsets_of<KPT, NW>(lds.cnt_tie, wave, lane, off);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const uint64_t m = __ballot(tie[e]);
            const uint32_t r = off[e] + rank_below(m);
            keep[e] = (e * NT + tid < nb) && (key[e] > prefix || (tie[e] && r < krem));
        }
    }

#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint64_t m = __ballot(keep[e]);
        if (lane == 0) lds.cnt[e * NW + wave] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    uint32_t off[KPT];
    offsets_of<KPT, NW>(lds.cnt, wave, lane, off);
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
        const uint64_t m = __ballot(keep[e]);
        const uint32_t pos = off[e] + rank_below(m);
        if (keep[e] && pos < (uint32_t)keff) out[pos] = e * NT + tid;
    }
}

// Keys per thread for nb blocks over nt threads, rounded up to an
// instantiated power of two (nb <= 32 * nt).
__host__ __device__ inline int select_kpt(int nb, int nt) {
    const int kpt = (nb + nt - 1) / nt;
    return kpt <= 1 ? 1 : kpt <= 2 ? 2 : kpt <= 4 ? 4 : kpt <= 8 ? 8 : kpt <= 16 ? 16 : 32;
}

}  // namespace kin
