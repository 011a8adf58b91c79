// select_key32.h -- top-k selection over the keys of one pair, by one
// workgroup, from the top 32 bits of each score's order key: held in LDS
// (the token-level step in one kernel: 32768 keys fit in 128 KiB, where
// their fp64 scores would not) or streamed from memory (the two-kernel
// token step: half the bytes of fp64 scores, written and read).
//
// The kept set is the one select.h defines: the k largest fp64 scores,
// ties to the lower index, indices ascending, then -1 (token-level TopK is
// the block method with blocks of one token: rebuttal "Kinetics: Rethinking
// Test-Time Scaling Law", Q2).
//
// The top 32 bits of a key (sign, exponent, 20 mantissa bits) order the
// keys except inside one 32-bit bin.  The radix select runs over them: the
// sign/exponent bin of the k-th key from a 4096-bin table counted while the
// scores were made, then digits of 8, 8 and 4 bits (one LDS histogram and
// one barrier per pass), stopping as soon as the bin holding the k-th key
// holds exactly the keys still needed.  If all 32 bits are used up, only
// the keys whose top word equals the k-th key's can still be in question;
// their low 32 bits are recomputed from K for exactly those keys, with the
// streaming loop's own arithmetic (exact_score_row), and ranked in four
// more 8-bit passes; keys equal in all 64 bits keep the lower indices.  The
// ordered compaction takes two sweeps (per (round, wave) counts of the keys
// kept for sure and of the exact ties, a workgroup scan, then the writes).
//
// Shared form (Key32Share, the few-pair two-kernel step): the nsplit
// workgroups of one pair, which all need the whole kept list, each sweep
// only their own contiguous range of the keys.  Every pass's 256 counts are
// summed over the splits through the workspace (agent-scope stores and
// loads, one arrival count per exchange), so every split takes the same
// decisions; the compaction exchanges the splits' totals the same way (the
// keys of the lower splits come first in index order), each split writes its kept
// indices into a list in the workspace, and every split reads the whole
// list back.  A split waits only for the other splits of its pair, which
// have all started by then (the splits of a pair take consecutive places in
// the launch's start order).
#pragma once

#include <type_traits>

#include "attn_impl.h"

namespace kin {

// keys of one thread read together: from LDS, or from memory (enough bytes
// in flight per workgroup to cover the memory latency)
constexpr int kKey32BatchLds = 8;
constexpr int kKey32BatchMem = 32;
constexpr int kExpBins = 4096;  // the sign/exponent count table (top 12 bits)

// LDS of the selection over at most MAXN keys after the exponent table has
// been read (it may overlay that table).
template <int NT, int MAXN>
struct Key32Scratch {
    static constexpr int kRounds = (MAXN + NT - 1) / NT;
    uint32_t hist[3][256];
    uint32_t cnt[kRounds * (NT / 64)];
    uint32_t cnt_tie[kRounds * (NT / 64)];
    uint32_t wsum[2][NT / 64];
    double qsum[kHeadDim];  // the group query sum, for the low words
};

// The fp64 score of one bf16 key row against the group query sum (qsum:
// per channel, the heads added in ascending order from +0.0), with the
// arithmetic of the streaming loop: per 8-channel slice s an FMA chain in
// channel order (slice_dot), then the pairing tree of fold4 over the 16
// slices -- x_i = (p_i + p_{i+8}) + (p_{7-i} + p_{15-i}), score =
// (x_0 + x_1) + (x_2 + x_3) -- and -0.0 made +0.0.  So it is bit for bit
// the score that loop made for the same row.
__device__ __noinline__ double exact_score_row(const uint16_t *row, const double *qsum) {
    double p[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(row + 8 * s);
        double acc = 0.0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fma(qsum[8 * s + 2 * e], (double)bf16_lo(w[e]), acc);
            acc = fma(qsum[8 * s + 2 * e + 1], (double)bf16_hi(w[e]), acc);
        }
        p[s] = acc;
    }
    double x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (p[i] + p[i + 8]) + (p[7 - i] + p[15 - i]);
    double v = (x[0] + x[1]) + (x[2] + x[3]);
    if (v == 0.0) v = 0.0;
    return v;
}

// exact_score_row of the pair's token map[j] (row0: the pair's first K row;
// map: a candidate list in memory).
__device__ __noinline__ double exact_score_mapped(const uint16_t *row0, const int32_t *map, int j,
                                                  const double *qsum) {
    return exact_score_row(row0 + (size_t)map[j] * kHeadDim, qsum);
}

// Exclusive prefix sums, in place, of a[0..n) and b[0..n) over the whole
// workgroup (each thread scans a contiguous segment); ta, tb: the totals.
// Ends with a barrier.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t *a, uint32_t *b, int n,
                                      uint32_t (&wsum)[2][NT / 64], uint32_t &ta,
                                      uint32_t &tb) {
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
    ta = tb = 0;
    for (int w = 0; w < NT / 64; ++w) {
        if (w < wave) {
            oa += wsum[0][w];
            ob += wsum[1][w];
        }
        ta += wsum[0][w];
        tb += wsum[1][w];
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

// Top words of keys j0 + u * NT + threadIdx.x, u < B (slots past n re-read
// key 0; callers ignore them).  A whole batch inside the keys (every batch
// but the last) reads from one base address at constant offsets.
template <int NT, int B>
__device__ __forceinline__ void key32_batch(const uint32_t *key, int n, int j0,
                                            uint32_t (&x)[B]) {
    if (j0 + B * NT <= n) {  // uniform
        const uint32_t *p = key + j0 + (int)threadIdx.x;
#pragma unroll
        for (int u = 0; u < B; ++u) x[u] = p[u * NT];
        return;
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const int j = j0 + u * NT + (int)threadIdx.x;
        x[u] = key[j < n ? j : 0];
    }
}

// coarse[i] = fine[16 i] + ... + fine[16 i + 15] for the kExpBins / 16
// coarse bins, by the whole NT-thread workgroup without LDS bank conflicts:
// consecutive lanes read consecutive bins, and each 16-lane row adds its 16
// bins with DPP row shifts (lane 15 of the row ends with the sum).  Every
// thread calls this; a barrier must follow before coarse is read.
template <int NT>
__device__ __forceinline__ void coarse_from_fine(const uint32_t *fine, uint32_t *coarse) {
    static_assert(kExpBins % NT == 0 && NT % 64 == 0, "whole waves over the table");
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i0 = 0; i0 < kExpBins; i0 += NT) {
        const int i = i0 + (int)threadIdx.x;
        uint32_t v = fine[i];
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
        v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
        if ((lane & 15) == 15) coarse[i >> 4] = v;
    }
}

// f(j0, x) for every batch of keys j0 + u * NT + threadIdx.x (u < B) with
// j0 in [lo, hi), in order (lo and hi multiples of B * NT, or hi = n).
template <int NT, int B, class F>
__device__ __forceinline__ void key32_sweep(const uint32_t *key, int n, int lo, int hi, F f) {
    for (int j0 = lo; j0 < hi; j0 += B * NT) {
        uint32_t x[B];
        key32_batch<NT, B>(key, n, j0, x);
        f(j0, x);
    }
}

// The splits of one pair that share its selection (ns == 1: none).
struct Key32Share {
    int ns, split;
    int lo, hi;       // this split's keys [lo, hi)
    uint32_t *hist;   // [2][ns][256] pass counts, by exchange parity
    int32_t *list;    // [k] the kept indices
    uint64_t *word;   // the pair's exchange count (zero on entry)
};

__device__ __forceinline__ Key32Share key32_alone(int n) {
    return Key32Share{1, 0, 0, n, nullptr, nullptr, nullptr};
}

// polls of one exchange before it gives up (about a second; a correct count
// is reached in microseconds)
constexpr uint32_t kSharePollLimit = 1u << 20;

// Agent-scope accesses to the exchange areas, through global-memory pointers
// (those areas are always in the workspace, never in LDS).
template <class T>
__device__ __forceinline__ void st_ws(T *p, T v) {
    typedef __attribute__((address_space(1))) T gT;
    __hip_atomic_store((gT *)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_ws(const T *p) {
    typedef __attribute__((address_space(1))) T gT;
    return __hip_atomic_load((gT *)const_cast<T *>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// This split's stores done, its arrival counted, then the wait until every
// split of the pair has made `round` arrivals.  Every thread calls this.
__device__ __forceinline__ void share_arrive_wait(const Key32Share &x, uint32_t round) {
    stores_complete();
    __syncthreads();
    if (threadIdx.x == 0) {
        typedef __attribute__((address_space(1))) uint64_t gu64;
        __hip_atomic_fetch_add((gu64 *)x.word, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t want = (uint64_t)round * (uint64_t)x.ns;
        uint32_t polls = 0;
        while (ld_ws(x.word) < want && ++polls < kSharePollLimit) __builtin_amdgcn_s_sleep(1);
    }
    __syncthreads();
}

// h[0..256) (LDS, this split's counts) becomes the sum over the pair's
// splits, added in split order.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void share_hist(uint32_t *h, const Key32Share &x, uint32_t &round) {
    if (x.ns == 1) return;
    uint32_t *slot = x.hist + (size_t)(round & 1u) * x.ns * 256;
    for (int i = threadIdx.x; i < 256; i += NT) st_ws(slot + x.split * 256 + i, h[i]);
    share_arrive_wait(x, ++round);
    for (int i = threadIdx.x; i < 256; i += NT) {
        uint32_t sum = 0;
        for (int sp = 0; sp < x.ns; ++sp) sum += ld_ws(slot + sp * 256 + i);
        h[i] = sum;
    }
    __syncthreads();
}

// The kept and tie counts of the splits before this one (its keys' ranks
// start there): every split's (gt, tie) in slots 2 split, 2 split + 1 of
// the zeroed LDS vector tv, summed over the splits.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ void share_totals(uint32_t *tv, uint32_t gt, uint32_t tie,
                                             const Key32Share &x, uint32_t &round,
                                             uint32_t &gt_before, uint32_t &tie_before) {
    if (threadIdx.x == 0) {
        tv[2 * x.split] = gt;
        tv[2 * x.split + 1] = tie;
    }
    __syncthreads();
    share_hist<NT>(tv, x, round);
    gt_before = tie_before = 0;
    for (int sp = 0; sp < x.split; ++sp) {
        gt_before += tv[2 * sp];
        tie_before += tv[2 * sp + 1];
    }
}

// Write out[0..k): the min(k, n) largest keys of the pair, their indices
// ascending, then -1.  key[0..n): top words of the order keys (LDS or global
// memory); fine: the kExpBins-bin count of their top 12 bits over all n
// keys (LDS, may share memory with sc); row0: the pair's first K row (bf16
// rows of kHeadDim) and qp: its first query head, for the low words; sh:
// the splits sharing the selection (key32_alone(n): none; this workgroup
// then sweeps every key).  Key j is token tok0 + j of the pair, or, when
// mapped, token map[j] (a candidate list; out then receives the kept keys'
// places j, which the caller turns into token numbers); out_key, if given,
// receives each kept key's top word (0 past keff).  Every thread
// of the NT-thread workgroup calls this; it ends with a barrier after the
// last write of `out`.  Requires 1 <= k and n <= MAXN.  B: keys per thread
// read together (kKey32BatchLds or kKey32BatchMem); coarse: kExpBins / 16
// words of LDS apart from fine and sc.
template <int NT, int MAXN, int B>
__device__ void select_key32(const uint32_t *key, int n, int k, int32_t *out,
                             const uint32_t *fine, uint32_t *coarse, Key32Scratch<NT, MAXN> &sc,
                             const uint16_t *row0, const uint16_t *qp, int gqa,
                             const Key32Share &sh, int tok0 = 0, bool mapped = false,
                             const int32_t *map = nullptr, uint32_t *out_key = nullptr) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int keff = min(k, n);
    // the exact fp64 score of key j (its K row, through the map if mapped)
    auto exact = [&](int j) -> double {
        return mapped ? exact_score_mapped(row0, map, j, sc.qsum)
                      : exact_score_row(row0 + (size_t)(tok0 + j) * kHeadDim, sc.qsum);
    };
    // this workgroup's keys and rounds (a round: NT consecutive keys)
    const int lo = sh.lo, hi = sh.hi;
    const int r_lo = lo / NT, R = (hi + NT - 1) / NT;
    uint32_t round = 0;  // exchanges made with the other splits

    for (int i = keff + tid; i < k; i += NT) {
        out[i] = -1;
        if (out_key) out_key[i] = 0u;
    }
    if (keff == n) {  // every key is kept
        for (int i = tid; i < n; i += NT) {
            out[i] = tok0 + i;
            if (out_key) out_key[i] = key[i];
        }
        __syncthreads();
        return;
    }

    // sign and exponent of the k-th key: the coarse bins (16 fine bins
    // each), then the 16 fine bins under the chosen one
    coarse_from_fine<NT>(fine, coarse);
    __syncthreads();
    uint32_t krem = (uint32_t)keff;
    uint32_t c[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] = coarse[255 - 4 * lane - r];
    const BinHit h1 = find_bin(c, krem, 255u, lane);
    krem -= h1.above;
#pragma unroll
    for (int r = 0; r < 4; ++r) c[r] = lane < 4 ? fine[16 * h1.digit + 15 - 4 * lane - r] : 0u;
    const BinHit h2 = find_bin(c, krem, 16u * h1.digit + 15u, lane);
    krem -= h2.above;
    uint32_t prefix = h2.digit << 20, pmask = 0xFFFu << 20;
    bool resolved = h2.in_bin == krem;
    __syncthreads();  // every wave has read the table: the scratch may overwrite it
    for (int i = tid; i < 256; i += NT) sc.hist[0][i] = 0u;
    __syncthreads();

    // digits of the top word: bits 19..12, 11..4, then 3..0
    int buf = 0, lo_bit = 12, width = 8;
    while (!resolved) {
        uint32_t *h = sc.hist[buf];
        const int nbuf = buf == 2 ? 0 : buf + 1;
        const uint32_t dmask = (1u << width) - 1u;
        key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
            // past the first digit few keys match: most batches of a wave
            // count nothing and skip the atomics altogether
            auto count = [&](auto whole) {
                auto match = [&](int u) {
                    return (whole.value || j0 + u * NT + tid < n) && (x[u] & pmask) == prefix;
                };
                uint64_t hit = 0;
#pragma unroll
                for (int u = 0; u < B; ++u) hit |= __builtin_amdgcn_ballot_w64(match(u));
                if (hit == 0ull) return;
#pragma unroll
                for (int u = 0; u < B; ++u)
                    if (match(u)) atomicAdd(&h[(x[u] >> lo_bit) & dmask], 1u);
            };
            if (j0 + B * NT <= n)  // uniform: a whole batch, no bound checks
                count(std::true_type());
            else
                count(std::false_type());
        });
        for (int i = tid; i < 256; i += NT) sc.hist[nbuf][i] = 0u;
        __syncthreads();
        share_hist<NT>(h, sh, round);
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] = h[255 - 4 * lane - r];
        const BinHit hb = find_bin(c, krem, 255u, lane);
        buf = nbuf;
        krem -= hb.above;
        prefix |= hb.digit << lo_bit;
        pmask |= dmask << lo_bit;
        if (hb.in_bin == krem) {
            resolved = true;
            break;
        }
        if (lo_bit == 0) break;  // all 32 top bits used
        if (lo_bit >= 8) {
            lo_bit -= 8;
        } else {
            width = lo_bit;
            lo_bit = 0;
        }
    }

    // Not settled by the top words: prefix is now the k-th key's whole top
    // word, and krem keys are still needed among those equal to it.  Rank
    // them on their recomputed low words.
    uint32_t lprefix = 0, lmask = 0;
    bool lresolved = resolved;
    if (!resolved) {
        if (tid < kHeadDim) {
            double s = 0.0;
            for (int hh = 0; hh < gqa; ++hh) s += (double)bf16_lo((uint32_t)qp[hh * kHeadDim + tid]);
            sc.qsum[tid] = s;
        }
        __syncthreads();
        for (int llo = 24;; llo -= 8) {
            uint32_t *h = sc.hist[buf];
            const int nbuf = buf == 2 ? 0 : buf + 1;
            key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int j = j0 + u * NT + tid;
                    if (j < n && x[u] == prefix) {
                        const uint32_t w = (uint32_t)order_key(
                            exact(j));
                        if ((w & lmask) == lprefix) atomicAdd(&h[(w >> llo) & 255u], 1u);
                    }
                }
            });
            for (int i = tid; i < 256; i += NT) sc.hist[nbuf][i] = 0u;
            __syncthreads();
            share_hist<NT>(h, sh, round);
#pragma unroll
            for (int r = 0; r < 4; ++r) c[r] = h[255 - 4 * lane - r];
            const BinHit hb = find_bin(c, krem, 255u, lane);
            buf = nbuf;
            krem -= hb.above;
            lprefix |= hb.digit << llo;
            lmask |= 255u << llo;
            if (hb.in_bin == krem) {
                lresolved = true;
                break;
            }
            if (llo == 0) break;  // all 64 bits used: the rest are exact ties
        }
    }

    // Shared: this split has written its kept indices, out[p0, p0 + cnt)
    // (its keys are consecutive in index order, so are their places); they
    // go to the workspace list, and every split reads the whole list back.
    auto gather = [&](uint32_t p0, uint32_t cnt) {
        if (sh.ns == 1) return;
        for (uint32_t i = p0 + tid; i < p0 + cnt; i += NT) st_ws(sh.list + i, out[i]);
        share_arrive_wait(sh, ++round);
        for (int i = tid; i < keff; i += NT) out[i] = ld_ws(sh.list + i);
        __syncthreads();
    };

    if (resolved) {
        // settled by the top words: kept = top word >= prefix (zeros below
        // its mask); no ties, no low words.  Lane u of a wave carries the
        // count (then the offset) of round j0 / NT + u of the batch, so a
        // round costs a compare, a ballot and a bit count.
        static_assert(B <= 64, "one lane per round of a batch");
        key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
            const int r0 = j0 / NT;
            auto counts = [&](auto whole) {
                uint32_t mine = 0;
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const bool keep = (whole.value || j0 + u * NT + tid < n) && x[u] >= prefix;
                    const uint32_t c = (uint32_t)__popcll(__builtin_amdgcn_ballot_w64(keep));
                    mine = lane == u ? c : mine;
                }
                return mine;
            };
            // uniform: a whole batch needs no bound checks
            const uint32_t mine = j0 + B * NT <= n ? counts(std::true_type())
                                                   : counts(std::false_type());
            if (lane < B && r0 + lane < R) {
                sc.cnt[(r0 + lane) * NW + wave] = mine;
                sc.cnt_tie[(r0 + lane) * NW + wave] = 0u;
            }
        });
        __syncthreads();
        uint32_t tot, tot_tie, before, before_tie;
        block_exclusive_scan2<NT>(sc.cnt + r_lo * NW, sc.cnt_tie + r_lo * NW, (R - r_lo) * NW,
                                  sc.wsum, tot, tot_tie);
        share_totals<NT>(sc.hist[buf], tot, 0u, sh, round, before, before_tie);
        key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
            const int r0 = j0 / NT;
            const uint32_t base = lane < B && r0 + lane < R ? sc.cnt[(r0 + lane) * NW + wave] : 0u;
            auto write = [&](auto whole) {
#pragma unroll
                for (int u = 0; u < B; ++u) {
                    const int j = j0 + u * NT + tid;
                    const bool keep = (whole.value || j < n) && x[u] >= prefix;
                    const uint64_t kb = __builtin_amdgcn_ballot_w64(keep);
                    if (kb == 0ull) continue;  // uniform: nothing kept in this round
                    const uint32_t pos = before + lane_value(base, u) + rank_below(kb);
                    if (keep) {
                        out[pos] = tok0 + j;
                        if (out_key) out_key[pos] = x[u];
                    }
                }
            };
            if (j0 + B * NT <= n)  // uniform: a whole batch, no bound checks
                write(std::true_type());
            else
                write(std::false_type());
        });
        __syncthreads();
        gather(before, tot);
        return;
    }

    // Class of key j: 2 = kept for sure, 1 = equal in all 64 bits to the
    // k-th key (the first krem of these in index order are kept), 0 = not.
    auto cls = [&](int j, uint32_t x) -> int {
        if (x != prefix) return x > prefix ? 2 : 0;
        const uint32_t w =
            (uint32_t)order_key(exact(j));
        if (lresolved) return w >= lprefix ? 2 : 0;
        return w > lprefix ? 2 : (w == lprefix ? 1 : 0);
    };

    // ordered compaction: counts per (round, wave), a scan, then the writes
    key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int r = j0 / NT + u;
            if (r >= R) break;  // uniform
            const int j = r * NT + tid;
            const int cl = j < n ? cls(j, x[u]) : 0;
            const uint64_t ma = __ballot(cl == 2), mt = __ballot(cl == 1);
            if (lane == 0) {
                sc.cnt[r * NW + wave] = (uint32_t)__popcll(ma);
                sc.cnt_tie[r * NW + wave] = (uint32_t)__popcll(mt);
            }
        }
    });
    __syncthreads();
    uint32_t tot, tot_tie, before, before_tie;
    block_exclusive_scan2<NT>(sc.cnt + r_lo * NW, sc.cnt_tie + r_lo * NW, (R - r_lo) * NW, sc.wsum,
                              tot, tot_tie);
    share_totals<NT>(sc.hist[buf], tot, tot_tie, sh, round, before, before_tie);
    key32_sweep<NT, B>(key, n, lo, hi, [&](int j0, const uint32_t (&x)[B]) {
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int r = j0 / NT + u;
            if (r >= R) break;  // uniform
            const int j = r * NT + tid;
            const int cl = j < n ? cls(j, x[u]) : 0;
            const uint64_t ma = __ballot(cl == 2), mt = __ballot(cl == 1);
            const uint32_t gt_before = before + sc.cnt[r * NW + wave] + rank_below(ma);
            const uint32_t tie_before = before_tie + sc.cnt_tie[r * NW + wave] + rank_below(mt);
            if (cl == 2 || (cl == 1 && tie_before < krem)) {
                const uint32_t pos = gt_before + min(tie_before, krem);
                out[pos] = tok0 + j;
                if (out_key) out_key[pos] = x[u];
            }
        }
    });
    __syncthreads();
    // this split's kept keys: its sure ones and its ties that are still kept
    const uint32_t ties_kept = min(before_tie + tot_tie, krem) - min(before_tie, krem);
    gather(before + min(before_tie, krem), tot + ties_kept);
}

}  // namespace kin
