// attn_impl.h -- device side of the decode attention: the kept-token list
// walk, the bf16 MFMA chunk (loads, scores, online softmax, P.V), the fp32
// VALU chunk, and the merge of a workgroup's waves.  Shared by the
// standalone attention kernels, the fused select+attend kernel and the
// single-kernel decode step.  See attn.hip for the design notes.
#pragma once

#include "select.h"

#include <math.h>

namespace kin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttnThreads = 256;  // standalone attention: 4 waves
constexpr int kStepThreads = 512;  // fused select + attention: 8 waves

struct AttnArgs {
    const void *q, *K, *V;
    const int32_t *idx;  // global kept-block list (standalone sparse attention)
    void *out;
    float *ws_o;   // [batch][hq][nsplit][128] unnormalised partial outputs
    float *ws_ml;  // [batch][hq][nsplit][2]   (running max in log2 units, sum)
    int hkv, gqa, t_cap, ctx_len, block, block_shift, nb, k, nsplit, n_chunks;
    float scale_log2;  // log2(e) / sqrt(head_dim)
    // variable lengths and paged caches (both null: every sequence holds
    // ctx_len tokens in a contiguous [pair][t_cap] cache)
    const int32_t *ctx_lens;  // [batch] tokens per sequence (clamped to [1, ctx_len])
    const int32_t *pages;     // [batch][max_pages] page of the pool per page_size tokens
    int page_shift, max_pages, num_pages;
    // shared prompts (share_n == 0: none): sequences b = p * share_n ..
    // p * share_n + share_n - 1 share prompt p, whose first prompt_len
    // tokens' K/V ([prompt][hkv][prompt_len][d]) and block summaries
    // ([prompt][hkv][prompt_len / block][d]) are stored once
    const void *Kp, *Vp, *Sp;
    int share_n, prompt_len, prompt_blocks;
};

// Where a pair's K/V live: one contiguous cache, a page pool, or a shared
// prompt's arrays followed by the pair's own cache.
enum CacheMode { kContig = 0, kPaged = 1, kShared = 2 };

// The (prompt, KV head) unit whose shared rows `pair` reads.
__device__ __forceinline__ int prompt_unit(const AttnArgs &a, int pair) {
    return (pair / a.hkv / a.share_n) * a.hkv + pair % a.hkv;
}

// This pair's arguments: its own context length, block count and chunk
// count when the sequences differ in length.
__device__ __forceinline__ AttnArgs for_pair(const AttnArgs &a, int pair) {
    AttnArgs p = a;
    if (a.ctx_lens) {
        const int L = min(max(a.ctx_lens[pair / a.hkv], 1), a.ctx_len);
        p.ctx_len = L;
        p.nb = (L + a.block - 1) >> a.block_shift;
        p.n_chunks = (min(a.k, p.nb) * a.block + kChunkBf16 - 1) / kChunkBf16;
    }
    return p;
}

// Row (in head_dim-element rows from the cache base) of token t of `pair`:
// [pair][t_cap] contiguous, or [page][hkv][page_size] through the page table
// (an entry outside the pool is clamped into it).
__device__ __forceinline__ int64_t token_row(const AttnArgs &a, int pair, int t) {
    if (!a.pages) return (int64_t)pair * a.t_cap + t;
    const int b = pair / a.hkv, g = pair % a.hkv;
    int page = a.pages[(size_t)b * a.max_pages + (t >> a.page_shift)];
    page = min(max(page, 0), a.num_pages - 1);
    return (((int64_t)page * a.hkv + g) << a.page_shift) + (t & ((1 << a.page_shift) - 1));
}

// Where the tokens of list positions p0 .. p0+15 (16 consecutive positions
// inside one block) live: run(p0, valid, t0) gives the K/V row (in
// head_dim-element rows from the cache base) of position p0's token and that
// token's index t0 in its sequence; the run's other tokens follow in the
// next rows.  valid = false if the slot is empty or past the list.  `safe`
// is a row that may always be read (for lanes whose token does not count).

// all tokens [0, ctx_len) of one pair, contiguous cache [pair][t_cap]
struct DenseRuns {
    static constexpr bool kPerToken = false;
    static constexpr bool kTwoBases = false;
    int64_t row0;  // the pair's first row
    int ctx_len;
    __device__ int64_t run(int p0, bool &valid, int &t0) const {
        valid = p0 < ctx_len;
        t0 = p0;
        return row0 + p0;
    }
    __device__ int64_t safe() const { return row0; }
};

// the kept blocks `sel` (global memory or LDS) of one pair, contiguous cache
struct ListRuns {
    static constexpr bool kPerToken = false;
    static constexpr bool kTwoBases = false;
    int64_t row0;
    const int32_t *sel;
    int k, nb, block, block_shift;
    __device__ int64_t run(int p0, bool &valid, int &t0) const {
        const int slot = p0 >> block_shift;
        const int id = slot < k ? sel[slot] : -1;
        valid = id >= 0 && id < nb;
        t0 = id * block + (p0 & (block - 1));
        return row0 + t0;
    }
    __device__ int64_t safe() const { return row0; }
};

// the kept blocks of one pair in a paged cache: selrow[slot] is the row of
// block sel[slot]'s first token (a block lies inside one page), or -1
struct PagedRuns {
    static constexpr bool kPerToken = false;
    static constexpr bool kTwoBases = false;
    const int32_t *sel;
    const int64_t *selrow;
    int64_t safe_row;
    int k, nb, block, block_shift;
    __device__ int64_t run(int p0, bool &valid, int &t0) const {
        const int slot = p0 >> block_shift;
        const int id = slot < k ? sel[slot] : -1;
        valid = id >= 0 && id < nb;
        const int off = p0 & (block - 1);
        t0 = id * block + off;
        return valid ? selrow[slot] + off : safe_row;
    }
    __device__ int64_t safe() const { return safe_row; }
};

// the kept tokens `sel` (one token per list position, token-level
// selection) of one pair, contiguous cache: every position has its own row
struct TokenRuns {
    static constexpr bool kPerToken = true;
    static constexpr bool kTwoBases = false;
    int64_t row0;
    const int32_t *sel;
    int k, ctx_len;
    __device__ int64_t row_of(int p, bool &valid) const {
        const int id = p < k ? sel[p] : -1;
        valid = id >= 0 && id < ctx_len;
        return valid ? row0 + id : row0;
    }
    __device__ int64_t safe() const { return row0; }
};

// the kept blocks of one pair whose first prompt_blocks blocks live in the
// prompt's shared arrays (Kp, Vp), the rest in the pair's own contiguous
// cache: run2() also says which of the two arrays the run is in
struct SharedRuns {
    static constexpr bool kPerToken = false;
    static constexpr bool kTwoBases = true;
    int64_t row0;   // the pair's own first row (in K, V)
    int64_t prow0;  // the prompt unit's first row (in Kp, Vp)
    const uint16_t *Kp, *Vp;
    const int32_t *sel;
    int k, nb, block, block_shift, prompt_blocks;
    __device__ int64_t run2(int p0, bool &valid, int &t0, bool &in_prompt) const {
        const int slot = p0 >> block_shift;
        const int id = slot < k ? sel[slot] : -1;
        valid = id >= 0 && id < nb;
        t0 = id * block + (p0 & (block - 1));
        in_prompt = valid && id < prompt_blocks;
        return (in_prompt ? prow0 : row0) + t0;
    }
    // rows that may always be read: the prompt's first row (the pair's own
    // first rows belong to the prompt and hold nothing)
    __device__ const uint16_t *safe_k() const { return Kp + prow0 * kHeadDim; }
    __device__ const uint16_t *safe_v() const { return Vp + prow0 * kHeadDim; }
};

// Launch order of the shared-prompt step: workgroup x runs on XCD x % 8, so
// the samples of one (prompt, KV head) unit are given consecutive slots of
// one XCD; the prompt rows they all read then come from that XCD's L2.
// Identity when the units do not spread evenly over the 8 XCDs.
__device__ __forceinline__ int shared_pair(const AttnArgs &a, int x, int pairs) {
    const int n = a.share_n;
    const int units = pairs / n;
    if (units % 8) return x;
    const int xcd = x & 7, slot = x >> 3;
    const int u = xcd + 8 * (slot / n), smp = slot % n;
    return ((u / a.hkv) * n + smp) * a.hkv + u % a.hkv;
}

// The newest block's mean-key summary row rebuilt by one wave from K and
// written to S ([pair][nb_cap] rows): fp64 sum in ascending token order,
// fp64 mean, fp32 then bf16 rounding, the arithmetic of the scoring phase's
// rebuild, so the row is bit for bit the one that path writes.  Lane l:
// channels 2l and 2l + 1.  `a` holds the pair's own length (for_pair).
__device__ inline void newest_row_bf16(const AttnArgs &a, void *S, int nb_cap, int pair,
                                       int lane) {
    const int jn = a.nb - 1;
    const int tn = min(a.block, a.ctx_len - jn * a.block);
    // the block lies inside one page: its rows are consecutive
    const uint32_t *k = static_cast<const uint32_t *>(a.K) +
                        token_row(a, pair, jn * a.block) * (kHeadDim / 2) + lane;
    double s0 = 0.0, s1 = 0.0;
#pragma unroll 16
    for (int t = 0; t < tn; ++t) {
        const uint32_t v = k[(size_t)t * (kHeadDim / 2)];
        s0 += (double)bf16_lo(v);
        s1 += (double)bf16_hi(v);
    }
    const double cnt = (double)tn;
    const float m0 = (float)(s0 / cnt), m1 = (float)(s1 / cnt);
    static_cast<uint32_t *>(S)[((size_t)pair * nb_cap + jn) * (kHeadDim / 2) + lane] =
        f32_to_bf16_bits(m0) | (f32_to_bf16_bits(m1) << 16);
}

// Launch order of a split launch (ns workgroups per pair, workgroup x =
// blockIdx.y * ns + blockIdx.x running on XCD x % 8): the ns splits of a
// pair are given slots of one XCD, so the pair's scores, which every split
// reads for its selection, are fetched into that XCD's L2 once rather than
// into ns of them (and the combine reads partials written on the same XCD).
// The pairs past the last multiple of 8 keep the plain order.
__device__ __forceinline__ void split_slot(int x, int ns, int pairs, int &pair, int &split) {
    const int full = pairs & ~7;
    if (x < full * ns) {
        const int slot = x >> 3;
        pair = (slot / ns) * 8 + (x & 7);
        split = slot % ns;
    } else {
        const int r = x - full * ns;
        pair = full + r / ns;
        split = r % ns;
    }
}

__device__ __forceinline__ SharedRuns shared_runs(const AttnArgs &a, int pair,
                                                  const int32_t *sel) {
    return SharedRuns{(int64_t)pair * a.t_cap, (int64_t)prompt_unit(a, pair) * a.prompt_len,
                      static_cast<const uint16_t *>(a.Kp), static_cast<const uint16_t *>(a.Vp),
                      sel, a.k, a.nb, a.block, a.block_shift, a.prompt_blocks};
}

// LDS the waves of one workgroup merge through: per wave, per head, the
// running max, running sum and unnormalised output.
template <int NW>
struct MergeLds {
    float o[NW][kMaxGqa][kHeadDim];
    float m[NW][kMaxGqa];
    float l[NW][kMaxGqa];
};

// Data handed between workgroups of one running kernel is written and read
// with agent-scope atomic accesses: the stores write through to the
// device-coherent level and the loads bypass the non-coherent caches, so
// the release / acquire of such a handoff reduce to the writer waiting for
// its stores to complete (stores_complete) before it signals.  This avoids
// the L2 writeback and invalidate of a full device-scope fence.
template <class T>
__device__ __forceinline__ void st_agent(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_agent(const T *p) {
    return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory access this wave issued has completed (the compiler fences
// keep the accesses on their side of the wait).
__device__ __forceinline__ void stores_complete() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Count an arrival at *ctr, a word that was zero when the launch began
// (cleared by an earlier kernel on the stream, or left at zero by the
// previous call's last arrival): one atomic round trip.
__device__ inline uint32_t arrive_add(uint64_t *ctr) {
    return (uint32_t)__hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) + 1u;
}

// Merge the NW waves' (m, l, o) of one workgroup in wave order and write the
// result (the output when nsplit == 1, else this split's partial; AGENT:
// the partial with agent-scope stores, for a combine in the same kernel).
// Uses the first 256 threads: 16 per head, 8 channels each.
template <int DT, int NW, bool AGENT = false>
__device__ void merge_waves_and_store(const AttnArgs &a, const MergeLds<NW> &sm, int pair,
                                      int split) {
    const int tid = threadIdx.x;
    const int h = tid >> 4;
    const int c0 = (tid & 15) * 8;
    if (tid >= 256 || h >= a.gqa) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][h]);
    float wt[NW];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wt[w] = (M == -INFINITY) ? 0.f : exp2f(sm.m[w][h] - M);
        L += wt[w] * sm.l[w][h];
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += wt[w] * sm.o[w][h][c0 + e];
        o[e] = acc;
    }
    const int b = pair / a.hkv, g = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const size_t row = (size_t)b * hq + (size_t)g * a.gqa + h;
    if (a.nsplit == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        if (DT == KIN_BF16) {
            u32x4 w4;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w4[e] = f32_to_bf16_bits(o[2 * e] * inv) | (f32_to_bf16_bits(o[2 * e + 1] * inv) << 16);
            *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(a.out) + row * kHeadDim + c0) = w4;
        } else {
            f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(a.out) + row * kHeadDim + c0);
            p[0] = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
            p[1] = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
        }
    } else {
        const size_t prow = row * a.nsplit + split;
        if (AGENT) {
            float *p = a.ws_o + prow * kHeadDim + c0;
#pragma unroll
            for (int e = 0; e < 8; ++e) st_agent(p + e, o[e]);
            if ((tid & 15) == 0) {
                st_agent(a.ws_ml + prow * 2 + 0, M);
                st_agent(a.ws_ml + prow * 2 + 1, L);
            }
        } else {
            f32x4 *p = reinterpret_cast<f32x4 *>(a.ws_o + prow * kHeadDim + c0);
            p[0] = f32x4{o[0], o[1], o[2], o[3]};
            p[1] = f32x4{o[4], o[5], o[6], o[7]};
            if ((tid & 15) == 0) {
                a.ws_ml[prow * 2 + 0] = M;
                a.ws_ml[prow * 2 + 1] = L;
            }
        }
    }
}

// LSE combine of the nsplit partials of one pair's query heads, read with
// agent-scope loads (written by other workgroups of the same kernel), 8
// splits per group with all of a group's loads issued together (one round
// trip per group): per group M' = max(M, m_s), the running sums rescaled by
// 2^(M - M'), then out = sum 2^(m_s - M) o_s / sum 2^(m_s - M) l_s, splits in
// ascending order.  Every thread of an NT-thread workgroup calls this.
template <int DT, int NT>
__device__ void combine_pair(const AttnArgs &a, int pair) {
    constexpr int kGroup = 8;
    const int b = pair / a.hkv, g = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    for (int i = threadIdx.x; i < a.gqa * (kHeadDim / 2); i += NT) {
        const int h = i / (kHeadDim / 2), c = 2 * (i % (kHeadDim / 2));
        const size_t row = (size_t)b * hq + (size_t)g * a.gqa + h;
        const float *ml = a.ws_ml + row * a.nsplit * 2;
        float M = -INFINITY, L = 0.f, o0 = 0.f, o1 = 0.f;
        for (int s0 = 0; s0 < a.nsplit; s0 += kGroup) {
            float m[kGroup], l[kGroup], x0[kGroup], x1[kGroup];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int s = min(s0 + u, a.nsplit - 1);  // repeats past the end are not used
                const float *po = a.ws_o + (row * a.nsplit + s) * kHeadDim + c;
                m[u] = ld_agent(ml + 2 * s);
                l[u] = ld_agent(ml + 2 * s + 1);
                x0[u] = ld_agent(po);
                x1[u] = ld_agent(po + 1);
            }
            float Mg = M;
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (s0 + u < a.nsplit) Mg = fmaxf(Mg, m[u]);
            const float r = (M == -INFINITY) ? 0.f : exp2f(M - Mg);
            L *= r;
            o0 *= r;
            o1 *= r;
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                if (s0 + u >= a.nsplit) continue;
                const float w = (Mg == -INFINITY) ? 0.f : exp2f(m[u] - Mg);
                L += w * l[u];
                o0 += w * x0[u];
                o1 += w * x1[u];
            }
            M = Mg;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        if (DT == KIN_BF16) {
            static_cast<uint32_t *>(a.out)[row * (kHeadDim / 2) + c / 2] =
                f32_to_bf16_bits(o0 * inv) | (f32_to_bf16_bits(o1 * inv) << 16);
        } else {
            reinterpret_cast<float2 *>(a.out)[row * (kHeadDim / 2) + c / 2] =
                make_float2(o0 * inv, o1 * inv);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16, MFMA
// ---------------------------------------------------------------------------

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-bit half `n & 1` of dword `n >> 1` of a and b, packed (a low, b high)
__device__ __forceinline__ uint32_t pick_pair(const u32x4 &a, const u32x4 &b, int n) {
    const uint32_t x = a[n >> 1], y = b[n >> 1];
    return (n & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
}

// The loads of one 32-token chunk held by one lane.
struct ChunkRegs {
    u32x4 k[2][4];  // K rows 16*tau + j, channels 32*kk + 8*g4 .. +8
    u32x4 v[8];     // V rows 16*tau + 4*g4 + r (e = 4*tau + r), channels 8j .. 8j+7
    uint32_t ok;    // bit e: token of V row e is a kept token inside the context
};

struct WaveState {
    f32x4 o[8];   // o[n][r]: head 4*g4 + r, channel 8*j + n
    float m_run;  // running max of head j (log2 units)
    float l_run;  // this lane's share of the running sum of head j
};

template <class Runs>
__device__ __forceinline__ void load_chunk(const AttnArgs &a, const Runs &runs, const uint16_t *K,
                                           const uint16_t *V, int c, int j, int g4,
                                           ChunkRegs &cr) {
    cr.ok = 0;
    if constexpr (Runs::kTwoBases) {
        // a run is in the prompt's arrays or in the pair's own cache
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            bool valid, pr;
            int t0;
            const int64_t row0 = runs.run2(c * kChunkBf16 + 16 * tau, valid, t0, pr);
            const uint16_t *Kb = pr ? runs.Kp : K;
            const uint16_t *Vb = pr ? runs.Vp : V;
            const bool okk = valid && t0 + j < a.ctx_len;
            const uint16_t *kr = okk ? Kb + (row0 + j) * kHeadDim : runs.safe_k();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) cr.k[tau][kk] = ld_nt16(kr + 32 * kk + 8 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int dv = 4 * g4 + r;
                const bool ok = valid && t0 + dv < a.ctx_len;
                cr.ok |= (ok ? 1u : 0u) << (4 * tau + r);
                const uint16_t *vr = ok ? Vb + (row0 + dv) * kHeadDim : runs.safe_v();
                cr.v[4 * tau + r] = ld_nt16(vr + 8 * j);
            }
        }
    } else if constexpr (Runs::kPerToken) {
        // K: row j of each 16-token tile; V: rows 4*g4 .. 4*g4+3
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            bool valid;
            const int64_t rowk = runs.row_of(c * kChunkBf16 + 16 * tau + j, valid);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                cr.k[tau][kk] = ld_nt16(K + rowk * kHeadDim + 32 * kk + 8 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bool ok;
                const int64_t rowv = runs.row_of(c * kChunkBf16 + 16 * tau + 4 * g4 + r, ok);
                cr.ok |= (ok ? 1u : 0u) << (4 * tau + r);
                cr.v[4 * tau + r] = ld_nt16(V + rowv * kHeadDim + 8 * j);
            }
        }
    } else {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            bool valid;
            int t0;
            const int64_t row0 = runs.run(c * kChunkBf16 + 16 * tau, valid, t0);
            const int64_t rowk = (valid && t0 + j < a.ctx_len) ? row0 + j : runs.safe();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                cr.k[tau][kk] = ld_nt16(K + rowk * kHeadDim + 32 * kk + 8 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int dv = 4 * g4 + r;
                const bool ok = valid && t0 + dv < a.ctx_len;
                cr.ok |= (ok ? 1u : 0u) << (4 * tau + r);
                cr.v[4 * tau + r] = ld_nt16(V + (ok ? row0 + dv : runs.safe()) * kHeadDim + 8 * j);
            }
        }
    }
}

__device__ __forceinline__ void compute_chunk(const ChunkRegs &cr, const bf16x8 (&qb)[4],
                                              float scale_log2, int g4, WaveState &st) {
    float s[8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cr.k[tau][kk]), qb[kk], acc,
                                                         0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s[4 * tau + r] = ((cr.ok >> (4 * tau + r)) & 1u) ? acc[r] * scale_log2 : -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(st.m_run - m_use);  // 0 while nothing was seen

    uint32_t pw[4];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t b0 = f32_to_bf16_bits(exp2f(s[2 * e] - m_use));
        const uint32_t b1 = f32_to_bf16_bits(exp2f(s[2 * e + 1] - m_use));
        psum += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
        pw[e] = b0 | (b1 << 16);
    }
    st.l_run = st.l_run * alpha + psum;
    st.m_run = m_new;

    // rescale O rows (heads 4*g4 + r) by their heads' alpha
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g4 + r);
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[n][r] *= ar;
    }
    const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const u32x4 vb = {pick_pair(cr.v[0], cr.v[1], n), pick_pair(cr.v[2], cr.v[3], n),
                          pick_pair(cr.v[4], cr.v[5], n), pick_pair(cr.v[6], cr.v[7], n)};
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(vb), st.o[n], 0, 0, 0);
    }
}

// One wave's share of a pair's chunks [c_beg, c_end), every `step`-th chunk
// starting at c_beg + first, then its (m, l, o) into merge slot `slot`.
// `runs` maps list positions to cache rows (DenseRuns, ListRuns, PagedRuns).
// PRE: when use_pre, the wave's first chunk is already loaded into pre (its
// loads may still be in flight).
template <class Runs, int NW, bool PRE = false>
__device__ void attend_bf16(const AttnArgs &a, const Runs &runs, int pair, int c_beg,
                            int c_end, int first, int step, int slot, MergeLds<NW> &sm,
                            const ChunkRegs *pre = nullptr, bool use_pre = false) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g4 = lane >> 4;
    const int b = pair / a.hkv, gk = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const uint16_t *Kp = static_cast<const uint16_t *>(a.K);
    const uint16_t *Vp = static_cast<const uint16_t *>(a.V);

    // B operand of S^T = K . Q^T: head j, channels 32*kk + 8*g4 .. +8
    bf16x8 qb[4];
    {
        const bool live = j < a.gqa;
        const uint16_t *qp = static_cast<const uint16_t *>(a.q) +
                             ((size_t)b * hq + (size_t)gk * a.gqa + (live ? j : 0)) * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            u32x4 v = *reinterpret_cast<const u32x4 *>(qp + 32 * kk + 8 * g4);
            if (!live) v = u32x4{0u, 0u, 0u, 0u};
            qb[kk] = as_bf16x8(v);
        }
    }
    WaveState st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    // two register buffers: chunk i computes while chunk i + 1 loads.  The
    // prefetch inside the loop is unconditional (the tail is peeled), so the
    // wait before a chunk's math covers only that chunk's loads.
    const int c0 = c_beg + first;
    const int n = c0 < c_end ? (c_end - c0 + step - 1) / step : 0;
    ChunkRegs ra, rb;
    if (n > 0) {
        if (PRE && use_pre)
            ra = *pre;
        else
            load_chunk(a, runs, Kp, Vp, c0, j, g4, ra);
        int i = 0;
        for (; i + 2 < n; i += 2) {
            load_chunk(a, runs, Kp, Vp, c0 + (i + 1) * step, j, g4, rb);
            compute_chunk(ra, qb, a.scale_log2, g4, st);
            load_chunk(a, runs, Kp, Vp, c0 + (i + 2) * step, j, g4, ra);
            compute_chunk(rb, qb, a.scale_log2, g4, st);
        }
        if (n - i == 2) {
            load_chunk(a, runs, Kp, Vp, c0 + (i + 1) * step, j, g4, rb);
            compute_chunk(ra, qb, a.scale_log2, g4, st);
            compute_chunk(rb, qb, a.scale_log2, g4, st);
        } else {
            compute_chunk(ra, qb, a.scale_log2, g4, st);
        }
    }

    float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (lane < 16) {
        sm.m[slot][lane] = st.m_run;
        sm.l[slot][lane] = l_tot;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n = 0; n < 8; ++n) sm.o[slot][4 * g4 + r][8 * j + n] = st.o[n][r];
}

__device__ __forceinline__ DenseRuns dense_runs(const AttnArgs &a, int pair) {
    return DenseRuns{(int64_t)pair * a.t_cap, a.ctx_len};
}
__device__ __forceinline__ ListRuns list_runs(const AttnArgs &a, int pair, const int32_t *sel) {
    return ListRuns{(int64_t)pair * a.t_cap, sel, a.k, a.nb, a.block, a.block_shift};
}

// Order LDS writes of one wave before its following LDS reads (the lanes of
// a wave run in lockstep and the LDS queue of a wave is in order; this only
// keeps the compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// fp32, MFMA (v_mfma_f32_16x16x4_f32), 16 tokens per chunk
// ---------------------------------------------------------------------------
//
// S^T[token][head] = K_tile . Q^T   32 MFMAs of 4 channels: k-step 4n + e
//                                   takes channel 16n + 4g + e, so lane (j, g)
//                                   (j = lane % 16, g = lane / 16) holds K row
//                                   j's channels 16n + 4g .. +3 as one 16 B
//                                   load per n (each instruction reads 64
//                                   contiguous bytes of 16 rows), and the
//                                   query the same channels of head j
// O[head][chan]   += P . V_tile     4 token k-steps x 8 column tiles: k-step
//                                   s, lane (j, g) supplies token 4g + s,
//                                   whose score (head j) it already holds in
//                                   row s of its S^T block, and the value
//                                   channels 8j .. 8j+7 of that token (column
//                                   j of tile n is channel 8j + n; 512
//                                   contiguous bytes per row)
// The weights stay fp32 (no rounding), the products are fp32 MFMAs with
// fp32 accumulation; every chunk's loads are issued while the previous
// chunk computes (two register buffers).

struct ChunkRegsF32 {
    f32x4 k[8];     // K row j of the tile, channels 16n + 4g .. +3
    f32x4 v[4][2];  // V row 4g + s, channels 8j .. 8j+3 and 8j+4 .. 8j+7
    uint32_t ok;    // bit s: the token of V row 4g + s is kept and inside the context
};

__device__ __forceinline__ f32x4 as_f32x4(u32x4 v) { return __builtin_bit_cast(f32x4, v); }

template <class Runs>
__device__ __forceinline__ void load_chunk_f32(const AttnArgs &a, const Runs &runs, const float *K,
                                               const float *V, int c, int j, int g,
                                               ChunkRegsF32 &cr) {
    static_assert(!Runs::kPerToken && !Runs::kTwoBases, "fp32: contiguous block lists");
    bool valid;
    int t0;
    const int64_t row0 = runs.run(c * kChunkF32, valid, t0);
    const int64_t rowk = (valid && t0 + j < a.ctx_len) ? row0 + j : runs.safe();
    const float *kr = K + rowk * kHeadDim + 4 * g;
#pragma unroll
    for (int n = 0; n < 8; ++n) cr.k[n] = as_f32x4(ld_nt16(kr + 16 * n));
    cr.ok = 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int dv = 4 * g + s;
        const bool ok = valid && t0 + dv < a.ctx_len;
        cr.ok |= (ok ? 1u : 0u) << s;
        const float *vr = V + (ok ? row0 + dv : runs.safe()) * kHeadDim + 8 * j;
        cr.v[s][0] = as_f32x4(ld_nt16(vr));
        cr.v[s][1] = as_f32x4(ld_nt16(vr + 4));
    }
}

__device__ __forceinline__ void compute_chunk_f32(const ChunkRegsF32 &cr, const f32x4 (&qf)[8],
                                                  float scale_log2, int g, WaveState &st) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(cr.k[n][e], qf[n][e], acc, 0, 0, 0);
    float s[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = ((cr.ok >> r) & 1u) ? acc[r] * scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(st.m_run - m_use);  // 0 while nothing was seen
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        p[r] = exp2f(s[r] - m_use);
        psum += p[r];
    }
    st.l_run = st.l_run * alpha + psum;
    st.m_run = m_new;
    // rescale O rows (heads 4g + r) by their heads' alpha
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[n][r] *= ar;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int n = 0; n < 8; ++n)
            st.o[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[t], cr.v[t][n >> 2][n & 3], st.o[n],
                                                          0, 0, 0);
}

// The B operand of the fp32 S^T = K . Q^T for this lane: head j = lane % 16
// (zero past the group), channels 16n + 4g .. +3, g = lane / 16.  Loaded by
// the kernels ahead of time, so its round trip overlaps earlier work.
__device__ __forceinline__ void load_q_f32(const AttnArgs &a, int pair, f32x4 (&qf)[8]) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g = lane >> 4;
    const int b = pair / a.hkv, gk = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const bool live = j < a.gqa;
    const float *qp = static_cast<const float *>(a.q) +
                      ((size_t)b * hq + (size_t)gk * a.gqa + (live ? j : 0)) * kHeadDim + 4 * g;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(qp + 16 * n);
        qf[n] = live ? v : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// One wave's share of a pair's chunks [c_beg, c_end), every `step`-th chunk
// starting at c_beg + first, then its (m, l, o) into merge slot `slot`
// (fp32; `runs` maps list positions to cache rows: DenseRuns, ListRuns;
// qf from load_q_f32).
template <class Runs, int NW>
__device__ void attend_f32(const AttnArgs &a, const Runs &runs, const f32x4 (&qf)[8], int c_beg,
                           int c_end, int first, int step, int slot, MergeLds<NW> &sm) {
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g = lane >> 4;
    const float *Kp = static_cast<const float *>(a.K);
    const float *Vp = static_cast<const float *>(a.V);
    WaveState st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m_run = -INFINITY;
    st.l_run = 0.f;

    // two register buffers: chunk i computes while chunk i + 1 loads (the
    // tail is peeled, so the loads inside the loop are unconditional)
    const int c0 = c_beg + first;
    const int n = c0 < c_end ? (c_end - c0 + step - 1) / step : 0;
    ChunkRegsF32 ra, rb;
    if (n > 0) {
        load_chunk_f32(a, runs, Kp, Vp, c0, j, g, ra);
        int i = 0;
        for (; i + 2 < n; i += 2) {
            load_chunk_f32(a, runs, Kp, Vp, c0 + (i + 1) * step, j, g, rb);
            compute_chunk_f32(ra, qf, a.scale_log2, g, st);
            load_chunk_f32(a, runs, Kp, Vp, c0 + (i + 2) * step, j, g, ra);
            compute_chunk_f32(rb, qf, a.scale_log2, g, st);
        }
        if (n - i == 2) {
            load_chunk_f32(a, runs, Kp, Vp, c0 + (i + 1) * step, j, g, rb);
            compute_chunk_f32(ra, qf, a.scale_log2, g, st);
            compute_chunk_f32(rb, qf, a.scale_log2, g, st);
        } else {
            compute_chunk_f32(ra, qf, a.scale_log2, g, st);
        }
    }

    float l_tot = st.l_run + __shfl_xor(st.l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (lane < 16) {
        sm.m[slot][lane] = st.m_run;
        sm.l[slot][lane] = l_tot;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n2 = 0; n2 < 8; ++n2) sm.o[slot][4 * g + r][8 * j + n2] = st.o[n2][r];
}

// Bytes of the split partials (o, then m and l) of one attention call.
inline size_t ws_for(const Geo &g, int ns) {
    return ns == 1 ? 0 : (size_t)g.batch * g.hq * ns * (kHeadDim + 2) * sizeof(float);
}

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Kernel arguments from a validated geometry and plan (host side).
inline void fill_args(AttnArgs &a, const Geo &g, const AttnPlan &p, const void *q, const void *K,
                      const void *V, const int32_t *idx, int k, void *out, void *ws) {
    a.q = q;
    a.K = K;
    a.V = V;
    a.idx = idx;
    a.out = out;
    // the partials follow the workspace's arrival words
    a.ws_o = reinterpret_cast<float *>(ws_body(ws));
    a.ws_ml = p.nsplit > 1 ? a.ws_o + (size_t)g.batch * g.hq * p.nsplit * kHeadDim : nullptr;
    a.hkv = g.hkv;
    a.gqa = g.gqa;
    a.t_cap = g.t_cap;
    a.ctx_len = g.ctx_len;
    a.block = g.block;
    a.block_shift = __builtin_ctz((unsigned)g.block);
    a.nb = g.nb;
    a.k = k;
    a.nsplit = p.nsplit;
    a.n_chunks = p.n_chunks;
    a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)kHeadDim));
    a.ctx_lens = g.ctx_lens;
    a.pages = g.pages;
    a.page_shift = g.page_shift;
    a.max_pages = g.max_pages;
    a.num_pages = g.num_pages;
    a.Kp = g.Kp;
    a.Vp = g.Vp;
    a.Sp = g.Sp;
    a.share_n = g.share_n;
    a.prompt_len = g.prompt_len;
    a.prompt_blocks = g.share_n ? g.prompt_len / g.block : 0;
}

}  // namespace kin
