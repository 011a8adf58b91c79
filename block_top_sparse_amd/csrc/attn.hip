// attn.hip -- K4/K6: split-KV decode attention over a token list, and K5,
// the log-sum-exp combine of the splits.
//
// For every query head h of KV head g,
//     out_h = sum_t softmax_t(q_h . k_t / sqrt(d)) v_t
// over the tokens of the kept blocks (sparse, the attention step of
// BlockTopKAttention in the skill summary "Kinetics: Memory-Aware Test-Time
// Scaling", Implementation: everything outside the kept blocks is masked
// before the softmax, which equals leaving it out), or over every token in
// [0, ctx_len) (dense, the comparison of the rebuttal "Kinetics: Rethinking
// Test-Time Scaling Law", "W2 & Q2: Real-world latency benchmarks").
//
// A pair's token list is cut into fixed chunks; a workgroup (4 waves) takes
// a contiguous range of chunks ("split"), its waves take chunks round-robin
// and keep a running max / sum / output (online softmax, base 2).  The 4
// waves are merged through LDS; with more than one split per pair the
// workgroup writes an unnormalised partial (o, m, l) and K5 merges them.
//
// bf16 path (MFMA, gfx950 v_mfma_f32_16x16x32_bf16), 32 tokens per chunk:
//   S^T[token][head] = K_chunk . Q^T   two 16-token tiles x 4 k-steps of 32
//                                      channels; the GQA group (<= 16 heads)
//                                      fills the 16 columns, unused ones are 0
//   O[head][chan]   += P . V_chunk     8 MFMAs over 16-channel tiles
// Lane l (j = l % 16, g = l / 16) loads K rows of tokens 16*tau + j (16 B
// slices at channel 32*kk + 8*g) and V rows of tokens 16*tau + 4*g + r,
// r = 0..3, channels 8j..8j+7 -- every V load instruction reads 4 whole
// 256 B rows.  The MFMA output leaves lane l holding the scores of head j
// for exactly the tokens whose V rows it loaded, so P needs no data
// movement; V's 8x8 (token x channel) register block is transposed with
// 16-bit permutes into the B operand, and output column j of tile n is
// channel 8j + n.  Softmax weights enter the MFMA as bf16; the running sum
// uses the same rounded weights, so the weights still sum to one.
//
// fp32 path (VALU), 64 tokens per chunk: lane = token for q.k (each lane
// reads its key row), LDS holds the weights, lane = 2 channels for p.v.
#include "kin_internal.h"

#include <math.h>

namespace kin {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = 4;

struct AttnArgs {
    const void *q, *K, *V;
    const int32_t *idx;
    void *out;
    float *ws_o;   // [batch][hq][nsplit][128] unnormalised partial outputs
    float *ws_ml;  // [batch][hq][nsplit][2]   (running max in log2 units, sum)
    int hkv, gqa, t_cap, ctx_len, block, block_shift, nb, k, nsplit, n_chunks;
    float scale_log2;  // log2(e) / sqrt(head_dim)
};

// Resolve list position p0 .. p0+15 (16 consecutive positions inside one
// block) to the first token of that run; valid = false if the slot is
// empty or past the list.
template <bool DENSE>
__device__ __forceinline__ int run_base(const AttnArgs &a, const int32_t *sel, int p0,
                                        bool &valid) {
    if (DENSE) {
        valid = p0 < a.ctx_len;
        return p0;
    }
    const int slot = p0 >> a.block_shift;
    const int id = slot < a.k ? sel[slot] : -1;
    valid = id >= 0 && id < a.nb;
    return id * a.block + (p0 & (a.block - 1));
}

// Merge the 4 waves' (m, l, o) of one workgroup and write the result.
// sm_o[w][h][c], sm_m[w][h], sm_l[w][h] are filled by the caller.
template <int DT>
__device__ void merge_waves_and_store(const AttnArgs &a, float (*sm_o)[kMaxGqa][kHeadDim],
                                      float (*sm_m)[kMaxGqa], float (*sm_l)[kMaxGqa], int pair,
                                      int split) {
    const int tid = threadIdx.x;
    const int h = tid >> 4;          // 16 threads per head
    const int c0 = (tid & 15) * 8;   // 8 channels per thread
    if (h >= a.gqa) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float wt[kAttnWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) {
        wt[w] = (M == -INFINITY) ? 0.f : exp2f(sm_m[w][h] - M);
        L += wt[w] * sm_l[w][h];
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) acc += wt[w] * sm_o[w][h][c0 + e];
        o[e] = acc;
    }
    const int b = pair / a.hkv, g = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const size_t row = (size_t)b * hq + (size_t)g * a.gqa + h;
    if (a.nsplit == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        if (DT == KIN_BF16) {
            uint32_t w4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w4[e] = f32_to_bf16_bits(o[2 * e] * inv) | (f32_to_bf16_bits(o[2 * e + 1] * inv) << 16);
            *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + row * kHeadDim + c0) =
                make_uint4(w4[0], w4[1], w4[2], w4[3]);
        } else {
            float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(a.out) + row * kHeadDim + c0);
            p[0] = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
            p[1] = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
        }
    } else {
        const size_t prow = row * a.nsplit + split;
        float4 *p = reinterpret_cast<float4 *>(a.ws_o + prow * kHeadDim + c0);
        p[0] = make_float4(o[0], o[1], o[2], o[3]);
        p[1] = make_float4(o[4], o[5], o[6], o[7]);
        if ((tid & 15) == 0) {
            a.ws_ml[prow * 2 + 0] = M;
            a.ws_ml[prow * 2 + 1] = L;
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

template <bool DENSE>
__global__ __launch_bounds__(kAttnThreads, 2) void k_attn_bf16(AttnArgs a) {
    __shared__ float sm_o[kAttnWaves][kMaxGqa][kHeadDim];
    __shared__ float sm_m[kAttnWaves][kMaxGqa];
    __shared__ float sm_l[kAttnWaves][kMaxGqa];

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int j = lane & 15, g4 = lane >> 4;
    const int split = blockIdx.x, pair = blockIdx.y;
    const int b = pair / a.hkv, gk = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const uint16_t *Kp = static_cast<const uint16_t *>(a.K) + (size_t)pair * a.t_cap * kHeadDim;
    const uint16_t *Vp = static_cast<const uint16_t *>(a.V) + (size_t)pair * a.t_cap * kHeadDim;
    const int32_t *sel = DENSE ? nullptr : a.idx + (size_t)pair * a.k;

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

    f32x4 o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;  // running max of head j (log2 units)
    float l_run = 0.f;        // this lane's share of the running sum of head j

    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);

    for (int c = c_beg + wave; c < c_end; c += kAttnWaves) {
        u32x4 kr[2][4], vr[8];
        bool okv[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            bool valid;
            const int base = run_base<DENSE>(a, sel, c * kChunkBf16 + 16 * tau, valid);
            const int tk = base + j;
            const int rowk = (valid && tk < a.ctx_len) ? tk : 0;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                kr[tau][kk] = ld_stream16(Kp + (size_t)rowk * kHeadDim + 32 * kk + 8 * g4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int tv = base + 4 * g4 + r;
                okv[4 * tau + r] = valid && tv < a.ctx_len;
                const int rowv = okv[4 * tau + r] ? tv : 0;
                vr[4 * tau + r] = ld_stream16(Vp + (size_t)rowv * kHeadDim + 8 * j);
            }
        }

        // scores: lane holds head j, tokens 16*tau + 4*g4 + r
        float s[8];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[tau][kk]), qb[kk], acc,
                                                             0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                s[4 * tau + r] = okv[4 * tau + r] ? acc[r] * a.scale_log2 : -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);  // 0 while nothing was seen

        uint32_t pw[4];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t b0 = f32_to_bf16_bits(exp2f(s[2 * e] - m_use));
            const uint32_t b1 = f32_to_bf16_bits(exp2f(s[2 * e + 1] - m_use));
            psum += __uint_as_float(b0 << 16) + __uint_as_float(b1 << 16);
            pw[e] = b0 | (b1 << 16);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // rescale O rows (heads 4*g4 + r) by their heads' alpha
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ar = __shfl(alpha, 4 * g4 + r);
#pragma unroll
            for (int n = 0; n < 8; ++n) o[n][r] *= ar;
        }
        const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const u32x4 vb = {pick_pair(vr[0], vr[1], n), pick_pair(vr[2], vr[3], n),
                              pick_pair(vr[4], vr[5], n), pick_pair(vr[6], vr[7], n)};
            o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, as_bf16x8(vb), o[n], 0, 0, 0);
        }
    }

    // per-wave results to LDS
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    if (lane < 16) {
        sm_m[wave][lane] = m_run;
        sm_l[wave][lane] = l_tot;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int n = 0; n < 8; ++n) sm_o[wave][4 * g4 + r][8 * j + n] = o[n][r];
    __syncthreads();
    merge_waves_and_store<KIN_BF16>(a, sm_o, sm_m, sm_l, pair, split);
}

// ---------------------------------------------------------------------------
// fp32, VALU
// ---------------------------------------------------------------------------

// Order LDS writes of one wave before its following LDS reads (the lanes of
// a wave run in lockstep and the LDS queue of a wave is in order; this only
// keeps the compiler from moving accesses across the point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool DENSE>
__global__ __launch_bounds__(kAttnThreads) void k_attn_f32(AttnArgs a) {
    __shared__ float sm_o[kAttnWaves][kMaxGqa][kHeadDim];
    __shared__ float sm_m[kAttnWaves][kMaxGqa];
    __shared__ float sm_l[kAttnWaves][kMaxGqa];
    __shared__ float sm_q[kMaxGqa][kHeadDim];
    __shared__ float sm_p[kAttnWaves][kMaxGqa][kChunkF32];
    __shared__ int sm_row[kAttnWaves][kChunkF32];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int split = blockIdx.x, pair = blockIdx.y;
    const int b = pair / a.hkv, gk = pair % a.hkv;
    const int hq = a.hkv * a.gqa;
    const int G = a.gqa;
    const float *Kp = static_cast<const float *>(a.K) + (size_t)pair * a.t_cap * kHeadDim;
    const float *Vp = static_cast<const float *>(a.V) + (size_t)pair * a.t_cap * kHeadDim;
    const int32_t *sel = DENSE ? nullptr : a.idx + (size_t)pair * a.k;

    for (int i = tid; i < kMaxGqa * kHeadDim; i += kAttnThreads) {
        const int h = i / kHeadDim, c = i % kHeadDim;
        sm_q[h][c] = h < G ? static_cast<const float *>(a.q)[((size_t)b * hq + gk * G + h) *
                                                              kHeadDim + c]
                           : 0.f;
    }
    __syncthreads();

    float m_run[kMaxGqa], l_run[kMaxGqa], o0[kMaxGqa], o1[kMaxGqa];
#pragma unroll
    for (int h = 0; h < kMaxGqa; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
        o0[h] = 0.f;
        o1[h] = 0.f;
    }

    const int cps = (a.n_chunks + a.nsplit - 1) / a.nsplit;
    const int c_beg = split * cps;
    const int c_end = min(a.n_chunks, c_beg + cps);

    for (int c = c_beg + wave; c < c_end; c += kAttnWaves) {
        // this lane's token: list position c*64 + lane
        const int p = c * kChunkF32 + lane;
        bool ok;
        int tok;
        if (DENSE) {
            tok = p;
            ok = p < a.ctx_len;
        } else {
            const int slot = p >> a.block_shift;
            const int id = slot < a.k ? sel[slot] : -1;
            tok = id * a.block + (p & (a.block - 1));
            ok = id >= 0 && id < a.nb && tok < a.ctx_len;
        }
        const int row = ok ? tok : 0;
        sm_row[wave][lane] = row;

        float s[kMaxGqa];
#pragma unroll
        for (int h = 0; h < kMaxGqa; ++h) s[h] = 0.f;
        const float4 *kr = reinterpret_cast<const float4 *>(Kp + (size_t)row * kHeadDim);
        for (int c4 = 0; c4 < kHeadDim / 4; ++c4) {
            const float4 kv = kr[c4];
#pragma unroll
            for (int h = 0; h < kMaxGqa; ++h) {
                if (h < G) {
                    s[h] = fmaf(sm_q[h][4 * c4 + 0], kv.x, s[h]);
                    s[h] = fmaf(sm_q[h][4 * c4 + 1], kv.y, s[h]);
                    s[h] = fmaf(sm_q[h][4 * c4 + 2], kv.z, s[h]);
                    s[h] = fmaf(sm_q[h][4 * c4 + 3], kv.w, s[h]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxGqa; ++h) {
            if (h >= G) continue;
            const float z = ok ? s[h] * a.scale_log2 : -INFINITY;
            float mx = z;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
            const float m_new = fmaxf(m_run[h], mx);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = exp2f(m_run[h] - m_use);
            const float pz = exp2f(z - m_use);
            l_run[h] = l_run[h] * alpha + pz;
            o0[h] *= alpha;
            o1[h] *= alpha;
            m_run[h] = m_new;
            sm_p[wave][h][lane] = pz;
        }
        wave_lds_sync();  // sm_p / sm_row rows of this wave are complete
        // p . v: lane owns channels 2*lane, 2*lane+1
        for (int t = 0; t < kChunkF32; ++t) {
            const float2 v =
                reinterpret_cast<const float2 *>(Vp + (size_t)sm_row[wave][t] * kHeadDim)[lane];
#pragma unroll
            for (int h = 0; h < kMaxGqa; ++h) {
                if (h < G) {
                    const float pt = sm_p[wave][h][t];
                    o0[h] = fmaf(pt, v.x, o0[h]);
                    o1[h] = fmaf(pt, v.y, o1[h]);
                }
            }
        }
        wave_lds_sync();  // every lane is done reading before the next chunk writes
    }

#pragma unroll
    for (int h = 0; h < kMaxGqa; ++h) {
        if (h >= G) continue;
        float l = l_run[h];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) l += __shfl_xor(l, d);
        if (lane == 0) {
            sm_m[wave][h] = m_run[h];
            sm_l[wave][h] = l;
        }
        sm_o[wave][h][2 * lane] = o0[h];
        sm_o[wave][h][2 * lane + 1] = o1[h];
    }
    __syncthreads();
    merge_waves_and_store<KIN_F32>(a, sm_o, sm_m, sm_l, pair, split);
}

// ---------------------------------------------------------------------------
// K5: combine the splits of each (sequence, query head)
// ---------------------------------------------------------------------------

template <int DT>
__global__ __launch_bounds__(64) void k_combine(const float *__restrict__ ws_o,
                                                const float *__restrict__ ws_ml,
                                                void *__restrict__ out, int nsplit) {
    const size_t row = blockIdx.x;  // b * hq + h
    const int lane = threadIdx.x;   // channels 2*lane, 2*lane+1
    const float *ml = ws_ml + row * nsplit * 2;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float w = (M == -INFINITY) ? 0.f : exp2f(ml[2 * s] - M);
        L += w * ml[2 * s + 1];
        const float2 v = reinterpret_cast<const float2 *>(ws_o + (row * nsplit + s) * kHeadDim)[lane];
        o0 += w * v.x;
        o1 += w * v.y;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (DT == KIN_BF16) {
        static_cast<uint32_t *>(out)[row * (kHeadDim / 2) + lane] =
            f32_to_bf16_bits(o0 * inv) | (f32_to_bf16_bits(o1 * inv) << 16);
    } else {
        reinterpret_cast<float2 *>(out)[row * (kHeadDim / 2) + lane] = make_float2(o0 * inv, o1 * inv);
    }
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

AttnPlan plan_attention(const Geo &g, int k, bool dense, int num_cu) {
    AttnPlan p;
    const int keff = dense ? 0 : (k < g.nb ? k : g.nb);
    p.n_tokens = dense ? g.ctx_len : keff * g.block;
    const int chunk = g.dtype == KIN_BF16 ? kChunkBf16 : kChunkF32;
    p.n_chunks = (p.n_tokens + chunk - 1) / chunk;
    // aim for ~2 workgroups per CU, but give every wave at least one chunk
    const int target = 2 * (num_cu > 0 ? num_cu : 256);
    int ns = (target + g.pairs - 1) / g.pairs;
    const int max_ns = p.n_chunks / kAttnWaves;
    if (ns > max_ns) ns = max_ns;
    if (ns > 64) ns = 64;
    if (ns < 1) ns = 1;
    p.nsplit = ns;
    p.ws_bytes = ns == 1 ? 0
                         : (size_t)g.batch * g.hq * ns * (kHeadDim + 2) * sizeof(float);
    return p;
}

hipError_t launch_attention(const Geo &g, const AttnPlan &p, const void *q, const void *K,
                            const void *V, const int32_t *idx, int k, void *out, void *ws,
                            hipStream_t s) {
    AttnArgs a;
    a.q = q;
    a.K = K;
    a.V = V;
    a.idx = idx;
    a.out = out;
    a.ws_o = static_cast<float *>(ws);
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
    const bool dense = idx == nullptr;
    dim3 grid(p.nsplit, g.pairs);
    if (g.dtype == KIN_BF16) {
        if (dense)
            k_attn_bf16<true><<<grid, kAttnThreads, 0, s>>>(a);
        else
            k_attn_bf16<false><<<grid, kAttnThreads, 0, s>>>(a);
    } else {
        if (dense)
            k_attn_f32<true><<<grid, kAttnThreads, 0, s>>>(a);
        else
            k_attn_f32<false><<<grid, kAttnThreads, 0, s>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    if (g.dtype == KIN_BF16)
        k_combine<KIN_BF16><<<g.batch * g.hq, 64, 0, s>>>(a.ws_o, a.ws_ml, out, p.nsplit);
    else
        k_combine<KIN_F32><<<g.batch * g.hq, 64, 0, s>>>(a.ws_o, a.ws_ml, out, p.nsplit);
    return hipGetLastError();
}

}  // namespace kin
