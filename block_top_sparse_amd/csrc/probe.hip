// probe.hip -- a measurement helper, not a step of the method: a plain
// streaming read of a device buffer, to measure the read bandwidth this
// device reaches.  The decode step's achieved bytes per second are quoted
// against it as well as against the published peak.
//
// The access pattern is the one the decode step's scoring scan streams
// with: one 8-wave workgroup per CU reads a contiguous tile of the buffer;
// the waves take consecutive 4 KiB batches (a wave's 4 loads of one batch
// are each 64 lanes x 16 bytes, 1 KiB consecutive), and every wave keeps a
// ring of 4 batches in flight, refilling a slot right after folding it.
// Loads past the tile re-read its last word and are not folded.  The words
// are XOR-folded per thread, per wave, and into the caller's 16-byte sink
// with one atomic per wave, so the loads are live and the sink receives
// the XOR of the whole buffer (every word read exactly once).
#include "kin_internal.h"

namespace kin {

constexpr int kProbeWaves = 8;
constexpr int kProbeRing = 4;
constexpr int kProbeBatch = 256;  // 16-byte words per batch (4 KiB)

__global__ __launch_bounds__(kProbeWaves * 64) void k_read_probe(const u32x4 *__restrict__ buf,
                                                                 size_t n16, size_t tile16,
                                                                 uint32_t *sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const size_t beg = (size_t)blockIdx.x * tile16;
    const size_t end = beg + tile16 < n16 ? beg + tile16 : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    if (beg < end) {
        const long nbat = (long)((end - beg + kProbeBatch - 1) / kProbeBatch);
        const long mine = wave < nbat ? (nbat - wave + kProbeWaves - 1) / kProbeWaves : 0;
        // word u of this lane in the wave's i-th batch (clamped inside the tile)
        auto word = [&](long i, int u) {
            const size_t x = beg + (size_t)(wave + i * kProbeWaves) * kProbeBatch + lane + 64 * u;
            return x < end ? x : end - 1;
        };
        u32x4 w[kProbeRing][4];
#pragma unroll
        for (int r = 0; r < kProbeRing; ++r)
#pragma unroll
            for (int u = 0; u < 4; ++u) w[r][u] = ld_nt16(buf + word(r, u));
        for (long i0 = 0; i0 < mine; i0 += kProbeRing) {
#pragma unroll
            for (int r = 0; r < kProbeRing; ++r) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const size_t x =
                        beg + (size_t)(wave + (i0 + r) * kProbeWaves) * kProbeBatch + lane + 64 * u;
                    const bool live = i0 + r < mine && x < end;
                    acc ^= live ? w[r][u] : u32x4{0u, 0u, 0u, 0u};
                    w[r][u] = ld_nt16(buf + word(i0 + r + kProbeRing, u));
                }
            }
        }
        // the last refills are read after the loop, so the compiler keeps
        // them unconditional (every wait then covers exactly one slot)
#pragma unroll
        for (int r = 0; r < kProbeRing; ++r)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                asm volatile("" ::"v"(w[r][u][0]), "v"(w[r][u][1]), "v"(w[r][u][2]),
                             "v"(w[r][u][3]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] ^= (uint32_t)__shfl_xor((int)acc[e], off);
    if (lane == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicXor(sink + e, acc[e]);
}

hipError_t launch_read_probe(const void *buf, size_t bytes, void *sink, int num_cu,
                             hipStream_t s) {
    const size_t n16 = bytes / 16;
    const size_t cu = (size_t)(num_cu > 0 ? num_cu : 256);
    // one tile per CU, whole batches
    size_t tile16 = (n16 + cu - 1) / cu;
    tile16 = (tile16 + kProbeBatch - 1) / kProbeBatch * kProbeBatch;
    const unsigned grid = (unsigned)((n16 + tile16 - 1) / tile16);
    k_read_probe<<<grid, kProbeWaves * 64, 0, s>>>(static_cast<const u32x4 *>(buf), n16, tile16,
                                                     static_cast<uint32_t *>(sink));
    return hipGetLastError();
}

}  // namespace kin
