// topk.hip -- K3: the standalone top-k call, one 512-thread workgroup per
// (sequence, KV head) pair.  The selection itself is select_topk (select.h).
#include "select.h"

namespace kin {

constexpr int kTopkThreads = 512;

template <int KPT>
__global__ __launch_bounds__(kTopkThreads) void k_block_topk(const double *__restrict__ scores,
                                                             int32_t *__restrict__ idx,
                                                             int nb_cap, int nb, int k) {
    __shared__ SelectLds<KPT, kTopkThreads> lds;
    const size_t pair = blockIdx.x;
    select_clear(lds);
    __syncthreads();
    select_topk<KPT, kTopkThreads, false>(scores + pair * (size_t)nb_cap, nb, k, idx + pair * (size_t)k,
                                   lds);
}

hipError_t launch_block_topk(const Geo &g, const double *scores, int k, int32_t *idx,
                             hipStream_t s) {
    dim3 grid(g.pairs);
    switch (select_kpt(g.nb, kTopkThreads)) {
    case 1: k_block_topk<1><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    case 2: k_block_topk<2><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    case 4: k_block_topk<4><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    case 8: k_block_topk<8><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    case 16: k_block_topk<16><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    default: k_block_topk<32><<<grid, kTopkThreads, 0, s>>>(scores, idx, g.nb_cap, g.nb, k); break;
    }
    return hipGetLastError();
}

}  // namespace kin
