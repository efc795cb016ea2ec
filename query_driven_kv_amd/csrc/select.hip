// select.hip - stage (b): keep the `keep` highest-scoring channels per
// (b, kv head) ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method
// details -> Technical framework, second step: order channels by relevance
// and prune the least relevant ones).
//
// One workgroup per (b, kv); the rank-count selection itself (select_row.h)
// is shared with the fused score-and-select kernel.  The keep-th and
// (keep+1)-th scores give the near-tie flag, evaluated in fp64.
#include "select_row.h"

namespace thinkkv {
namespace {

constexpr int kSelectThreads = 256;

__global__ __launch_bounds__(kSelectThreads) void k_select(const float* __restrict__ scores,
                                                           int D, int keep,
                                                           int32_t* __restrict__ kept_idx,
                                                           int32_t* __restrict__ near_tie) {
    const int kv = blockIdx.x, b = blockIdx.y, Hkv = gridDim.x;
    __shared__ __align__(16) float s[256];
    __shared__ int scratch[kSelectThreads];
    __shared__ float cut[2];
    const size_t row = (size_t)b * Hkv + kv;
    if (threadIdx.x < D) s[threadIdx.x] = scores[row * D + threadIdx.x];
    __syncthreads();
    int32_t* const tie = near_tie ? near_tie + row : nullptr;
    if (D == 128)
        select_row<128, kSelectThreads>(s, D, keep, kSelectThreads, scratch, cut,
                                        kept_idx + row * keep, tie);
    else
        select_row<0, kSelectThreads>(s, D, keep, kSelectThreads, scratch, cut,
                                      kept_idx + row * keep, tie);
}

}  // namespace

hipError_t launch_select(const think_dims& d, const float* scores, int keep, int32_t* kept_idx,
                         int32_t* near_tie, hipStream_t s) {
    dim3 grid(d.n_kv_heads, d.batch);
    k_select<<<grid, kSelectThreads, 0, s>>>(scores, d.head_dim, keep, kept_idx, near_tie);
    return hipGetLastError();
}

}  // namespace thinkkv
