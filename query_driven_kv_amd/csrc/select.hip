// select.hip - stage (b): keep the `keep` highest-scoring channels per
// (b, kv head) ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method
// details -> Technical framework, second step: order channels by relevance
// and prune the least relevant ones).
//
// One workgroup per (b, kv).  With D <= 256 the whole score row sits in LDS
// and each lane computes the rank of its channel under the total order
// (score descending, channel ascending) by counting; rank < keep is kept.
// Ranks are a permutation, so no sort is needed, ties resolve to the lower
// channel exactly, and the output slot of a kept channel is the number of
// kept channels below it (ascending order).  The keep-th and (keep+1)-th
// scores give the near-tie flag, evaluated in fp64.
#include "think_common.h"

namespace thinkkv {
namespace {

__global__ __launch_bounds__(256) void k_select(const float* __restrict__ scores, int D, int keep,
                                                int32_t* __restrict__ kept_idx,
                                                int32_t* __restrict__ near_tie) {
    const int kv = blockIdx.x, b = blockIdx.y, Hkv = gridDim.x;
    const int c = threadIdx.x;
    __shared__ float s[256];
    __shared__ int kept[256];
    __shared__ float cut[2];
    const size_t row = (size_t)b * Hkv + kv;
    if (c < D) s[c] = scores[row * D + c];
    if (c == 0) { cut[0] = 0.0f; cut[1] = 0.0f; }
    __syncthreads();
    int rank = D;
    if (c < D) {
        const float x = s[c];
        rank = 0;
        for (int o = 0; o < D; ++o) {
            const float y = s[o];
            rank += (y > x) | ((y == x) & (o < c));
        }
    }
    const bool take = rank < keep;
    kept[c] = take;
    if (c < D && rank == keep - 1) cut[0] = s[c];
    if (c < D && rank == keep) cut[1] = s[c];
    __syncthreads();
    if (take) {
        int pos = 0;
        for (int o = 0; o < c; ++o) pos += kept[o];
        kept_idx[row * keep + pos] = c;
    }
    if (c == 0 && near_tie) {
        int flag = 0;
        if (keep < D) {
            const double hi = (double)cut[0], lo = (double)cut[1];
            flag = (hi - lo) <= 1e-5 * hi;
        }
        near_tie[row] = flag;
    }
}

}  // namespace

hipError_t launch_select(const think_dims& d, const float* scores, int keep, int32_t* kept_idx,
                         int32_t* near_tie, hipStream_t s) {
    dim3 grid(d.n_kv_heads, d.batch);
    k_select<<<grid, 256, 0, s>>>(scores, d.head_dim, keep, kept_idx, near_tie);
    return hipGetLastError();
}

}  // namespace thinkkv
