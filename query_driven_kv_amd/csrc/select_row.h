// select_row.h - the per-(b, kv head) channel selection shared by the
// stand-alone select kernel and the fused score-and-select kernel.
//
// "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework, second step: order the channels by relevance and
// prune the least relevant.  Order: score descending, ties to the lower
// channel; the kept channels are written in ascending channel order.
#pragma once

#include "think_common.h"

namespace thinkkv {

// Called by every thread of the workgroup (blockDim.x a multiple of 64 and
// >= D); s[0..D) holds the scores in LDS, 16-byte aligned.  scratch
// (>= blockDim.x ints) and cut (2 floats) are LDS scratch.  The rank of each
// channel under the total order is the number of channels ahead of it; the
// count is split over up to 16 thread groups of whole 4-channel blocks (read
// as one 16-byte LDS load each, so the reads pipeline) and their partial
// counts are added in a fixed order.  Ranks form a permutation, so no sort is
// needed; the output slot of a kept channel (ascending order) comes from wave
// ballots and prefix popcounts.  mask_out (LDS, ceil(D/32) words, optional)
// receives the kept set as a bit mask, bit c of word c/32 for channel c.
__device__ __forceinline__ void select_row(const float* s, int D, int keep, int* scratch,
                                           float* cut, int32_t* __restrict__ idx_out,
                                           int32_t* __restrict__ tie_out,
                                           uint32_t* mask_out = nullptr) {
    const int tid = threadIdx.x, nth = blockDim.x;
    int parts = nth / D;
    if (parts > 16) parts = 16;
    while (parts > 1 && D % (4 * parts) != 0) --parts;   // D is a multiple of 8
    const int c = tid % D, part = tid / D;
    __shared__ int wave_kept[16];
    if (tid == 0) {
        cut[0] = 0.0f;
        cut[1] = 0.0f;
    }
    if (part < parts) {
        const float x = s[c];
        const int o0 = part * (D / parts), o1 = o0 + D / parts;
        int cnt = 0;
#pragma unroll 4
        for (int o = o0; o < o1; o += 4) {
            const float4 y = *reinterpret_cast<const float4*>(s + o);
            cnt += (y.x > x) | ((y.x == x) & (o < c));
            cnt += (y.y > x) | ((y.y == x) & (o + 1 < c));
            cnt += (y.z > x) | ((y.z == x) & (o + 2 < c));
            cnt += (y.w > x) | ((y.w == x) & (o + 3 < c));
        }
        scratch[part * D + c] = cnt;
    }
    __syncthreads();
    int rank = D;
    if (tid < D) {
        rank = 0;
        for (int p = 0; p < parts; ++p) rank += scratch[p * D + tid];
        if (rank == keep - 1) cut[0] = s[tid];
        if (rank == keep) cut[1] = s[tid];
    }
    const bool take = rank < keep;
    const int lane = tid & 63, wave = tid >> 6;
    const unsigned long long m = __ballot(take);
    if (lane == 0 && wave < 16) wave_kept[wave] = __popcll(m);
    if (mask_out && lane == 0 && wave * 64 < D) {
        mask_out[2 * wave] = (uint32_t)m;
        if (wave * 64 + 32 < D) mask_out[2 * wave + 1] = (uint32_t)(m >> 32);
    }
    __syncthreads();
    if (take) {
        int pos = __popcll(m & ((1ull << lane) - 1ull));
        for (int w = 0; w < wave; ++w) pos += wave_kept[w];
        idx_out[pos] = tid;
    }
    if (tid == 0 && tie_out) {
        int flag = 0;
        if (keep < D) {
            const double hi = (double)cut[0], lo = (double)cut[1];
            flag = (hi - lo) <= 1e-5 * hi;
        }
        *tie_out = flag;
    }
}

}  // namespace thinkkv
