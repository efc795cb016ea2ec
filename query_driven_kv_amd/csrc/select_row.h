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

// One 64-bit key per channel that orders channels as the selection does:
// the score's fp32 bits mapped to an unsigned order (negative scores below
// positive ones, -0 as +0) above the inverted channel index, so channel o is
// ahead of channel c exactly when key(o) > key(c) (score descending, ties to
// the lower channel).  D <= 256.
__device__ __forceinline__ unsigned long long select_key(float v, int c) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;                           // -0 ranks as +0
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)u << 8) | (unsigned long long)(255 - c);
}

// Thread groups that share the rank count of one channel: up to 16, whole
// 2-key blocks each.
__host__ __device__ constexpr int select_parts(int nth, int D) {
    int parts = nth / D;
    if (parts > 16) parts = 16;
    while (parts > 1 && D % (2 * parts) != 0) --parts;   // D is a multiple of 8
    return parts;
}

// Called by every thread of the workgroup (nth threads, a multiple of 64 and
// >= D); s[0..D) holds the scores in LDS.  scratch (>= nth ints) and cut (2
// floats) are LDS scratch.  DC and NTH, when nonzero, fix D and nth at
// compile time (the index arithmetic then folds; callers with D = 128 use
// it).  The rank of each channel under the total order is the number of
// channels ahead of it: every channel's key is written to LDS once, then each
// thread counts the keys above its own over a share of the channels (16-byte
// LDS loads of two keys, one 64-bit compare per key) and the partial counts
// are added in a fixed order.  Ranks form a permutation, so no sort is
// needed; the output slot of a kept channel (ascending order) comes from wave
// ballots and prefix popcounts.  mask_out (LDS, ceil(D/32) words, optional)
// receives the kept set as a bit mask, bit c of word c/32 for channel c.
// (Counting on the float scores with the channel tie-break, which compiled to
// lane-mask logic on the scalar unit, and with D and nth at run time took
// 1.8 us per call for 128 channels and 512 threads, measured in isolation;
// keys with D and nth fixed take 1.0 us.)
template <int DC = 0, int NTH = 0>
__device__ __forceinline__ void select_row(const float* s, int D_, int keep, int nth_, int* scratch,
                                           float* cut, int32_t* __restrict__ idx_out,
                                           int32_t* __restrict__ tie_out,
                                           uint32_t* mask_out = nullptr) {
    const int D = DC > 0 ? DC : D_;
    const int nth = NTH > 0 ? NTH : nth_;
    const int tid = threadIdx.x;
    const int parts = (DC > 0 && NTH > 0) ? select_parts(NTH, DC) : select_parts(nth, D);
    const int c = tid % D, part = tid / D;
    __shared__ int wave_kept[16];
    __shared__ __align__(16) unsigned long long keys[256];
    if (tid == 0) {
        cut[0] = 0.0f;
        cut[1] = 0.0f;
    }
    if (tid < D) keys[tid] = select_key(s[tid], tid);
    __syncthreads();
    if (part < parts) {
        const unsigned long long kc = keys[c];
        const int span = D / parts, o0 = part * span;
        int cnt = 0;
#pragma unroll 8
        for (int o = 0; o < span; o += 2) {
            const ulonglong2 y = *reinterpret_cast<const ulonglong2*>(keys + o0 + o);
            cnt += y.x > kc;
            cnt += y.y > kc;
        }
        scratch[part * D + c] = cnt;
    }
    __syncthreads();
    int rank = D;
    if (tid < D) {
        rank = 0;
#pragma unroll 4
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
