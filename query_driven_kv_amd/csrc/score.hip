// score.hip - stage (a): per-channel relevance of the key cache.
//
// "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework (first step) and Key design (1).  Reading: channel c's
// score is the Frobenius norm of its rank-1 logit term Q_w[:,c] K[:,c]^T,
// i.e. ||K[:,c]|| * sum over the group's query heads of ||Q_w[:,c]||.
//
// Two kernels:
//   k_score_partial   streams K once.  A workgroup owns a token range and a
//                     group of <= 256 16-byte column vectors of the token row
//                     (all kv heads side by side), so every load is a
//                     coalesced dwordx4 and each lane keeps the per-channel
//                     sums of its vector in registers across tokens.  Squares
//                     are summed in fp32 runs of <= 16 tokens, runs in fp64;
//                     the workgroup's row-interleaved lanes are reduced in LDS
//                     in a fixed order and written as one fp32 partial per
//                     (split, channel).
//   k_score_finalize  one workgroup per (b, kv): sums the splits in fp64 in a
//                     fixed order, forms the window-query norms and the score.
// No atomics: results are bitwise reproducible.
#include "think_common.h"

namespace thinkkv {
namespace {

constexpr int kThreads = 256;
constexpr int kRun = 16;   // tokens per fp32 run before folding into fp64

template <int DT>
__global__ __launch_bounds__(kThreads) void k_score_partial(
        const uint4* __restrict__ k_vec, const int32_t* __restrict__ seq_lens, int s_cap,
        int nvec, int tpw, int nsplit, float* __restrict__ partials) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const int split = blockIdx.x, cg = blockIdx.y, b = blockIdx.z;
    const int len = clamp_len(seq_lens, b, s_cap);
    const int t0 = split * tpw;
    if (t0 >= len) return;                       // finalize never reads this split
    const int t1 = min(t0 + tpw, len);

    const int v0 = cg * kThreads;
    const int nvg = min(kThreads, nvec - v0);    // vectors in this column group
    const int rpi = kThreads / nvg;              // token rows covered per step
    const int tid = threadIdx.x;
    const bool active = tid < rpi * nvg;
    const int col = active ? tid % nvg : 0;
    const int rsub = active ? tid / nvg : 0;

    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;

    if (active) {
        const uint4* base = k_vec + (size_t)b * s_cap * nvec + v0 + col;
        for (int t = t0 + rsub; t < t1; t += kRun * rpi) {
            uint4 v[kRun];
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                const int tt = t + u * rpi;
                v[u] = tt < t1 ? ldg_stream(base + (size_t)tt * nvec) : make_uint4(0u, 0u, 0u, 0u);
            }
            float run[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) run[e] = 0.0f;
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                float x[EPV];
                unpack(v[u], x, E{});
#pragma unroll
                for (int e = 0; e < EPV; ++e) run[e] = fmaf(x[e], x[e], run[e]);
            }
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] += (double)run[e];
        }
    }

    __shared__ double red[kThreads * 8];
    if (active) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) red[(rsub * nvg + col) * EPV + e] = acc[e];
    }
    __syncthreads();
    const int R = nvec * EPV;                    // channels per token row (Hkv*D)
    float* out = partials + ((size_t)b * nsplit + split) * R + (size_t)v0 * EPV;
    for (int o = tid; o < nvg * EPV; o += kThreads) {
        double s = 0.0;
        for (int r = 0; r < rpi; ++r) s += red[r * nvg * EPV + o];
        out[o] = (float)s;
    }
}

template <int DT>
__global__ __launch_bounds__(1024) void k_score_finalize(
        const float* __restrict__ partials, const int32_t* __restrict__ seq_lens, int s_cap,
        int tpw, int nsplit, const typename Elem<DT>::T* __restrict__ q_obs, int W, int Hq,
        int Hkv, int D, int sg_count, float* __restrict__ scores) {
    using E = Elem<DT>;
    const int kv = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x;
    const int c = tid % D, sg = tid / D;
    const int G = Hq / Hkv;
    const int len = clamp_len(seq_lens, b, s_cap);
    const int ns = (len + tpw - 1) / tpw;
    const int R = Hkv * D;

    // Sub-group sg sums splits sg, sg+SG, sg+2SG, ... into four interleaved
    // fp64 accumulators (independent loads), combined in a fixed order.
    const float* p = partials + (size_t)b * nsplit * R + (size_t)kv * D + c;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int s = sg;
    for (; s + 3 * sg_count < ns; s += 4 * sg_count) {
        a0 += (double)p[(size_t)s * R];
        a1 += (double)p[(size_t)(s + sg_count) * R];
        a2 += (double)p[(size_t)(s + 2 * sg_count) * R];
        a3 += (double)p[(size_t)(s + 3 * sg_count) * R];
    }
    for (; s < ns; s += sg_count) a0 += (double)p[(size_t)s * R];
    const double k2 = (a0 + a1) + (a2 + a3);

    __shared__ double kred[1024];
    __shared__ double qn[16 * 256];
    kred[tid] = k2;
    for (int g = sg; g < G; g += sg_count) {
        const int h = kv * G + g;
        double q2 = 0.0;
        for (int i = 0; i < W; ++i) {
            const double x = E::load(q_obs, (((size_t)b * W + i) * Hq + h) * D + c);
            q2 += x * x;
        }
        qn[g * D + c] = sqrt(q2);
    }
    __syncthreads();
    if (sg == 0) {
        double K2 = 0.0;
        for (int r = 0; r < sg_count; ++r) K2 += kred[r * D + c];
        double qsum = 0.0;
        for (int g = 0; g < G; ++g) qsum += qn[g * D + c];
        scores[((size_t)b * Hkv + kv) * D + c] = (float)(sqrt(K2) * qsum);
    }
}

}  // namespace

ScoreGeom score_geom(const think_dims& d) {
    ScoreGeom g{};
    const int e = elem_bytes(d.dtype);
    g.nvec = d.n_kv_heads * d.head_dim * e / 16;
    g.ncg = (g.nvec + kThreads - 1) / kThreads;
    // aim for ~512 workgroups (two per CU); tokens per workgroup a multiple of 16
    const int64_t rows = (int64_t)d.seq_capacity * d.batch * g.ncg;
    int64_t tpw = (rows + 511) / 512;
    tpw = (tpw + 15) / 16 * 16;
    if (tpw < 16) tpw = 16;
    if (tpw > 4096) tpw = 4096;
    g.tpw = (int)tpw;
    g.nsplit = (int)((d.seq_capacity + tpw - 1) / tpw);
    g.ws_bytes = (size_t)d.batch * g.nsplit * d.n_kv_heads * d.head_dim * sizeof(float);
    return g;
}

hipError_t launch_score(const think_dims& d, const ScoreGeom& g, const void* k_cache,
                        const int32_t* seq_lens, const void* q_obs, int W, float* scores,
                        float* partials, hipStream_t s) {
    dim3 grid1(g.nsplit, g.ncg, d.batch);
    int sg_count = 1024 / d.head_dim;
    if (sg_count > 8) sg_count = 8;
    dim3 grid2(d.n_kv_heads, d.batch);
    if (d.dtype == THINK_BF16) {
        k_score_partial<THINK_BF16><<<grid1, kThreads, 0, s>>>(
            (const uint4*)k_cache, seq_lens, d.seq_capacity, g.nvec, g.tpw, g.nsplit, partials);
        k_score_finalize<THINK_BF16><<<grid2, d.head_dim * sg_count, 0, s>>>(
            partials, seq_lens, d.seq_capacity, g.tpw, g.nsplit, (const uint16_t*)q_obs, W,
            d.n_q_heads, d.n_kv_heads, d.head_dim, sg_count, scores);
    } else {
        k_score_partial<THINK_F32><<<grid1, kThreads, 0, s>>>(
            (const uint4*)k_cache, seq_lens, d.seq_capacity, g.nvec, g.tpw, g.nsplit, partials);
        k_score_finalize<THINK_F32><<<grid2, d.head_dim * sg_count, 0, s>>>(
            partials, seq_lens, d.seq_capacity, g.tpw, g.nsplit, (const float*)q_obs, W,
            d.n_q_heads, d.n_kv_heads, d.head_dim, sg_count, scores);
    }
    return hipGetLastError();
}

}  // namespace thinkkv
