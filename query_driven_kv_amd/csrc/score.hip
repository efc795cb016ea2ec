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
//                     (split, channel).  When the key cache is small enough
//                     for the last-level cache (the 256 MB Infinity Cache,
//                     which keeps plain loads but not non-temporal ones), the
//                     pass reads with plain loads so that the compaction that
//                     follows finds much of K there; larger caches are read
//                     non-temporally.  Workgroups placed after the key
//                     workgroups sum the window queries' squares per (b, q
//                     head, channel) in fp64 meanwhile.
//   k_score_finalize  one workgroup per (b, kv): sums the splits in fp64 in a
//                     fixed order, forms the score from them and the window
//                     sums, and optionally selects the kept channels right
//                     there.
// No atomics: results are bitwise reproducible.
#include "select_row.h"

namespace thinkkv {
namespace {

constexpr int kThreads = 512;   // partial pass: ~256 workgroups of 8 waves stream K best
constexpr int kColGroup = 256;  // 16-byte column vectors per workgroup
constexpr int kRun = 16;   // tokens per fp32 run before folding into fp64
constexpr int kQVec = 32;  // window-row vectors per window-query workgroup

template <int DT, bool KEEP_IN_LLC>
__global__ __launch_bounds__(kThreads) void k_score_partial(
        const uint4* __restrict__ k_vec, const int32_t* __restrict__ seq_lens, int s_cap,
        int nvec, int tpw, int nsplit, int ncg, float* __restrict__ partials, int nb,
        const uint4* __restrict__ q_vec, int W, int nqv, double* __restrict__ q2) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    // one-dimensional grid: the key workgroups (split fastest, then column
    // group, then sequence), then the window-query workgroups
    const uint32_t nkey = (uint32_t)nsplit * ncg * nb;
    const uint32_t wg = blockIdx.x;
    const int split = (int)(wg % nsplit), cg = (int)(wg / nsplit % ncg);
    int b = (int)(wg / ((uint32_t)nsplit * ncg));
    __shared__ double red[kThreads * 8];         // lane sums, reduced in a fixed order
    if (wg >= nkey) {
        // window-query sums of squares of sequence b, for every query head and
        // channel: Q2[b][h][c] = sum over the W window rows in fp64 (a bf16 or
        // fp32 square is exact in fp64).  Each window-query workgroup takes
        // kQVec 16-byte vectors of the window row; its lanes split
        // the rows into kQGroups contiguous groups, summed in row order, and
        // the groups are added in ascending order.  They come after every key
        // workgroup in the grid, so they are dispatched last and never delay
        // the key stream.
        const int nqb = (nqv + kQVec - 1) / kQVec;           // units per sequence
        const int u = (int)(wg - nkey);
        const int qb = u % nqb;
        b = u / nqb;
        constexpr int kQGroups = kThreads / kQVec;
        const int vq = qb * kQVec + (int)threadIdx.x % kQVec;
        const int rg = (int)threadIdx.x / kQVec;
        const int i0 = rg * W / kQGroups, i1 = (rg + 1) * W / kQGroups;
        const uint4* src = q_vec + (size_t)b * W * nqv + min(vq, nqv - 1);
        double acc[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
        for (int i = i0; i < i1; i += 8) {
            uint4 x[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = src[(size_t)min(i + k, W - 1) * nqv];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                float f[EPV];
                unpack(x[k], f, E{});
                const bool ok = i + k < i1;
#pragma unroll
                for (int e = 0; e < EPV; ++e) acc[e] += ok ? (double)f[e] * (double)f[e] : 0.0;
            }
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) red[(rg * kQVec + threadIdx.x % kQVec) * EPV + e] = acc[e];
        __syncthreads();
        for (int o = threadIdx.x; o < kQVec * EPV; o += kThreads) {
            const int v = qb * kQVec + o / EPV;
            if (v >= nqv) continue;
            double t = 0.0;
            for (int r = 0; r < kQGroups; ++r) t += red[r * kQVec * EPV + o];
            q2[(size_t)b * nqv * EPV + (size_t)v * EPV + o % EPV] = t;
        }
        return;
    }
    const int len = clamp_len(seq_lens, b, s_cap);
    const int t0 = split * tpw;
    if (t0 >= len) return;                       // finalize never reads this split
    const int t1 = min(t0 + tpw, len);

    const int v0 = cg * kColGroup;
    const int nvg = min(kColGroup, nvec - v0);    // vectors in this column group
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
                const uint4* a = base + (size_t)tt * nvec;
                v[u] = tt < t1 ? (KEEP_IN_LLC ? *a : ldg_stream(a)) : make_uint4(0u, 0u, 0u, 0u);
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

// One workgroup per (b, kv), blockDim = (D/4) x SG threads.
//  K2:  thread (channel quad cq, split group sg) sums splits sg, sg+SG, ...
//       in ascending order, reading float4 partials eight splits at a time
//       so the loads overlap; the SG group sums are added in ascending order.
//  Q:   from the cache path, the window-query sums Q2 the partial pass wrote
//       (q2 [B][Hq][D] fp64).  From the prefill state (STATE), the group's
//       window rows (G*D contiguous query elements) are summed here: thread
//       (16-byte vector v, row group rg) sums the squares of its vector over
//       a contiguous range of rows (loads issued eight rows at a time); the
//       row groups are added in ascending order.
//  s  = sqrt(K2) * sum_g sqrt(Q2[g]), fp64, stored as fp32; with SELECT the
//       same workgroup then picks the kept channels (select_row.h).
// STATE: the sums come from the prefill-write state instead (fp64 slots
// [B][nsplit][Hkv*D], every slot complete; no length is read).
template <int DT, bool SELECT, bool STATE>
__global__ __launch_bounds__(1024) void k_score_finalize(
        const void* __restrict__ part, const int32_t* __restrict__ seq_lens, int s_cap,
        int tpw, int nsplit, const typename Elem<DT>::T* __restrict__ q_obs,
        const double* __restrict__ q2, int W, int Hq, int Hkv, int D,
        float* __restrict__ scores, int keep, int32_t* __restrict__ kept_idx,
        int32_t* __restrict__ near_tie) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const int kv = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int G = Hq / Hkv, R = Hkv * D, Q = D / 4, SG = nth / Q;
    __shared__ double red[4096];                 // [SG][D] split-group sums, then [RG][G*D]
    __shared__ double qn[4096];                  // [g][c] sqrt(Q2)  (G * D <= 4096)
    __shared__ __align__(16) float s_sc[256];
    __shared__ int s_scratch[1024];
    __shared__ float s_cut[2];

    // The first round of loads is issued before any is waited on: the length
    // (a vector load, so waiting for it leaves the rest in flight), this
    // thread's first eight split partials and its first eight window rows.
    // Their indices are clamped into range instead of branched on, and the
    // slots past the length's split count or past the row group are dropped
    // when summed (a dropped slot adds +0.0, so the sums are those of the
    // plain loops).
    const int cq = tid % Q, sg = tid / Q;
    int len_v = 0;
    const float4* p = nullptr;
    const size_t sstride = (size_t)R / 4;
    float4 v[8];
    if constexpr (!STATE) {
        len_v = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(seq_lens + b, 4u), 0, 0, 0);
        p = reinterpret_cast<const float4*>(static_cast<const float*>(part) +
                                            (size_t)b * nsplit * R + (size_t)kv * D) + cq;
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = p[(size_t)min(sg + k * SG, nsplit - 1) * sstride];
    }

    const int GD = G * D, nv = GD / EPV;         // 16-byte vectors per window row
    int RG = nth / nv;
    if (RG > 4096 / GD) RG = 4096 / GD;
    if (RG > W) RG = W;
    if (RG < 1) RG = 1;
    const int qv = tid % nv, rg = tid / nv;
    const bool qact = STATE && rg < RG;
    const int i0 = qact ? rg * W / RG : 0, i1 = qact ? (rg + 1) * W / RG : 0;
    const uint4* qb = reinterpret_cast<const uint4*>(
        q_obs + ((size_t)b * W * Hq + (size_t)kv * G) * D) + qv;
    const size_t rstride = (size_t)Hq * D / EPV;     // vectors between window rows
    uint4 x[8];
    if constexpr (STATE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = qb[(size_t)min(i0 + k, W - 1) * rstride];
    } else {
        // the group's Q2 rows straight into their norms (read before any wait
        // on the partials, so both loads overlap)
        const double* qs = q2 + ((size_t)b * Hq + (size_t)kv * G) * D;
        for (int pr = tid; pr < GD; pr += nth) qn[pr] = sqrt(qs[pr]);
    }

    if constexpr (STATE) {
        // four channels per thread as two 16-byte double pairs per slot
        const double2* p2 = reinterpret_cast<const double2*>(
            static_cast<const double*>(part) + (size_t)b * nsplit * R + (size_t)kv * D + 4 * cq);
        const size_t s2 = (size_t)R / 2;
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        for (int s0 = sg; s0 < nsplit; s0 += 8 * SG) {
            double2 w0[8], w1[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const size_t o = (size_t)min(s0 + k * SG, nsplit - 1) * s2;
                w0[k] = p2[o];
                w1[k] = p2[o + 1];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool ok = s0 + k * SG < nsplit;
                a0 += ok ? w0[k].x : 0.0;
                a1 += ok ? w0[k].y : 0.0;
                a2 += ok ? w1[k].x : 0.0;
                a3 += ok ? w1[k].y : 0.0;
            }
        }
        red[sg * D + 4 * cq + 0] = a0;
        red[sg * D + 4 * cq + 1] = a1;
        red[sg * D + 4 * cq + 2] = a2;
        red[sg * D + 4 * cq + 3] = a3;
    } else {
    const int len_raw = __builtin_amdgcn_readfirstlane(len_v);
    const int len = len_raw < 0 ? 0 : (len_raw > s_cap ? s_cap : len_raw);
    const int ns = (len + tpw - 1) / tpw;

    {
        double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
        auto add = [&](const float4 (&w)[8], int s0) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const bool ok = s0 + k * SG < ns;
                a0 += ok ? (double)w[k].x : 0.0;
                a1 += ok ? (double)w[k].y : 0.0;
                a2 += ok ? (double)w[k].z : 0.0;
                a3 += ok ? (double)w[k].w : 0.0;
            }
        };
        if (sg < ns) add(v, sg);
        for (int s0 = sg + 8 * SG; s0 < ns; s0 += 8 * SG) {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = p[(size_t)min(s0 + k * SG, nsplit - 1) * sstride];
            add(v, s0);
        }
        red[sg * D + 4 * cq + 0] = a0;
        red[sg * D + 4 * cq + 1] = a1;
        red[sg * D + 4 * cq + 2] = a2;
        red[sg * D + 4 * cq + 3] = a3;
    }
    }
    // window-query squares of this thread's vector over its rows, in row order
    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
    auto addq = [&](const uint4 (&w)[8], int r0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float f[EPV];
            unpack(w[k], f, E{});
            const bool ok = r0 + k < i1;
#pragma unroll
            for (int e = 0; e < EPV; ++e) acc[e] += ok ? (double)f[e] * (double)f[e] : 0.0;
        }
    };
    if constexpr (STATE) {
        if (i0 < i1) addq(x, i0);
        for (int i = i0 + 8; i < i1; i += 8) {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = qb[(size_t)min(i + k, W - 1) * rstride];
            addq(x, i);
        }
    }

    __syncthreads();
    double K2 = 0.0;
    if (tid < D)
        for (int r = 0; r < SG; ++r) K2 += red[r * D + tid];
    if constexpr (STATE) {
        __syncthreads();                         // red is reused below
        if (qact) {
#pragma unroll
            for (int e = 0; e < EPV; ++e) red[rg * GD + qv * EPV + e] = acc[e];
        }
        __syncthreads();
        for (int pr = tid; pr < GD; pr += nth) {
            double t = 0.0;
            for (int r = 0; r < RG; ++r) t += red[r * GD + pr];
            qn[pr] = sqrt(t);                    // index g*D + c
        }
    }
    __syncthreads();

    if (tid < D) {
        double qsum = 0.0;
        for (int g = 0; g < G; ++g) qsum += qn[g * D + tid];
        const float sc = (float)(sqrt(K2) * qsum);
        if (scores) scores[((size_t)b * Hkv + kv) * D + tid] = sc;
        s_sc[tid] = sc;
    }
    if (SELECT) {
        __syncthreads();
        const size_t row = (size_t)b * Hkv + kv;
        int32_t* const tie = near_tie ? near_tie + row : nullptr;
        if (D == 128)
            select_row<128>(s_sc, D, keep, nth, s_scratch, s_cut, kept_idx + row * keep, tie);
        else
            select_row(s_sc, D, keep, nth, s_scratch, s_cut, kept_idx + row * keep, tie);
    }
}

}  // namespace

ScoreGeom score_geom(const think_dims& d) {
    ScoreGeom g{};
    const int e = elem_bytes(d.dtype);
    g.nvec = d.n_kv_heads * d.head_dim * e / 16;
    g.ncg = (g.nvec + kColGroup - 1) / kColGroup;
    // aim for ~256 workgroups (one per CU); tokens per workgroup a multiple of 16
    const int64_t rows = (int64_t)d.seq_capacity * d.batch * g.ncg;
    int64_t tpw = (rows + 255) / 256;
    tpw = (tpw + 15) / 16 * 16;
    if (tpw < 16) tpw = 16;
    if (tpw > 4096) tpw = 4096;
    g.tpw = (int)tpw;
    g.nsplit = (int)((d.seq_capacity + tpw - 1) / tpw);
    // up to 192 MiB of K (by capacity) is read with plain loads: a second read
    // of that much was measured 1.6-1.9x faster than the first on this part
    const size_t k_bytes = (size_t)d.batch * d.seq_capacity * g.nvec * 16;
    g.keep_in_llc = k_bytes <= ((size_t)192 << 20);
    // fp32 partials [B][nsplit][Hkv*D], then (16-byte aligned) the window
    // query sums Q2 [B][Hq][D] fp64
    g.q2_offset = ((size_t)d.batch * g.nsplit * d.n_kv_heads * d.head_dim * sizeof(float) + 15) /
                  16 * 16;
    g.ws_bytes = g.q2_offset + (size_t)d.batch * d.n_q_heads * d.head_dim * sizeof(double);
    return g;
}

hipError_t launch_score(const think_dims& d, const ScoreGeom& g, const void* k_cache,
                        const int32_t* seq_lens, const void* q_obs, int W, float* scores,
                        void* workspace, int keep, int32_t* kept_idx, int32_t* near_tie,
                        hipStream_t s) {
    float* partials = reinterpret_cast<float*>(workspace);
    double* q2 = reinterpret_cast<double*>(static_cast<char*>(workspace) + g.q2_offset);
    const int nqv = d.n_q_heads * d.head_dim * elem_bytes(d.dtype) / 16;
    // key workgroups, then the window-query workgroups, in one dimension
    const size_t nq_units = (size_t)d.batch * ((nqv + kQVec - 1) / kQVec);
    dim3 grid1((unsigned)((size_t)g.nsplit * g.ncg * d.batch + nq_units));
    const int Q = d.head_dim / 4;
    int sg = 1024 / Q;
    if (sg > 64) sg = 64;
    dim3 grid2(d.n_kv_heads, d.batch);
    const int threads2 = Q * sg;
#define THINK_FINALIZE(DT, SEL, T)                                                               \
    k_score_finalize<DT, SEL, false><<<grid2, threads2, 0, s>>>(                                \
        partials, seq_lens, d.seq_capacity, g.tpw, g.nsplit, (const T*)q_obs, q2, W,            \
        d.n_q_heads, d.n_kv_heads, d.head_dim, scores, keep, kept_idx, near_tie)
#define THINK_PARTIAL(DT, LLC)                                                                   \
    k_score_partial<DT, LLC><<<grid1, kThreads, 0, s>>>(                                        \
        (const uint4*)k_cache, seq_lens, d.seq_capacity, g.nvec, g.tpw, g.nsplit, g.ncg,         \
        partials, d.batch, (const uint4*)q_obs, W, nqv, q2)
    if (d.dtype == THINK_BF16) {
        if (g.keep_in_llc) THINK_PARTIAL(THINK_BF16, true);
        else THINK_PARTIAL(THINK_BF16, false);
        if (kept_idx) THINK_FINALIZE(THINK_BF16, true, uint16_t);
        else THINK_FINALIZE(THINK_BF16, false, uint16_t);
    } else {
        if (g.keep_in_llc) THINK_PARTIAL(THINK_F32, true);
        else THINK_PARTIAL(THINK_F32, false);
        if (kept_idx) THINK_FINALIZE(THINK_F32, true, float);
        else THINK_FINALIZE(THINK_F32, false, float);
    }
#undef THINK_PARTIAL
#undef THINK_FINALIZE
    return hipGetLastError();
}

hipError_t launch_score_k2(const think_dims& d, int nslots, const double* state, const void* q_obs,
                           int W, float* scores, int keep, int32_t* kept_idx, int32_t* near_tie,
                           hipStream_t s) {
    const int Q = d.head_dim / 4;
    int sg = 1024 / Q;
    if (sg > 64) sg = 64;
    dim3 grid2(d.n_kv_heads, d.batch);
    const int threads2 = Q * sg;
#define THINK_FINALIZE_K2(DT, SEL, T)                                                            \
    k_score_finalize<DT, SEL, true><<<grid2, threads2, 0, s>>>(                                 \
        state, nullptr, d.seq_capacity, 1, nslots, (const T*)q_obs, nullptr, W, d.n_q_heads,    \
        d.n_kv_heads, d.head_dim, scores, keep, kept_idx, near_tie)
    if (d.dtype == THINK_BF16) {
        if (kept_idx) THINK_FINALIZE_K2(THINK_BF16, true, uint16_t);
        else THINK_FINALIZE_K2(THINK_BF16, false, uint16_t);
    } else {
        if (kept_idx) THINK_FINALIZE_K2(THINK_F32, true, float);
        else THINK_FINALIZE_K2(THINK_F32, false, float);
    }
#undef THINK_FINALIZE_K2
    return hipGetLastError();
}

}  // namespace thinkkv
