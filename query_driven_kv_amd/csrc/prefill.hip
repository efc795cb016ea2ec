// prefill.hip - prefill-fused scoring, write half (the step before the path).
//
// Stage (a) reads the keys only through K2[b,kv,c] = sum_t K[b,t,kv,c]^2
// ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework, first step, in the closed form used for the score).
// The prompt's keys pass through the cache write anyway, so this kernel writes
// a chunk of new K and V rows into the caches and gathers the chunk's sums of
// squares on the way; the score then needs no key read.
//
// Workgroup = (slot, column group, b): the chunk's rows are split into
// `nslots` contiguous ranges, one per slot.  Lanes own one 16-byte column
// vector across rows (as in the score pass): they copy the K and V vectors to
// the caches and keep fp32 runs of at most 16 squares folded into fp64.  The
// lanes' sums are reduced in LDS in a fixed order and added to the slot's fp64
// entry in the state [B][nslots][Hkv*D]: each entry has one writer per call and
// calls on a stream are ordered, so no atomics and bitwise reproducible.
// Rows at positions >= min(len_b, S_cap) are neither written nor counted.
#include "think_common.h"

namespace thinkkv {
namespace {

constexpr int kThreads = 512;
constexpr int kColGroup = 256;   // 16-byte column vectors per workgroup
constexpr int kRun = 16;         // rows per fp32 run before folding into fp64

template <int DT>
__global__ __launch_bounds__(kThreads) void k_prefill_write(
        const uint4* __restrict__ k_rows, const uint4* __restrict__ v_rows, int t0, int n_rows,
        int rpw, const int32_t* __restrict__ seq_lens, int s_cap, int nvec,
        uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, double* __restrict__ state,
        int nslots) {
    using E = Elem<DT>;
    constexpr int EPV = E::kPerVec;
    const int slot = blockIdx.x, cg = blockIdx.y, b = blockIdx.z;
    const int len = clamp_len(seq_lens, b, s_cap);
    const int r0 = slot * rpw;
    const int r1 = min(min(r0 + rpw, n_rows), len - t0);   // chunk rows this slot writes

    const int v0 = cg * kColGroup;
    const int nvg = min(kColGroup, nvec - v0);
    const int rpi = kThreads / nvg;
    const int tid = threadIdx.x;
    const bool active = tid < rpi * nvg;
    const int col = active ? tid % nvg : 0;
    const int rsub = active ? tid / nvg : 0;

    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
    if (active) {
        const uint4* ks = k_rows + (size_t)b * n_rows * nvec + v0 + col;
        const uint4* vs = v_rows + (size_t)b * n_rows * nvec + v0 + col;
        uint4* kd = k_cache + ((size_t)b * s_cap + t0) * nvec + v0 + col;
        uint4* vd = v_cache + ((size_t)b * s_cap + t0) * nvec + v0 + col;
        for (int t = r0 + rsub; t < r1; t += kRun * rpi) {
            uint4 kx[kRun], vx[kRun];
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                const int tt = t + u * rpi;
                kx[u] = tt < r1 ? ldg_stream(ks + (size_t)tt * nvec) : make_uint4(0u, 0u, 0u, 0u);
                vx[u] = tt < r1 ? ldg_stream(vs + (size_t)tt * nvec) : make_uint4(0u, 0u, 0u, 0u);
            }
            float run[EPV];
#pragma unroll
            for (int e = 0; e < EPV; ++e) run[e] = 0.0f;
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                const int tt = t + u * rpi;
                if (tt < r1) {
                    kd[(size_t)tt * nvec] = kx[u];
                    vd[(size_t)tt * nvec] = vx[u];
                }
                float x[EPV];
                unpack(kx[u], x, E{});
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
    const int R = nvec * EPV;
    double* st = state + ((size_t)b * nslots + slot) * R + (size_t)v0 * EPV;
    for (int o = tid; o < nvg * EPV; o += kThreads) {
        double s = 0.0;
        for (int r = 0; r < rpi; ++r) s += red[r * nvg * EPV + o];
        st[o] += s;
    }
}

}  // namespace

K2Geom k2_geom(const think_dims& d) {
    K2Geom g{};
    g.nvec = d.n_kv_heads * d.head_dim * elem_bytes(d.dtype) / 16;
    g.ncg = (g.nvec + kColGroup - 1) / kColGroup;
    int slots = 256 / (d.batch * g.ncg);
    g.nslots = slots < 1 ? 1 : slots;
    g.bytes = (size_t)d.batch * g.nslots * d.n_kv_heads * d.head_dim * sizeof(double);
    return g;
}

hipError_t launch_prefill_write(const think_dims& d, const K2Geom& g, const void* k_rows,
                                const void* v_rows, int t0, int n_rows, const int32_t* seq_lens,
                                void* k_cache, void* v_cache, double* state, hipStream_t s) {
    const int rpw = (n_rows + g.nslots - 1) / g.nslots;
    dim3 grid(g.nslots, g.ncg, d.batch);
    if (d.dtype == THINK_BF16)
        k_prefill_write<THINK_BF16><<<grid, kThreads, 0, s>>>(
            (const uint4*)k_rows, (const uint4*)v_rows, t0, n_rows, rpw, seq_lens, d.seq_capacity,
            g.nvec, (uint4*)k_cache, (uint4*)v_cache, state, g.nslots);
    else
        k_prefill_write<THINK_F32><<<grid, kThreads, 0, s>>>(
            (const uint4*)k_rows, (const uint4*)v_rows, t0, n_rows, rpw, seq_lens, d.seq_capacity,
            g.nvec, (uint4*)k_cache, (uint4*)v_cache, state, g.nslots);
    return hipGetLastError();
}

}  // namespace thinkkv
