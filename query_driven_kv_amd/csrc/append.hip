// append.hip - decode-time append, the step after the decode attention:
// inference continues on the pruned key cache ("ThinK: Thinner Key Cache by
// Query-Driven Pruning", Method details -> Technical framework, last step),
// so a generated token's key is stored pruned with the kept set already chosen
// for its (b, kv) and its value in full:
//
//   k_thin[b,len_b,kv,j] = k_new[b,kv,kept_idx[b,kv,j]]
//   v_cache[b,len_b,kv,:] = v_new[b,kv,:]            then len_b += 1
//
// One workgroup per sequence.  Every thread reads len_b, the rows are written
// (the value row as 16-byte vectors, the thin key row element by element since
// odd keep leaves it 2-byte aligned), and after a barrier, so that no thread
// still has to read the old length, one thread stores len_b + 1.  A sequence
// already at capacity is left as it is.  A byte copy: exact by construction.
#include "think_common.h"

namespace thinkkv {
namespace {

constexpr int kThreads = 256;

template <typename E>
__global__ __launch_bounds__(kThreads) void k_append(
        const E* __restrict__ k_new, const uint4* __restrict__ v_new, int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, E* __restrict__ k_thin, uint4* __restrict__ v_cache,
        int s_cap, int Hkv, int D, int keep) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const int t = clamp_len(seq_lens, b, s_cap);
    if (t >= s_cap) return;                      // full: left as it is
    const int Ro = Hkv * keep;
    E* krow = k_thin + ((size_t)b * s_cap + t) * Ro;
    for (int o = tid; o < Ro; o += kThreads) {
        const int kv = o / keep;
        int c = kept_idx[(size_t)b * Ro + o];
        c = c < 0 ? 0 : (c >= D ? D - 1 : c);
        krow[o] = k_new[((size_t)b * Hkv + kv) * D + c];
    }
    const int nv = Hkv * D * (int)sizeof(E) / 16;    // 16-byte vectors per value row
    uint4* vrow = v_cache + ((size_t)b * s_cap + t) * nv;
    for (int v = tid; v < nv; v += kThreads) vrow[v] = v_new[(size_t)b * nv + v];
    __syncthreads();
    if (tid == 0) seq_lens[b] = t + 1;
}

}  // namespace

hipError_t launch_append(const think_dims& d, const void* k_new, const void* v_new,
                         int32_t* seq_lens, const int32_t* kept_idx, int keep, void* k_thin,
                         void* v_cache, hipStream_t s) {
    dim3 grid(d.batch);
    if (d.dtype == THINK_BF16)
        k_append<uint16_t><<<grid, kThreads, 0, s>>>(
            (const uint16_t*)k_new, (const uint4*)v_new, seq_lens, kept_idx, (uint16_t*)k_thin,
            (uint4*)v_cache, d.seq_capacity, d.n_kv_heads, d.head_dim, keep);
    else
        k_append<float><<<grid, kThreads, 0, s>>>(
            (const float*)k_new, (const uint4*)v_new, seq_lens, kept_idx, (float*)k_thin,
            (uint4*)v_cache, d.seq_capacity, d.n_kv_heads, d.head_dim, keep);
    return hipGetLastError();
}

}  // namespace thinkkv
