// compact.hip - stage (c): write the thinner key cache ("ThinK: Thinner Key
// Cache by Query-Driven Pruning", title and Method details -> Technical
// framework: inference runs on the pruned key cache).
//
//   k_thin[b,t,kv,j] = k_cache[b,t,kv,kept_idx[b,kv,j]]    t < len_b
//
// The kept channels are scattered inside every 2-byte (bf16) or 4-byte (fp32)
// key row, so the whole row has to be read.  A workgroup owns `tile` whole
// token rows of one sequence (all kv heads): it reads them into LDS with
// coalesced dwordx4 loads, then emits its output, which is ONE contiguous
// range of tile*Hkv*keep elements, as a flat stream of 16-byte stores
// gathered from LDS through a per-workgroup source map.  This keeps stores
// 16-byte wide even when keep is odd (per-head thin rows of 154 or 102 bytes).
// Only the two 16-byte chunks at the ends of the range can be partial; those
// are written element by element.  Loads and stores are non-temporal (each
// byte is touched once per call).  A pure copy: bit-exact by construction.
#include "think_common.h"

namespace thinkkv {
namespace {

constexpr int kThreads = 256;

template <typename E>
__global__ __launch_bounds__(kThreads) void k_compact(
        const E* __restrict__ k_cache, const int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, E* __restrict__ k_thin, int s_cap, int Hkv,
        int D, int keep, int tile) {
    extern __shared__ uint4 lds[];
    constexpr int CE = 16 / sizeof(E);           // elements per 16-byte chunk
    const int b = blockIdx.y;
    const int t0 = blockIdx.x * tile;
    const int len = clamp_len(seq_lens, b, s_cap);
    if (t0 >= len) return;
    const int nt = min(tile, len - t0);
    const int R = Hkv * D, Ro = Hkv * keep;
    E* rows = reinterpret_cast<E*>(lds);
    uint16_t* srcmap = reinterpret_cast<uint16_t*>(rows + (size_t)tile * R);
    const int tid = threadIdx.x;

    const int nvec = nt * R * (int)sizeof(E) / 16;
    const uint4* src = reinterpret_cast<const uint4*>(k_cache + ((size_t)b * s_cap + t0) * R);
    // The first kFirst row vectors per thread (32 KiB per workgroup: every
    // tile of up to 32 KiB) are loaded into registers first, through a
    // descriptor bounded to the tile (vectors past it read zero without
    // touching memory), so they are in flight together with the kept-index
    // loads of the source map: one memory round trip instead of two.  Larger
    // tiles load the rest after.
    constexpr int kFirst = 8;
    const auto rsrc = make_rsrc(src, (uint32_t)nvec * 16u);
    uint4 first[kFirst];
#pragma unroll
    for (int k = 0; k < kFirst; ++k)
        first[k] = ldb_stream(rsrc, (uint32_t)(tid + k * kThreads) * 16u);
    for (int o = tid; o < Ro; o += kThreads) {
        const int kv = o / keep, j = o - kv * keep;
        int c = kept_idx[((size_t)b * Hkv + kv) * keep + j];
        c = c < 0 ? 0 : (c >= D ? D - 1 : c);
        srcmap[o] = (uint16_t)(kv * D + c);
    }
#pragma unroll
    for (int k = 0; k < kFirst; ++k)
        if (tid + k * kThreads < nvec) lds[tid + k * kThreads] = first[k];
    for (int v = tid + kFirst * kThreads; v < nvec; v += kThreads) lds[v] = ldg_stream(src + v);
    __syncthreads();

    const size_t E0 = ((size_t)b * s_cap + t0) * Ro;
    const size_t E1 = E0 + (size_t)nt * Ro;
    const size_t c0 = E0 / CE, c1 = (E1 + CE - 1) / CE;
    for (size_t ch = c0 + tid; ch < c1; ch += kThreads) {
        const size_t lo = ch * CE;
        if (lo >= E0 && lo + CE <= E1) {
            const int f = (int)(lo - E0);
            int r = f / Ro, o = f - r * Ro;
            union { uint4 v; E e[CE]; } pack;
#pragma unroll
            for (int k = 0; k < CE; ++k) {
                pack.e[k] = rows[r * R + srcmap[o]];
                if (++o == Ro) { o = 0; ++r; }
            }
            __builtin_nontemporal_store(u32x4_t{pack.v.x, pack.v.y, pack.v.z, pack.v.w},
                                        reinterpret_cast<u32x4_t*>(k_thin + lo));
        } else {
            const size_t a = lo > E0 ? lo : E0;
            const size_t z = lo + CE < E1 ? lo + CE : E1;
            for (size_t e = a; e < z; ++e) {
                const int f = (int)(e - E0);
                const int r = f / Ro, o = f - r * Ro;
                k_thin[e] = rows[r * R + srcmap[o]];
            }
        }
    }
}

}  // namespace

CompactGeom compact_geom(const think_dims& d, int keep) {
    CompactGeom g{};
    const int row_bytes = d.n_kv_heads * d.head_dim * elem_bytes(d.dtype);
    // 16 KiB tiles (8 rows of a 2 KiB row): enough workgroups per CU to keep
    // the loads and stores of several tiles in flight.  Wide rows (many kv
    // heads) take at least 4 rows (up to 64 KiB), so the per-workgroup source
    // map of Hkv*keep kept channels is built for enough data to pay for itself.
    int tile = 16384 / row_bytes;
    if (tile < 4) tile = 65536 / row_bytes < 4 ? 65536 / row_bytes : 4;
    if (tile > 64) tile = 64;
    if (tile < 1) tile = 1;
    g.tile = tile;
    const size_t map_bytes = ((size_t)d.n_kv_heads * keep * 2 + 15) / 16 * 16;
    g.lds = (size_t)tile * row_bytes + map_bytes;
    return g;
}

hipError_t launch_compact(const think_dims& d, const CompactGeom& g, const void* k_cache,
                          const int32_t* seq_lens, const int32_t* kept_idx, int keep,
                          void* k_thin, hipStream_t s) {
    dim3 grid((d.seq_capacity + g.tile - 1) / g.tile, d.batch);
    if (d.dtype == THINK_BF16)
        k_compact<uint16_t><<<grid, kThreads, g.lds, s>>>(
            (const uint16_t*)k_cache, seq_lens, kept_idx, (uint16_t*)k_thin, d.seq_capacity,
            d.n_kv_heads, d.head_dim, keep, g.tile);
    else
        k_compact<uint32_t><<<grid, kThreads, g.lds, s>>>(
            (const uint32_t*)k_cache, seq_lens, kept_idx, (uint32_t*)k_thin, d.seq_capacity,
            d.n_kv_heads, d.head_dim, keep, g.tile);
    return hipGetLastError();
}

}  // namespace thinkkv
