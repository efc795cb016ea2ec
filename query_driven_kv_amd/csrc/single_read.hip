// single_read.hip - stages (a), (b) and (c) in one pass over the key cache.
//
// "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework: score every key channel against the observation
// window, keep the most relevant, and store the pruned key cache.  The
// scores need every token of a sequence before any thin row can be written,
// so the plain schedule reads K twice (score pass, then compaction).  When
// the whole key cache fits in the register files of the chip (512 KiB per
// CU, half of it used here: 64 MiB over 256 CUs), one launch with one
// workgroup per compute unit reads it once:
//
//   phase 1  every workgroup (one per CU) loads its tile of token rows of one
//            sequence (each XCD a contiguous run of tiles) into registers (16-byte vectors, all loads in flight at
//            once), sums the per-channel squares of the tile (fp32 runs of
//            <= 16 tokens folded into fp64, the rows of a column reduced in
//            LDS in a fixed order) and writes one fp32 partial per channel;
//            the window-query sums of squares (fp64) are spread over the
//            workgroups as well;
//            each workgroup then raises its "tile done" flag;
//   phase 2  workgroup (b, kv) waits for every tile flag, sums its row's
//            partials in fp64 in tile order, forms the scores
//            sqrt(K2) * sum_g sqrt(Q2), selects the kept channels
//            (select_row.h) and publishes the kept set as 16-bit mask chunks,
//            each in a 64-bit word with the launch's tag above it;
//   phase 3  every workgroup waits for the mask words of its own sequence
//            (the kept set arrives with the wait itself) and writes the thin
//            rows of its tile from the registers, through LDS, as one
//            contiguous stream of 16-byte stores (as the stand-alone
//            compaction does).
//
// A flag is a 64-bit word in the caller's workspace set to a tag that is new
// for every launch (a generation word in the workspace that every launch
// advances, so graph replays differ too, with the call's own counter below
// it), so a workspace with any previous contents works.  Every flag has one
// writer, which stores it once the data it publishes (written through to
// memory with device-scope stores) is complete; waiters read it with a
// relaxed agent-scope atomic load, which is a device-coherent (sc1) load that
// reads past this chiplet's cached copy (ordinary loads returned a copy cached
// in the chiplet's L2, 12 us late), then take one acquire fence.  (One arrival counter updated by every workgroup
// serialised the arrivals: about 1 ms per call when tried.)  The grid is at
// most one workgroup per compute unit and the occupancy query confirms that
// one fits, so every workgroup is resident at once, or becomes resident as
// the workgroups of other kernels finish; two launches of this kind running
// at once could each hold part of the device, which the interface forbids.
// Every wait is bounded all the same: should one run out, the kernel sets an
// error word and finishes, so nothing hangs.  (A cooperative launch, which
// the runtime refuses unless all workgroups fit at once, cost about 17 us
// more per call here.)  No float atomics: results are bitwise reproducible.
#include <atomic>
#include <chrono>

#include "select_row.h"

namespace thinkkv {
namespace {

constexpr int kSrThreads = 512;     // one workgroup per CU, 8 waves, <= 256 registers each
constexpr int kSrRun = 16;          // tokens per fp32 run before folding into fp64
constexpr int kQRowGroups = 32;     // threads per window-query unit (row ranges)
constexpr int kQUnits = kSrThreads / kQRowGroups;   // units per pass
constexpr int kQEarly = 4;          // window rows per thread loaded with the K tile
constexpr int kSrSubK = 16;         // k-slices (of 512 vectors) per compaction sub-tile: 128 KiB
constexpr uint32_t kSrSpinLimit = 1u << 22;

// Raise a flag once the whole workgroup's stores are done.  The data a flag
// publishes (tile partials, window-query sums) is stored with device-scope
// stores, which write through to memory; each thread waits until its own
// have completed, so no cache write-back is needed before the flag (a release
// fence here wrote back the chiplet's L2 once per workgroup: 2 us per launch).
__device__ __forceinline__ void signal_flag(unsigned long long* f, unsigned long long tag) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        __hip_atomic_store(f, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until flags[0..n) all hold the tag (thread i watches flags i, i+512,
// ...); the workgroup's later loads see everything their writers stored.  A
// flag is read with a relaxed agent-scope atomic load (a device-coherent sc1
// load: an ordinary load can return a copy cached on this chiplet); one
// acquire fence for the workgroup after the waits.
__device__ __forceinline__ void wait_flags(unsigned long long* f, int n,
                                           unsigned long long tag, unsigned long long want,
                                           uint32_t limit, unsigned long long* err) {
    for (int i = threadIdx.x; i < n; i += kSrThreads) {
        for (uint32_t spin = 0;; ++spin) {
            if (__hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want)
                break;
            if (spin >= limit) {
                __hip_atomic_store(err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
}

struct SrParams {
    const uint4* k_vec;        // K [B][S_cap][nvec] 16-byte vectors
    const int32_t* seq_lens;
    const uint4* q_vec;        // Q_w [B][W][nqv]
    float* partials;           // [nwg][R] fp32
    double* q2;                // [B][Hq][D] fp64
    float* scores;             // [B][Hkv][D] or NULL
    int32_t* kept_idx;         // [B][Hkv][keep]
    int32_t* near_tie;         // [B][Hkv] or NULL
    void* k_thin;              // [B][S_cap][Hkv][keep]
    unsigned long long* tile_done;   // [nwg] flags
    unsigned long long* selected;    // [B][Hkv][ceil(D/16)] tag << 16 | 16 mask bits
    unsigned long long* err;         // the tag of a launch whose wait ran out, else 0
    unsigned long long* gen;         // launch generation, advanced by every launch
    unsigned long long tag;          // per call, low 24 bits nonzero (frozen in a captured graph)
    unsigned long long want_xor;     // 0; nonzero only to test the give-up report (no wait matches)
    uint32_t spin_limit;             // polls before a wait gives up
    int s_cap, nvec, rpw, wps, nb, W, nqv, Hq, Hkv, D, keep;
};

// DC: head_dim fixed at compile time (128), or 0 for any head_dim; the
// phases after the stream are chains of dependent steps, where index
// arithmetic on a run-time head_dim (divisions, loops of unknown trip count)
// shows up directly in the launch's duration.
template <int DT, int NV, int DC>
__global__ __launch_bounds__(kSrThreads) void k_score_compact_resident(SrParams p) {
    using E = Elem<DT>;
    using T = typename E::T;
    constexpr int EPV = E::kPerVec;
    constexpr int CE = 16 / sizeof(T);
    extern __shared__ uint4 lds[];
    const int w = blockIdx.x, nwg = gridDim.x;
    const int tid = threadIdx.x;
    // tile number: consecutive workgroups are dealt round-robin over the 8
    // XCDs, so tw gives each XCD one contiguous run of tiles; tiles
    // interleaved between the XCDs every 256 KiB stream K a third slower.
    // The selection roles of phase 2 (and the window-query units) keep the
    // hardware order w, which spreads them over every XCD.
    const int xcd = w % 8;
    const int tw = xcd * (nwg / 8) + min(xcd, nwg % 8) + w / 8;
    const int b = tw / p.wps, part = tw - b * p.wps;
    const int nvec = p.nvec, R = nvec * EPV;     // channels per token row (Hkv*D)
    const int t0 = part * p.rpw;
    const int len = clamp_len(p.seq_lens, b, p.s_cap);
    const int nt = max(0, min(p.rpw, len - t0));  // valid rows of this tile
    // the flags' 48-bit tag: the workspace's launch generation (which
    // workgroup 0 advances once every workgroup has read it) above the call's
    // 24-bit value.  Launches on one workspace differ in the generation, so
    // replays of a captured launch, whose arguments are frozen, tag afresh
    // too; the call's value guards against a workspace of unrelated bytes.
    const unsigned long long gen =
            __hip_atomic_load(p.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long tag = ((gen & 0xffffffull) << 24) | (p.tag & 0xffffffull);
    const unsigned long long want = tag ^ p.want_xor;
    // The error word holds the tag of a launch whose wait ran out.  Workgroup 0
    // clears whatever an earlier launch left, unless a workgroup of this launch
    // has already reported (possible only if workgroup 0 started late), so the
    // word describes the latest launch on the workspace.
    if (w == 0 && tid == 0) {
        const unsigned long long e =
                __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long ex = e;
        if (e != tag)
            __hip_atomic_compare_exchange_strong(p.err, &ex, 0ull, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- phase 1: the tile into registers (vector tid + k*512 of the tile;
    // nvec divides 512, so every vector of a thread is in column tid % nvec)
    const uint4* tile = p.k_vec + ((size_t)b * p.s_cap + min(t0, p.s_cap)) * nvec;
    const auto rs = make_rsrc(tile, (uint32_t)nt * (uint32_t)nvec * 16u);
    uint4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) v[k] = ldb_stream(rs, (uint32_t)(tid + k * kSrThreads) * 16u);

    // window-query units: (sequence, 16-byte vector of the window row), B*nqv
    // in all, dealt in contiguous runs of upw over the workgroups; 32 threads
    // per unit each take a contiguous range of the W rows.  The first
    // kQEarly rows of the first pass are loaded here, behind the K loads.
    const int nunits = p.nb * p.nqv;
    const int upw = (nunits + nwg - 1) / nwg;
    const int uslot = tid / kQRowGroups, qr = tid % kQRowGroups;
    const int qi0 = qr * p.W / kQRowGroups, qi1 = (qr + 1) * p.W / kQRowGroups;
    const auto rq = make_rsrc(p.q_vec, (uint32_t)((size_t)p.nb * p.W * p.nqv * 16u));
    auto q_off = [&](int u, int i) -> uint32_t {   // byte offset of unit u, row i
        if (u >= nunits || u >= (w + 1) * upw || i >= qi1) return kOff;
        const int bq = u / p.nqv, vq = u - bq * p.nqv;
        return (uint32_t)((((size_t)bq * p.W + i) * p.nqv + vq) * 16u);
    };
    uint4 qe[kQEarly];
#pragma unroll
    for (int k = 0; k < kQEarly; ++k)
        qe[k] = ldb_stream(rq, q_off(w * upw + uslot, qi0 + k));

    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
#pragma unroll
    for (int k0 = 0; k0 < NV; k0 += kSrRun) {
        float run[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) run[e] = 0.0f;
#pragma unroll
        for (int k = k0; k < k0 + kSrRun && k < NV; ++k) {
            float x[EPV];
            unpack(v[k], x, E{});                // rows past the length read as zero
#pragma unroll
            for (int e = 0; e < EPV; ++e) run[e] = fmaf(x[e], x[e], run[e]);
        }
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[e] += (double)run[e];
    }
    double* red = reinterpret_cast<double*>(lds);   // [512/nvec][nvec*EPV]
    const int col = tid % nvec, rsub = tid / nvec, nsub = kSrThreads / nvec;
#pragma unroll
    for (int e = 0; e < EPV; ++e) red[(rsub * nvec + col) * EPV + e] = acc[e];
    __syncthreads();
    for (int o = tid; o < R; o += kSrThreads) {
        double s = 0.0;
        for (int r = 0; r < nsub; ++r) s += red[r * R + o];
        __hip_atomic_store(p.partials + (size_t)tw * R + o, (float)s, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }

    // window-query sums of squares of this workgroup's units: each thread
    // sums its rows in row order (fp64; a bf16 or fp32 square is exact), the
    // 32 row groups are added in ascending order
    for (int u0 = w * upw; u0 < min((w + 1) * upw, nunits); u0 += kQUnits) {
        const int u = u0 + uslot;
        double qa[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e) qa[e] = 0.0;
        auto addq = [&](const uint4& x) {
            float f[EPV];
            unpack(x, f, E{});                   // rows out of range read as zero
#pragma unroll
            for (int e = 0; e < EPV; ++e) qa[e] += (double)f[e] * (double)f[e];
        };
        if (u0 == w * upw) {
#pragma unroll
            for (int k = 0; k < kQEarly; ++k) addq(qe[k]);
            for (int i = qi0 + kQEarly; i < qi1; ++i) addq(ldb_stream(rq, q_off(u, i)));
        } else {
            for (int i = qi0; i < qi1; ++i) addq(ldb_stream(rq, q_off(u, i)));
        }
        __syncthreads();                         // red is free again
#pragma unroll
        for (int e = 0; e < EPV; ++e) red[(qr * kQUnits + uslot) * EPV + e] = qa[e];
        __syncthreads();
        for (int o = tid; o < kQUnits * EPV; o += kSrThreads) {
            const int uu = u0 + o / EPV;
            if (uu >= nunits || uu >= (w + 1) * upw) continue;
            double t = 0.0;
            for (int r = 0; r < kQRowGroups; ++r) t += red[r * kQUnits * EPV + o];
            __hip_atomic_store(p.q2 + (size_t)uu * EPV + o % EPV, t, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);     // [b][nqv][EPV] = [b][Hq][D]
        }
    }

    signal_flag(p.tile_done + tw, tag);

    // ---- phase 2: scores and selection, one workgroup per (b, kv)
    if (w < p.nb * p.Hkv) {
        // what does not depend on other workgroups' data (the sequence
        // length, the index arithmetic) is done before the wait, so that the
        // loads after it start at once
        const int bb = w / p.Hkv, kv = w - bb * p.Hkv;
        const int D = DC > 0 ? DC : p.D, G = p.Hq / p.Hkv, Q = D / 4, SG = kSrThreads / Q;
        const int lenb = clamp_len(p.seq_lens, bb, p.s_cap);
        const int np = min(p.wps, (lenb + p.rpw - 1) / p.rpw);   // tiles holding rows
        double* red2 = reinterpret_cast<double*>(lds);           // [SG][D]
        double* qn = red2 + SG * D;                               // [G][D]
        float* s_sc = reinterpret_cast<float*>(qn + G * D);      // [256]
        int* scratch = reinterpret_cast<int*>(s_sc + 256);       // [512]
        float* cut = reinterpret_cast<float*>(scratch + kSrThreads);
        const int cq = tid % Q, sg = tid / Q;
        wait_flags(p.tile_done, nwg, tag, want, p.spin_limit, p.err);
        // every workgroup has stored its flag, so every one has read gen
        if (w == 0 && tid == 0)
            __hip_atomic_store(p.gen, gen + 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the group's window sums first, so both loads are in flight together
        const double* qs = p.q2 + ((size_t)bb * p.Hq + (size_t)kv * G) * D;
        double qv[4096 / kSrThreads];
#pragma unroll
        for (int k = 0; k < 4096 / kSrThreads; ++k) {
            const int i = tid + k * kSrThreads;
            qv[k] = i < G * D ? qs[i] : 0.0;
        }
        if (sg < SG) {
            const float4* pp = reinterpret_cast<const float4*>(
                    p.partials + (size_t)bb * p.wps * R + (size_t)kv * D) + cq;
            double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
            for (int s0 = sg; s0 < np; s0 += 16 * SG) {
                float4 x[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) x[k] = pp[(size_t)min(s0 + k * SG, np - 1) * (R / 4)];
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const bool ok = s0 + k * SG < np;
                    a0 += ok ? (double)x[k].x : 0.0;
                    a1 += ok ? (double)x[k].y : 0.0;
                    a2 += ok ? (double)x[k].z : 0.0;
                    a3 += ok ? (double)x[k].w : 0.0;
                }
            }
            red2[sg * D + 4 * cq + 0] = a0;
            red2[sg * D + 4 * cq + 1] = a1;
            red2[sg * D + 4 * cq + 2] = a2;
            red2[sg * D + 4 * cq + 3] = a3;
        }
#pragma unroll
        for (int k = 0; k < 4096 / kSrThreads; ++k) {
            const int i = tid + k * kSrThreads;
            if (i < G * D) qn[i] = sqrt(qv[k]);
        }
        __syncthreads();
        if (tid < D) {
            double K2 = 0.0;
            for (int r = 0; r < SG; ++r) K2 += red2[r * D + tid];
            double qsum = 0.0;
            for (int g = 0; g < G; ++g) qsum += qn[g * D + tid];
            const float sc = (float)(sqrt(K2) * qsum);
            if (p.scores) p.scores[((size_t)bb * p.Hkv + kv) * D + tid] = sc;
            s_sc[tid] = sc;
        }
        __syncthreads();
        const size_t row = (size_t)bb * p.Hkv + kv;
        uint32_t* s_mask = reinterpret_cast<uint32_t*>(cut + 4);      // [8]
        int32_t* const tie = p.near_tie ? p.near_tie + row : nullptr;
        if (D == 128)
            select_row<128, kSrThreads>(s_sc, D, p.keep, kSrThreads, scratch, cut,
                                        p.kept_idx + row * p.keep, tie, s_mask);
        else
            select_row<0, kSrThreads>(s_sc, D, p.keep, kSrThreads, scratch, cut,
                                      p.kept_idx + row * p.keep, tie, s_mask);
        __syncthreads();
        const int nw = (D + 15) / 16;
        if (tid < nw)
            __hip_atomic_store(p.selected + row * nw + tid,
                               (tag << 16) | ((s_mask[tid / 2] >> (16 * (tid % 2))) & 0xffffu),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- phase 3: the thin rows of the tile, from the registers
    const int keep = p.keep, Ro = p.Hkv * keep;
    constexpr int SK = NV < kSrSubK ? NV : kSrSubK;           // k-slices per sub-tile
    T* rows = reinterpret_cast<T*>(lds);                      // [SK * 512 vectors]
    uint16_t* srcmap = reinterpret_cast<uint16_t*>(lds + SK * kSrThreads);
    uint32_t* kmask = reinterpret_cast<uint32_t*>(srcmap + (Ro + 7) / 8 * 8);   // [Hkv][nw]
    const int Dh = DC > 0 ? DC : p.D;
    const int nw = (Dh + 15) / 16;
    T* k_thin = static_cast<T*>(p.k_thin);
    const int sub_rows = SK * kSrThreads / nvec;              // token rows per sub-tile
    // Whole thin rows of 16-byte chunks (Ro*e a multiple of 16, so every row
    // starts on a chunk): thread tid always builds chunk cp of rows rr,
    // rr + rpp, ...; its CE source channels are the same for every row, read
    // from the source map once.  (Worked out before the wait for the kept
    // channels, which they do not depend on.)
    const int cpr = Ro / CE;
    const bool whole = Ro % CE == 0 && cpr <= kSrThreads;
    const int rpp = whole ? kSrThreads / cpr : 1;
    const bool builds = whole && tid < rpp * cpr;
    const int cp = builds ? tid % cpr : 0;
    const int rr = builds ? tid / cpr : (1 << 30);            // threads past rpp*cpr: none
    // phase 2's LDS is free once its mask chunks are published (with 4 vectors
    // per thread the arrays below start at 32 KiB and can reach them)
    __syncthreads();
    for (int o = tid; o < Ro; o += kSrThreads) srcmap[o] = 0;  // only a torn mask leaves gaps
    {
        unsigned long long* words = p.selected + (size_t)b * p.Hkv * nw;
        for (int i = tid; i < p.Hkv * nw; i += kSrThreads) {
            unsigned long long x = 0;
            for (uint32_t spin = 0;; ++spin) {
                x = __hip_atomic_load(words + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((x >> 16) == want) break;
                if (spin >= p.spin_limit) {
                    __hip_atomic_store(p.err, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
            kmask[i] = (uint32_t)x & 0xffffu;
        }
    }
    __syncthreads();
    // srcmap[kv*keep + j] = kv*D + (the j-th kept channel of head kv): one
    // thread per 16-bit chunk counts the kept channels of the chunks below it,
    // then hands out the next slots to its own kept channels in ascending order
    for (int i = tid; i < p.Hkv * nw; i += kSrThreads) {
        const int kv = i / nw, wi = i - kv * nw;
        int j = 0;                               // kept channels of the chunks below
#pragma unroll
        for (int x = 0; x < 16; ++x) {           // every read in range, all issued at once
            const uint32_t w = kmask[kv * nw + (x < nw ? x : 0)];
            j += x < wi ? __popc(w) : 0;
        }
        for (uint32_t m = kmask[i]; m != 0u; m &= m - 1u) {
            const int c = wi * 16 + __builtin_ctz(m);
            if (j < keep && c < Dh) srcmap[kv * keep + j] = (uint16_t)(kv * Dh + c);
            ++j;
        }
    }
    int src[CE];
    __syncthreads();                                          // srcmap built
#pragma unroll
    for (int k = 0; k < CE; ++k) src[k] = builds ? srcmap[cp * CE + k] : 0;
#pragma unroll
    for (int s = 0; s < NV / SK; ++s) {
        const int r0 = s * sub_rows;
        if (r0 >= nt) break;                                  // uniform
        __syncthreads();                                      // rows free
#pragma unroll
        for (int kk = 0; kk < SK; ++kk) lds[tid + kk * kSrThreads] = v[SK * s + kk];
        __syncthreads();
        const int ns = min(sub_rows, nt - r0);
        if (whole) {
            T* dst = k_thin + ((size_t)b * p.s_cap + t0 + r0) * Ro + (size_t)cp * CE;
            for (int r = rr; r < ns; r += rpp) {
                union { uint4 q; T e[CE]; } pack;
#pragma unroll
                for (int k = 0; k < CE; ++k) pack.e[k] = rows[r * R + src[k]];
                __builtin_nontemporal_store(u32x4_t{pack.q.x, pack.q.y, pack.q.z, pack.q.w},
                                            reinterpret_cast<u32x4_t*>(dst + (size_t)r * Ro));
            }
            continue;
        }
        const size_t E0 = ((size_t)b * p.s_cap + t0 + r0) * Ro;
        const size_t E1 = E0 + (size_t)ns * Ro;
        const size_t c0 = E0 / CE, c1 = (E1 + CE - 1) / CE;
        for (size_t ch = c0 + tid; ch < c1; ch += kSrThreads) {
            const size_t lo = ch * CE;
            if (lo >= E0 && lo + CE <= E1) {
                const int f = (int)(lo - E0);
                int r = f / Ro, o = f - r * Ro;
                union { uint4 q; T e[CE]; } pack;
#pragma unroll
                for (int k = 0; k < CE; ++k) {
                    pack.e[k] = rows[r * R + srcmap[o]];
                    if (++o == Ro) { o = 0; ++r; }
                }
                __builtin_nontemporal_store(u32x4_t{pack.q.x, pack.q.y, pack.q.z, pack.q.w},
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
}

// dynamic LDS of every phase: phase 1 [512][EPV] fp64 (32 KiB), phase 2
// [SG][D] + [G][D] fp64 and the selection scratch, phase 3 the sub-tile (up
// to 128 KiB) and the source map
size_t sr_lds_bytes(const think_dims& d, int keep, int nv) {
    const int D = d.head_dim, G = d.n_q_heads / d.n_kv_heads;
    const size_t p1 = (size_t)kSrThreads * (16 / elem_bytes(d.dtype)) * sizeof(double);
    const size_t p2 = ((size_t)kSrThreads * 4 + (size_t)G * D) * sizeof(double) + 256 * 4 +
                      kSrThreads * 4 + 16 + 32;
    const int sk = nv < kSrSubK ? nv : kSrSubK;
    const size_t p3 = (size_t)sk * kSrThreads * 16 +
                      ((size_t)d.n_kv_heads * keep + 7) / 8 * 16 +
                      (size_t)d.n_kv_heads * ((D + 15) / 16) * 8;
    size_t m = p1 > p2 ? p1 : p2;
    return m > p3 ? m : p3;
}

template <int DT, int NV>
const void* sr_kernel(int D) {
    return D == 128 ? reinterpret_cast<const void*>(&k_score_compact_resident<DT, NV, 128>)
                    : reinterpret_cast<const void*>(&k_score_compact_resident<DT, NV, 0>);
}

const void* sr_kernel_for(int dtype, int nv, int D) {
    if (dtype == THINK_BF16) {
        switch (nv) {
            case 4: return sr_kernel<THINK_BF16, 4>(D);
            case 8: return sr_kernel<THINK_BF16, 8>(D);
            case 16: return sr_kernel<THINK_BF16, 16>(D);
            case 32: return sr_kernel<THINK_BF16, 32>(D);
        }
    } else {
        switch (nv) {
            case 4: return sr_kernel<THINK_F32, 4>(D);
            case 8: return sr_kernel<THINK_F32, 8>(D);
            case 16: return sr_kernel<THINK_F32, 16>(D);
            case 32: return sr_kernel<THINK_F32, 32>(D);
        }
    }
    return nullptr;
}

// test hook (think_single_read_test_give_up): this thread's launches wait for
// a tag nobody writes and give up after a few polls
thread_local bool g_sr_test_give_up = false;

// the call's share of the tag: a process-wide counter seeded from the clock,
// 24 bits, never 0
unsigned long long next_tag() {
    static std::atomic<unsigned long long> counter{
            (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count()};
    for (;;) {
        const unsigned long long t = counter.fetch_add(1) & 0xffffffull;
        if (t) return t;
    }
}

}  // namespace

void set_single_read_test_give_up(bool on) { g_sr_test_give_up = on; }

SingleReadGeom single_read_geom(const think_dims& d, int keep) {
    SingleReadGeom g{};
    const int e = elem_bytes(d.dtype);
    const int nvec = d.n_kv_heads * d.head_dim * e / 16;
    const int R = d.n_kv_heads * d.head_dim;
    g.part_bytes = ((size_t)kSrMaxWorkgroups * R * sizeof(float) + 15) / 16 * 16;
    g.q2_offset = g.part_bytes;
    g.bar_offset = g.q2_offset +
                   ((size_t)d.batch * d.n_q_heads * d.head_dim * sizeof(double) + 15) / 16 * 16;
    // tile flags [kSrMaxWorkgroups], mask words [B][Hkv][ceil(D/16)], the error
    // word and the launch generation
    g.err_offset = g.bar_offset +
                   ((size_t)kSrMaxWorkgroups +
                    (size_t)d.batch * d.n_kv_heads * ((d.head_dim + 15) / 16)) * 8;
    g.ws_bytes = g.err_offset + 16;
    // shape conditions of the kernel (the device's share is decided at launch)
    g.shape_ok = nvec <= kSrThreads && kSrThreads % nvec == 0 &&
                 (d.n_q_heads / d.n_kv_heads) * d.head_dim <= 4096 &&
                 d.batch * d.n_kv_heads <= kSrMaxWorkgroups && d.batch <= kSrMaxWorkgroups &&
                 sr_lds_bytes(d, keep, 32) <= 163840;
    return g;
}

// Whether the current device can hold every tile at once; if so, the vectors
// per thread (nv), the workgroups per sequence (wps) and the token rows per
// workgroup (rpw) of the launch.
bool single_read_plan(const think_dims& d, int keep, const SingleReadGeom& g, SrPlan* plan) {
    if (!g.shape_ok) return false;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    const int nvec = d.n_kv_heads * d.head_dim * elem_bytes(d.dtype) / 16;
    int slots = ncu < kSrMaxWorkgroups ? ncu : kSrMaxWorkgroups;
    const int wps = slots / d.batch;
    // every (b, kv) row is selected by workgroup b*Hkv + kv of the grid
    if (wps < 1 || d.n_kv_heads > wps) return false;
    const int rpw = (d.seq_capacity + wps - 1) / wps;
    const int64_t need = (int64_t)rpw * nvec;    // vectors per tile
    int nv = 0;
    for (int c : {4, 8, 16, 32})
        if ((int64_t)c * kSrThreads >= need) { nv = c; break; }
    if (!nv) return false;
    const size_t lds = sr_lds_bytes(d, keep, nv);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sr_kernel_for(d.dtype, nv, d.head_dim),
                                                     kSrThreads, lds) != hipSuccess ||
        per_cu < 1)
        return false;
    plan->nv = nv;
    plan->wps = wps;
    plan->rpw = rpw;
    plan->lds = lds;
    return true;
}

hipError_t launch_single_read(const think_dims& d, const SingleReadGeom& g, const SrPlan& pl,
                              const void* k_cache, const int32_t* seq_lens,
                              const void* q_obs, int W, float* scores, int keep,
                              int32_t* kept_idx, int32_t* near_tie, void* k_thin,
                              void* workspace, hipStream_t s) {
    SrParams p{};
    char* ws = static_cast<char*>(workspace);
    p.k_vec = static_cast<const uint4*>(k_cache);
    p.seq_lens = seq_lens;
    p.q_vec = static_cast<const uint4*>(q_obs);
    p.partials = reinterpret_cast<float*>(ws);
    p.q2 = reinterpret_cast<double*>(ws + g.q2_offset);
    p.scores = scores;
    p.kept_idx = kept_idx;
    p.near_tie = near_tie;
    p.k_thin = k_thin;
    p.tile_done = reinterpret_cast<unsigned long long*>(ws + g.bar_offset);
    p.selected = p.tile_done + kSrMaxWorkgroups;
    p.err = p.selected + (size_t)d.batch * d.n_kv_heads * ((d.head_dim + 15) / 16);
    p.gen = p.err + 1;
    p.tag = next_tag();
    p.spin_limit = kSrSpinLimit;
    if (g_sr_test_give_up) {      // test hook: every wait runs out after a few polls
        p.want_xor = 1ull << 47;
        p.spin_limit = 4;
    }
    p.s_cap = d.seq_capacity;
    p.nvec = d.n_kv_heads * d.head_dim * elem_bytes(d.dtype) / 16;
    p.rpw = pl.rpw;
    p.wps = pl.wps;
    p.nb = d.batch;
    p.W = W;
    p.nqv = d.n_q_heads * d.head_dim * elem_bytes(d.dtype) / 16;
    p.Hq = d.n_q_heads;
    p.Hkv = d.n_kv_heads;
    p.D = d.head_dim;
    p.keep = keep;
    void* args[] = {&p};
    return hipLaunchKernel(sr_kernel_for(d.dtype, pl.nv, d.head_dim), dim3(d.batch * pl.wps),
                           dim3(kSrThreads), args, pl.lds, s);
}

}  // namespace thinkkv
