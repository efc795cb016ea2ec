// decode.hip - stage (d): one decode step of attention on the pruned keys
// ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework, last step; the step is memory-bandwidth bound per
// "Keyformer: KV Cache Reduction through Key Tokens Selection for Efficient
// Generative Inference", original abstract).
//
//   qS[j] = q[b,h,kept_idx[b,kv,j]]
//   l_t   = scale * sum_j qS[j] * k_thin[b,t,kv,j]       t < len_b
//   out   = softmax(l) . V[b,:,kv,:]                     (values unpruned)
//
// Split-K ("flash decoding") over tokens: a workgroup owns one token chunk of
// one (b, kv head) and all G query heads of that group, so the G heads share
// every byte of K_thin and V it streams.  It writes per-head partials
// (running max m, sum l, unnormalised o[D]) to the workspace; a combine
// kernel merges the chunks of each (b, h) in ascending chunk order.
//
// This file holds the geometry, the dispatch and the combine kernel.  The
// chunk passes are the bf16 matrix-core kernel for the bandwidth-critical
// shapes (decode_mfma.hip) and the general kernel (any dtype, any keep,
// G <= 16; decode_general_impl.h, built per dtype); both write the same
// partial records.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "decode_general.h"

namespace thinkkv {

// Scratch of the allocation-free decode (think_decode_attn_static): the chunk
// pass's partial records and the stashed lengths live in this array instead of
// a caller workspace.  Each GPU holds its own copy for the life of the
// process; every call on a GPU shares it and leaves its contents behind (the
// records are written before they are read, so nothing needs clearing), so
// calls that overlap in time on one GPU race.  In host code the name is only a
// stand-in: kernels take the device address that hipGetSymbolAddress returns
// for the current device, fetched once per device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
std::atomic<int> g_cu_count[kMaxDevices];   // compute units per device, 0 until asked
}  // namespace

hipError_t static_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

// defined in decode_mfma.hip
bool mfma_decode_supported(const think_dims& d, int keep);
hipError_t launch_decode_mfma(const think_dims& d, const DecodeGeom& g, const void* q,
                              const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                              const int32_t* kept_idx, int keep, float scale, float* partials,
                              int32_t* stash, hipStream_t s);

namespace {

int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Merge the chunks of one (b, h), or of one slice of its output columns
// (blockIdx.z of gridDim.z equal slices of D/4 column quads: each slice
// reads the slots' maxima and sums and its own columns of the records, so a
// head whose records run to many kilobytes is pulled in by several compute
// units; every column's arithmetic is the same in any slicing).  The block is
// (D/4/slices) x SG threads, each thread owning four output columns (one
// 16-byte record load per slot):
// sub-group sg merges a contiguous range of the nsplit chunk slots in
// ascending order, eight at a time with a running maximum, then the SG results
// are merged pairwise in a fixed tree (log2 SG rounds; merged one after
// another by the first sub-group, 32 of them cost 3.2 us a call: D 256 at
// 32K tokens, 40.5 -> 37.2 us).  Fixed order, so the result is bitwise
// reproducible.  Fixed and per-sequence chunks: the ranges are fixed by nsplit
// rather than by the length, so the record loads do not wait for the length
// load; slots at or past the sequence's chunk count are dropped after loading
// (their contents are never used).  Balanced slots: every wave first derives
// the sequence's slot range from all B lengths (balanced_slots), then loads.
// Fused append (ap.stash set): the lengths are the ones the chunk pass
// stashed; the new token, at position len_b below capacity, is merged last as
// one more term (its logit from the kept channels of q and k_new, a fixed-
// order sum, its value row v_new), then its thin key and value rows are
// written and seq_lens[b] advanced (no workgroup of this grid reads seq_lens).
template <int DT>
__global__ __launch_bounds__(1024) void k_decode_combine(
        const float* __restrict__ partials, const int32_t* __restrict__ seq_lens, int s_cap,
        int chunk, int mode, int nsplit, int rec, int D, int sg_count,
        typename Elem<DT>::T* __restrict__ out, AppendArgs ap) {
    using E = Elem<DT>;
    using MT = LogitT<DT>;
    constexpr MT kNone = -3.402823466e38f;      // finite stand-in for an empty maximum
    const int h = blockIdx.x, b = blockIdx.y, Hq = gridDim.x, nb = gridDim.y;
    const int tid = threadIdx.x;
    const int D4 = (D >> 2) / gridDim.z;         // column quads of this slice
    const int d4 = tid % D4, sg = tid / D4;
    const int q4 = blockIdx.z * D4 + d4;         // the thread's column quad in the row
    const float* base = partials + ((size_t)b * Hq + h) * nsplit * rec;
    const int32_t* lens = ap.stash ? ap.stash : seq_lens;
    int nrange = nsplit, used = 0;               // slots in the ranges; used: balanced only
    int len_raw = 0;
    if (mode == kBalanced) {
        const int lane = tid & 63;   // lanes past B read zero
        const int lr = __builtin_amdgcn_raw_buffer_load_b32(
                make_rsrc(lens, (uint32_t)nb * 4u), lane * 4, 0, 0);
        const SeqSlots ss = balanced_slots(lr < 0 ? 0 : (lr > s_cap ? s_cap : lr), nsplit * nb,
                                           kDecodeUnit, kDecodeMinChunk);
        const int first = __builtin_amdgcn_readfirstlane(__shfl(ss.first, b));
        used = __builtin_amdgcn_readfirstlane(__shfl(ss.used, b));
        base = partials + ((size_t)h * nsplit * nb + first) * rec;
        nrange = used;
    } else {
        len_raw = lens[b];
    }
    const int lo = (int)((unsigned)(sg * nrange) / (unsigned)sg_count);
    const int hi = (int)((unsigned)((sg + 1) * nrange) / (unsigned)sg_count);
    MT M = kNone;
    float L = 0.0f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = lo; s0 < hi; s0 += 8) {
        MT mk[8];
        float lk[8];
        float4 ov[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float* r = base + (size_t)min(s0 + k, nrange - 1) * rec;
            if constexpr (DT == THINK_F32) {
                const float4 h4 = *reinterpret_cast<const float4*>(r);
                mk[k] = (MT)h4.x + (MT)h4.z;     // maximum plus its residual
                lk[k] = h4.y;
            } else {
                const float2 h2 = *reinterpret_cast<const float2*>(r);
                mk[k] = h2.x;
                lk[k] = h2.y;
            }
            ov[k] = *reinterpret_cast<const float4*>(r + 4 + 4 * q4);
        }
        // the record loads above are issued before the length is waited on
        asm volatile("" : "+s"(len_raw)::"memory");
        const int len = len_raw < 0 ? 0 : (len_raw > s_cap ? s_cap : len_raw);
        const int cb = mode == kSeqChunk ? seq_chunk(len, chunk, nsplit) : chunk;
        const int ns = mode == kBalanced ? used : (len + cb - 1) / cb;
        MT mv[8];
        float lv[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool ok = s0 + k < hi && s0 + k < ns;
            mv[k] = ok ? mk[k] : kNone;
            lv[k] = ok ? lk[k] : 0.0f;
            if (!ok) ov[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        MT Mn = M;
#pragma unroll
        for (int k = 0; k < 8; ++k) Mn = mv[k] > Mn ? mv[k] : Mn;
        const float f = expf((float)(M - Mn));
        L *= f;
        O.x *= f;
        O.y *= f;
        O.z *= f;
        O.w *= f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float w = expf((float)(mv[k] - Mn));
            L = fmaf(w, lv[k], L);
            O.x = fmaf(w, ov[k].x, O.x);
            O.y = fmaf(w, ov[k].y, O.y);
            O.z = fmaf(w, ov[k].z, O.z);
            O.w = fmaf(w, ov[k].w, O.w);
        }
        M = Mn;
    }
    __shared__ MT sM[64];
    __shared__ float sL[64];
    __shared__ float4 sO[1024];
    __shared__ MT s_prod[256], s_dot[4];
    // fused append: the new token's logit, q . k_new over the kept channels
    // (one product per channel, summed in channel order in four runs of 64,
    // the runs added in order)
    const int Hkv = ap.n_kv_heads, kv = h / (Hq / (Hkv > 0 ? Hkv : 1));
    int lenb = 0;
    bool app = false;
    if (ap.stash) {
        lenb = ap.stash[b];
        app = lenb < s_cap;
        const int32_t* idx = ap.kept_idx + ((size_t)b * Hkv + kv) * ap.keep;
        for (int j = tid; j < 256; j += blockDim.x) {
            MT prod = 0;
            if (j < ap.keep) {
                int c = idx[j];
                c = c < 0 ? 0 : (c >= D ? D - 1 : c);
                prod = (MT)E::load((const typename E::T*)ap.q, ((size_t)b * Hq + h) * D + c) *
                       (MT)E::load((const typename E::T*)ap.k_new, ((size_t)b * Hkv + kv) * D + c);
            }
            s_prod[j] = prod;
        }
    }
    // the sub-groups' results merged pairwise in a fixed tree: in the round of
    // stride st, sub-group sg (a multiple of 2 st) takes sub-group sg + st,
    // each thread keeping its own state in registers.  A round's senders
    // publish slots that no unfinished reader of an earlier round uses, so
    // one barrier a round suffices.
    for (int st = 1; st < sg_count; st *= 2) {
        if (sg % (2 * st) == st) {
            if (d4 == 0) {
                sM[sg] = M;
                sL[sg] = L;
            }
            sO[tid] = O;
        }
        __syncthreads();
        if (sg % (2 * st) == 0 && sg + st < sg_count) {
            const MT Mb = sM[sg + st];
            const float Lb = sL[sg + st];
            const float4 Ob = sO[tid + st * D4];
            const MT Mn = Mb > M ? Mb : M;
            const float fa = L > 0.0f ? expf((float)(M - Mn)) : 0.0f;
            const float fb = Lb > 0.0f ? expf((float)(Mb - Mn)) : 0.0f;
            L = fmaf(fa, L, fb * Lb);
            O.x = fmaf(fa, O.x, fb * Ob.x);
            O.y = fmaf(fa, O.y, fb * Ob.y);
            O.z = fmaf(fa, O.z, fb * Ob.z);
            O.w = fmaf(fa, O.w, fb * Ob.w);
            M = Mn;
        }
    }
    if (ap.stash) {                              // uniform: a kernel argument
        __syncthreads();                         // s_prod complete
        if (tid < 4) {
            MT t = 0;
            for (int i = 0; i < 64; ++i) t += s_prod[tid * 64 + i];
            s_dot[tid] = t;
        }
        __syncthreads();
    }
    if (sg == 0) {
        const MT MM = M;
        float LL = L;
        float4 OO = O;
        if (app) {
            const MT lnew = (((s_dot[0] + s_dot[1]) + s_dot[2]) + s_dot[3]) * (MT)ap.scale;
            const MT Mf = lnew > MM ? lnew : MM;
            const float a = LL > 0.0f ? expf((float)(MM - Mf)) : 0.0f;
            const float wn = expf((float)(lnew - Mf));
            const size_t v0 = ((size_t)b * Hkv + kv) * D + 4 * q4;
            const typename E::T* vn = (const typename E::T*)ap.v_new;
            LL = fmaf(LL, a, wn);
            OO.x = fmaf(OO.x, a, wn * E::load(vn, v0 + 0));
            OO.y = fmaf(OO.y, a, wn * E::load(vn, v0 + 1));
            OO.z = fmaf(OO.z, a, wn * E::load(vn, v0 + 2));
            OO.w = fmaf(OO.w, a, wn * E::load(vn, v0 + 3));
        }
        const bool any = LL > 0.0f;
        const size_t o0 = ((size_t)b * Hq + h) * D + 4 * q4;
        E::store(out, o0 + 0, any ? OO.x / LL : 0.0f);
        E::store(out, o0 + 1, any ? OO.y / LL : 0.0f);
        E::store(out, o0 + 2, any ? OO.z / LL : 0.0f);
        E::store(out, o0 + 3, any ? OO.w / LL : 0.0f);
    }
    // fused append: the new token's rows (one workgroup per kv head) and the
    // advanced length, from the first column slice
    if (app && blockIdx.z == 0) {
        using T = typename E::T;
        if (h % (Hq / Hkv) == 0) {
            const int32_t* idx = ap.kept_idx + ((size_t)b * Hkv + kv) * ap.keep;
            const T* kn = (const T*)ap.k_new + ((size_t)b * Hkv + kv) * D;
            T* kt = (T*)ap.k_thin + (((size_t)b * s_cap + lenb) * Hkv + kv) * ap.keep;
            for (int j = tid; j < ap.keep; j += blockDim.x) {
                int c = idx[j];
                c = c < 0 ? 0 : (c >= D ? D - 1 : c);
                kt[j] = kn[c];
            }
            const T* vn = (const T*)ap.v_new + ((size_t)b * Hkv + kv) * D;
            T* vr = (T*)ap.v_cache + (((size_t)b * s_cap + lenb) * Hkv + kv) * D;
            for (int e = tid; e < D; e += blockDim.x) vr[e] = vn[e];
        }
        if (h == 0 && tid == 0) ap.seq_lens[b] = lenb + 1;
    }
}

}  // namespace

// Tile shape of the general chunk pass.  Value quads and key units per thread
// cover the tile (powers of two); 64-token tiles when the tile's loads take at
// most 24 registers a thread with 16-byte key units (small rows: fewer tiles,
// so less per-tile work per byte).  kp: keep rounded up to whole 4-channel
// chunks for each of the 256 / TT logit lanes; ks: the key tile's LDS row
// stride, kp or kp + 4 * LP so that it is an odd number of lane-group spans
// and the 16-byte logit reads of neighbouring rows fall in different banks.
GeneralTile general_tile(const think_dims& d, int keep) {
    GeneralTile t{};
    const int e = d.dtype == THINK_F32 ? 4 : 2;
    const int D = d.head_dim;
    const int row = keep * e;                    // bytes of a thin row
    t.kb = row % 16 == 0 ? 16 : row % 8 == 0 ? 8 : row % 4 == 0 && e == 2 ? 4 : e;
    t.gm = d.n_q_heads / d.n_kv_heads <= 4 ? 4 : kGenMaxG;
    auto vr_for = [&](int tt) {
        const int tgs = kGenThreads / (D / 4);
        return pow2_at_least((tt + tgs - 1) / tgs);
    };
    auto kr_for = [&](int tt) {
        const int units = tt * (keep * e / t.kb);
        const int k = pow2_at_least((units + kGenThreads - 1) / kGenThreads);
        return t.kb == 16 ? k : t.kb > e ? (k < 4 ? 4 : k) : (k < 8 ? 8 : k);
    };
    t.tt = 32;
    if (t.kb == 16) {
        const int vr = vr_for(64), kr = kr_for(64);
        if (vr <= (e == 2 ? 8 : 4) && kr <= 2 && kr * 4 + vr * (e == 4 ? 4 : 2) <= 24) t.tt = 64;
    }
    t.vr = vr_for(t.tt);
    t.kr = kr_for(t.tt);
    const int span = 4 * (kGenThreads / t.tt);
    t.kp = (keep + span - 1) / span * span;
    t.ks = (t.kp / span) % 2 == 1 ? t.kp : t.kp + span;
    return t;
}

size_t general_lds_bytes(const think_dims& d, int keep, const GeneralTile& t) {
    const int G = d.n_q_heads / d.n_kv_heads;
    const size_t lt = d.dtype == THINK_F32 ? 8 : 4;
    const size_t kt = (size_t)t.tt * t.ks > (size_t)kGenThreads * 4 ? (size_t)t.tt * t.ks
                                                                   : (size_t)kGenThreads * 4;
    return (size_t)kGenMaxG * t.tt * lt + kGenMaxG * lt + 2 * kGenMaxG * 4 +
           (size_t)kGenMaxG * t.tt * 4 + (size_t)G * t.kp * 4 + kt * 4;
}

// 256 tokens a workgroup, halved (down to 64) while the halved chunk's
// workgroups all fit on the GPU at once (the instance's workgroups per compute
// unit times the compute units): a call that fills less than one wave of
// resident workgroups leaves per-tile latency uncovered, one that spills into
// a second wave pays a tail (bf16 D 256, 4 kv heads, 32K tokens: 512 -> 1024
// workgroups at four a unit, 46.3 -> 42.0 us; fp32 D 128, 32 kv heads, 4K
// tokens, three a unit: stays at 512, 38.1 us at 1024 against 32.4).  Without a
// device to ask (a size query on a host with no GPU) the chunk stays 256.
int general_chunk(const think_dims& d, int keep) {
    const int per_cu = d.dtype == THINK_BF16 ? general_blocks_per_cu_bf16(d, keep)
                                             : general_blocks_per_cu_f32(d, keep);
    int dev = 0;
    if (per_cu <= 0 || hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kGenChunk;
    }
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            return kGenChunk;
        }
        g_cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    const int64_t resident = (int64_t)per_cu * cus;
    auto wgs = [&](int c) {
        return (int64_t)((d.seq_capacity + c - 1) / c) * d.n_kv_heads * d.batch;
    };
    int chunk = kGenChunk;
    while (chunk > 64 && wgs(chunk / 2) <= resident) chunk /= 2;
    return chunk;
}

// Tokens per workgroup of the matrix-core chunk pass: a multiple of 128 (one
// 32-token step per wave), sized for about 512 workgroups (two per CU) and at
// most 256 chunks per sequence.  A batch of 2..64 sequences with 16-byte
// aligned thin rows of at most 64 channels (an instance small enough for three
// workgroups per CU) is sized for about 768: measured faster there (8 x 16K,
// keep 64: 75.7 -> 71.7 us), while one sequence streams best at two per CU
// (128K: 69 -> 71.5 us at 768).  Floor: 512 tokens (four steps per wave) for
// those batches, so the prologue and the merge stay small next to the stream
// (8 x 4K x 8 heads: 27.6 us, 31.2 at a 256 floor); for one sequence (or more
// than 64) the floor is what gives about one workgroup per CU, between 128
// and 512, so a small call still spreads over the chip (4K x 8 heads, keep 64:
// 15.5 -> 12.2 us; 8K x 8 heads 16.0 -> 13.8; 4K x 32 heads keeps 512).
// The head-dim-64 instance moves half the value bytes per 32-token step with
// the same instructions, so its single sequences are sized for about 256
// workgroups, one per CU (32K x 8 heads 17.7 -> 17.2 us, 128K 43.5 -> 41.9;
// at head_dim 128, 256 workgroups lose: 128K 67.7 -> 72.2 us).
int mfma_decode_chunk(const think_dims& d, int keep) {
    const bool balanced = d.batch >= 2 && d.batch <= 64;
    const bool three = balanced && keep % 8 == 0 && keep <= 64;
    const int64_t wgs = three ? 768 : (!balanced && d.head_dim == 64 ? 256 : 512);
    const int64_t work = (int64_t)d.seq_capacity * d.n_kv_heads * d.batch;
    int64_t chunk = (work + wgs - 1) / wgs;
    const int64_t min_chunk = ((int64_t)d.seq_capacity + 255) / 256;
    if (chunk < min_chunk) chunk = min_chunk;
    chunk = (chunk + 127) / 128 * 128;
    int64_t floor = kDecodeMinChunk;
    if (!balanced) {
        floor = ((work + 255) / 256 + 127) / 128 * 128;
        if (floor < kDecodeUnit) floor = kDecodeUnit;
        if (floor > kDecodeMinChunk) floor = kDecodeMinChunk;
    }
    if (chunk < floor) chunk = floor;
    return (int)chunk;
}

// Column slices of the merge: doubled while one head's records (its chunk
// slots times the record size) exceed 16 KiB a slice, as long as the slices
// divide the D/4 column quads and keep at least 8 of them (32 columns).  One
// compute unit pulls records in at a few tens of GB/s; at 32K tokens slicing
// took 0.3-1.1 us off a call (D 256, 266 KiB of records a head: 41.6 -> 40.5
// us), and with the tree merge below 0.9-4.4 us.
constexpr int64_t kCombineSliceBytes = 16 * 1024;

static int combine_slices(const think_dims& d, const DecodeGeom& g) {
    const int q4 = d.head_dim / 4;
    const int64_t bytes = (int64_t)g.nsplit * g.rec * (int64_t)sizeof(float);
    int n = 1;
    while (bytes > kCombineSliceBytes * n && q4 % (2 * n) == 0 && q4 / (2 * n) >= 8) n *= 2;
    return n;
}

DecodeGeom decode_geom(const think_dims& d, int keep) {
    DecodeGeom g{};
    g.mfma = mfma_decode_supported(d, keep);
    g.mode = !g.mfma ? kFixedChunk : (d.batch >= 2 && d.batch <= 64 ? kBalanced : kSeqChunk);
    g.chunk = g.mfma ? mfma_decode_chunk(d, keep) : general_chunk(d, keep);
    g.nsplit = (d.seq_capacity + g.chunk - 1) / g.chunk;
    g.rec = d.head_dim + 4;
    g.stash_offset = (size_t)d.batch * d.n_q_heads * g.nsplit * g.rec * sizeof(float);
    g.ws_bytes = g.stash_offset + ((size_t)d.batch * sizeof(int32_t) + 15) / 16 * 16;
    return g;
}

hipError_t launch_decode_partial(const think_dims& d, const DecodeGeom& g, const void* q,
                                 const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                                 const int32_t* kept_idx, int keep, float scale, float* partials,
                                 int32_t* stash, hipStream_t s) {
    if (g.mfma)
        return launch_decode_mfma(d, g, q, k_thin, v_cache, seq_lens, kept_idx, keep, scale,
                                  partials, stash, s);
    if (d.dtype == THINK_BF16)
        return launch_decode_general_bf16(d, g.chunk, g.nsplit, g.rec, q, k_thin, v_cache,
                                          seq_lens, kept_idx, keep, scale, partials, stash, s);
    return launch_decode_general_f32(d, g.chunk, g.nsplit, g.rec, q, k_thin, v_cache, seq_lens,
                                     kept_idx, keep, scale, partials, stash, s);
}

hipError_t launch_decode(const think_dims& d, const DecodeGeom& g, const void* q,
                         const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                         const int32_t* kept_idx, int keep, float scale, void* out,
                         void* workspace, hipStream_t s) {
    float* partials = static_cast<float*>(workspace);
    hipError_t e = launch_decode_partial(d, g, q, k_thin, v_cache, seq_lens, kept_idx, keep,
                                         scale, partials, nullptr, s);
    if (e != hipSuccess) return e;
    return launch_decode_combine(d, g, seq_lens, out, partials, nullptr, s);
}

hipError_t launch_decode_combine(const think_dims& d, const DecodeGeom& g, const int32_t* seq_lens,
                                 void* out, const float* partials, const AppendArgs* app,
                                 hipStream_t s) {
    AppendArgs ap{};
    if (app) ap = *app;
    const int slices = combine_slices(d, g);
    dim3 cgrid(d.n_q_heads, d.batch, slices);
    // sub-groups: at least min(16, 1024 / D), and enough that each merges at
    // most 8 chunk slots (one batch of record loads in flight), within 1024
    // threads
    const int d4 = d.head_dim / 4 / slices;
    int sg_count = 1024 / d.head_dim;
    if (sg_count > 16) sg_count = 16;
    const int sg_slots = (g.nsplit + 7) / 8;
    if (sg_count < sg_slots) sg_count = sg_slots;
    if (sg_count > 1024 / d4) sg_count = 1024 / d4;
    if (sg_count > 64) sg_count = 64;
    const int cthreads = d4 * sg_count;
    if (d.dtype == THINK_BF16)
        k_decode_combine<THINK_BF16><<<cgrid, cthreads, 0, s>>>(
            partials, seq_lens, d.seq_capacity, g.chunk, g.mode, g.nsplit, g.rec, d.head_dim,
            sg_count, (uint16_t*)out, ap);
    else
        k_decode_combine<THINK_F32><<<cgrid, cthreads, 0, s>>>(
            partials, seq_lens, d.seq_capacity, g.chunk, g.mode, g.nsplit, g.rec, d.head_dim,
            sg_count, (float*)out, ap);
    return hipGetLastError();
}

}  // namespace thinkkv
