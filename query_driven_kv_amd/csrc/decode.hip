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
// This file holds the general kernel (any dtype, any keep, G <= 16) and the
// combine kernel.  The bf16 matrix-core kernel for the bandwidth-critical
// shapes is in decode_mfma.hip and writes the same partial records.
#include <type_traits>

#include "think_common.h"

namespace thinkkv {

// defined in decode_mfma.hip
bool mfma_decode_supported(const think_dims& d, int keep);
int mfma_decode_chunk(const think_dims& d, int keep);
hipError_t launch_decode_mfma(const think_dims& d, const DecodeGeom& g, const void* q,
                              const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                              const int32_t* kept_idx, int keep, float scale, float* partials,
                              int32_t* stash, hipStream_t s);

namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 256;    // tokens per workgroup (general kernel)
constexpr int kMaxG = 16;

// Logits and running maxima of fp32 inputs are kept in fp64: with fp32 inputs
// of large magnitude (a logit of a few hundred has an fp32 ulp of 3e-5) an
// fp32 logit alone would spend the fp32 accuracy bound on its rounding.  The
// record's maximum is stored as its fp32 rounding plus the fp32 residual (in
// the record's third word).  bf16 inputs keep fp32 throughout.
template <int DT>
using LogitT = typename std::conditional<DT == THINK_F32, double, float>::type;

template <int DT>
__global__ __launch_bounds__(kThreads) void k_decode_partial(
        const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k_thin,
        const typename Elem<DT>::T* __restrict__ v_cache, const int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, int s_cap, int Hkv, int G, int D, int keep,
        float scale, int nsplit, int rec, float* __restrict__ partials,
        int32_t* __restrict__ stash) {
    using E = Elem<DT>;
    const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
    const int len = clamp_len(seq_lens, b, s_cap);
    if (stash && split == 0 && kv == 0 && threadIdx.x == 0) stash[b] = len;   // fused append
    const int t0 = split * kChunk;
    if (t0 >= len) return;                       // the combine stops before this chunk
    const int nt = min(kChunk, len - t0);
    const int Hq = Hkv * G;
    const int tid = threadIdx.x;

    using LT = LogitT<DT>;
    __shared__ float qs[kMaxG * 256];            // gathered query, [g][j]
    __shared__ LT p[kMaxG * kChunk];             // logits, then probabilities, [g][t]
    __shared__ LT mrow[kMaxG];
    __shared__ float lrow[kMaxG];

    for (int i = tid; i < G * keep; i += kThreads) {
        const int g = i / keep, j = i - g * keep;
        int c = kept_idx[((size_t)b * Hkv + kv) * keep + j];
        c = c < 0 ? 0 : (c >= D ? D - 1 : c);
        qs[i] = E::load(q, ((size_t)b * Hq + kv * G + g) * D + c);
    }
    __syncthreads();

    if (tid < nt) {
        const size_t kr = (((size_t)b * s_cap + t0 + tid) * Hkv + kv) * keep;
        LT acc[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) acc[g] = 0;
        for (int j = 0; j < keep; ++j) {
            const LT x = E::load(k_thin, kr + j);
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)
                if (g < G) acc[g] = fma((LT)qs[g * keep + j], x, acc[g]);
        }
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
            if (g < G) p[g * kChunk + tid] = acc[g] * (LT)scale;
    }
    __syncthreads();

    if (tid < G) {
        LT* pr = p + tid * kChunk;
        LT m = pr[0];
        for (int t = 1; t < nt; ++t) m = pr[t] > m ? pr[t] : m;
        float l = 0.0f;
        for (int t = 0; t < nt; ++t) {
            const float e = expf((float)(pr[t] - m));
            pr[t] = e;
            l += e;
        }
        mrow[tid] = m;
        lrow[tid] = l;
    }
    __syncthreads();

    for (int d = tid; d < D; d += kThreads) {
        float o[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) o[g] = 0.0f;
        for (int t = 0; t < nt; ++t) {
            const float v = E::load(v_cache, (((size_t)b * s_cap + t0 + t) * Hkv + kv) * D + d);
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)
                if (g < G) o[g] = fmaf((float)p[g * kChunk + t], v, o[g]);
        }
#pragma unroll
        for (int g = 0; g < kMaxG; ++g)
            if (g < G)
                partials[(((size_t)b * Hq + kv * G + g) * nsplit + split) * rec + 4 + d] = o[g];
    }
    if (tid < G) {
        float* r = partials + (((size_t)b * Hq + kv * G + tid) * nsplit + split) * rec;
        const LT m = mrow[tid];
        r[0] = (float)m;
        r[1] = lrow[tid];
        r[2] = (float)(m - (LT)(float)m);        // zero for bf16
    }
}

// Merge the chunks of one (b, h).  The block is (D/4) x SG threads, each
// thread owning four output columns (one 16-byte record load per slot):
// sub-group sg merges a contiguous range of the nsplit chunk slots in
// ascending order, eight at a time with a running maximum, then the SG results
// are merged in ascending sg order.  Fixed order, so the result is bitwise
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
    const int D4 = D >> 2;
    const int d4 = tid % D4, sg = tid / D4;
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
            ov[k] = *reinterpret_cast<const float4*>(r + 4 + 4 * d4);
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
    if (d4 == 0) {
        sM[sg] = M;
        sL[sg] = L;
    }
    sO[tid] = O;
    __syncthreads();
    if (ap.stash) {                              // uniform: a kernel argument
        if (tid < 4) {
            MT t = 0;
            for (int i = 0; i < 64; ++i) t += s_prod[tid * 64 + i];
            s_dot[tid] = t;
        }
        __syncthreads();
    }
    if (sg == 0) {
        MT MM = sM[0];
        for (int r = 1; r < sg_count; ++r) MM = sM[r] > MM ? sM[r] : MM;
        float LL = 0.0f;
        float4 OO = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int r = 0; r < sg_count; ++r) {
            const float f = sL[r] > 0.0f ? expf((float)(sM[r] - MM)) : 0.0f;
            const float4 o = sO[r * D4 + d4];
            LL = fmaf(f, sL[r], LL);
            OO.x = fmaf(f, o.x, OO.x);
            OO.y = fmaf(f, o.y, OO.y);
            OO.z = fmaf(f, o.z, OO.z);
            OO.w = fmaf(f, o.w, OO.w);
        }
        if (app) {
            const MT lnew = (((s_dot[0] + s_dot[1]) + s_dot[2]) + s_dot[3]) * (MT)ap.scale;
            const MT Mf = lnew > MM ? lnew : MM;
            const float a = LL > 0.0f ? expf((float)(MM - Mf)) : 0.0f;
            const float wn = expf((float)(lnew - Mf));
            const size_t v0 = ((size_t)b * Hkv + kv) * D + 4 * d4;
            const typename E::T* vn = (const typename E::T*)ap.v_new;
            LL = fmaf(LL, a, wn);
            OO.x = fmaf(OO.x, a, wn * E::load(vn, v0 + 0));
            OO.y = fmaf(OO.y, a, wn * E::load(vn, v0 + 1));
            OO.z = fmaf(OO.z, a, wn * E::load(vn, v0 + 2));
            OO.w = fmaf(OO.w, a, wn * E::load(vn, v0 + 3));
        }
        const bool any = LL > 0.0f;
        const size_t o0 = ((size_t)b * Hq + h) * D + 4 * d4;
        E::store(out, o0 + 0, any ? OO.x / LL : 0.0f);
        E::store(out, o0 + 1, any ? OO.y / LL : 0.0f);
        E::store(out, o0 + 2, any ? OO.z / LL : 0.0f);
        E::store(out, o0 + 3, any ? OO.w / LL : 0.0f);
    }
    // fused append: the new token's rows (one workgroup per kv head) and the
    // advanced length
    if (app) {
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

DecodeGeom decode_geom(const think_dims& d, int keep) {
    DecodeGeom g{};
    g.mfma = mfma_decode_supported(d, keep);
    g.mode = !g.mfma ? kFixedChunk : (d.batch >= 2 && d.batch <= 64 ? kBalanced : kSeqChunk);
    g.chunk = g.mfma ? mfma_decode_chunk(d, keep) : kChunk;
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
    const int G = d.n_q_heads / d.n_kv_heads;
    dim3 grid(g.nsplit, d.n_kv_heads, d.batch);
    if (d.dtype == THINK_BF16)
        k_decode_partial<THINK_BF16><<<grid, kThreads, 0, s>>>(
            (const uint16_t*)q, (const uint16_t*)k_thin, (const uint16_t*)v_cache, seq_lens,
            kept_idx, d.seq_capacity, d.n_kv_heads, G, d.head_dim, keep, scale, g.nsplit, g.rec,
            partials, stash);
    else
        k_decode_partial<THINK_F32><<<grid, kThreads, 0, s>>>(
            (const float*)q, (const float*)k_thin, (const float*)v_cache, seq_lens, kept_idx,
            d.seq_capacity, d.n_kv_heads, G, d.head_dim, keep, scale, g.nsplit, g.rec, partials,
            stash);
    return hipGetLastError();
}

hipError_t launch_decode_combine(const think_dims& d, const DecodeGeom& g, const int32_t* seq_lens,
                                 void* out, const float* partials, const AppendArgs* app,
                                 hipStream_t s) {
    AppendArgs ap{};
    if (app) ap = *app;
    dim3 cgrid(d.n_q_heads, d.batch);
    int sg_count = 1024 / d.head_dim;
    if (sg_count > 16) sg_count = 16;
    const int cthreads = d.head_dim / 4 * sg_count;
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
