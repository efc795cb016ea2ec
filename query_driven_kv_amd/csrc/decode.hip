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
#include <atomic>
#include <mutex>
#include <type_traits>

#include "think_common.h"

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

// The general chunk pass (any dtype, any head_dim that is a multiple of 8 up
// to 256, any keep, G <= 16): workgroup = (256-token chunk, kv head, b), the
// chunk walked in tiles of kTT = 32 tokens.  Per tile:
//  * the tile's thin key rows of this head (keep contiguous elements each, at
//    the token stride Hkv*keep) are loaded with consecutive lanes on
//    consecutive elements and stored to LDS as fp32 (row stride keep + 1, so
//    the logit reads below hit different banks);
//  * its value rows (D contiguous elements, 16-byte aligned) are loaded as
//    4-element quads straight into registers; both loads of the next tile are
//    issued while this tile computes;
//  * logits: 8 threads per token, each summing every 8th kept channel for all
//    G heads, the 8 partial sums added across lanes;
//  * online softmax: one wave per head (lane = token);
//  * values: thread (column quad cq, token group tg) accumulates the G output
//    rows of its columns over its tokens, rescaled when the running maximum
//    moves; the token groups are added in order at the end.
// Loads are buffer loads bounded to the tile's valid rows, so padding rows
// read as zero and their logits are masked.
constexpr int kTT = 32;

template <int DT>
__device__ __forceinline__ float elem_f32(uint32_t x) {
    if constexpr (DT == THINK_F32) return __uint_as_float(x);
    else return bf16_to_f32(x & 0xffffu);
}

template <int DT, int VR, int KR, int GM>
__global__ __launch_bounds__(kThreads) void k_decode_partial(
        const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k_thin,
        const typename Elem<DT>::T* __restrict__ v_cache, const int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, int s_cap, int Hkv, int G, int D, int keep,
        float scale, int nsplit, int rec, float* __restrict__ partials,
        int32_t* __restrict__ stash) {
    using E = Elem<DT>;
    using LT = LogitT<DT>;
    constexpr int e = E::kBytes;
    const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
    const int len = clamp_len(seq_lens, b, s_cap);
    if (stash && split == 0 && kv == 0 && threadIdx.x == 0) stash[b] = len;   // fused append
    const int t0 = split * kChunk;
    if (t0 >= len) return;                       // the combine stops before this chunk
    const int nt = min(kChunk, len - t0);
    const int Hq = Hkv * G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    extern __shared__ __align__(16) unsigned char smem[];
    LT* lg = reinterpret_cast<LT*>(smem);        // logits [kMaxG][kTT]
    LT* ms = lg + kMaxG * kTT;                   // running maxima [kMaxG]
    float* ls = reinterpret_cast<float*>(ms + kMaxG);   // running sums [kMaxG]
    float* al = ls + kMaxG;                      // this tile's rescale factors [kMaxG]
    float* pf = al + kMaxG;                      // probabilities [kMaxG][kTT]
    float* qs = pf + kMaxG * kTT;                // gathered query [G][keep]
    float* kt = qs + G * keep;                   // thin key rows [kTT][keep + 1], then a
    const int ks = keep + 1;                     // reduction buffer [kThreads][4]

    for (int i = tid; i < G * keep; i += kThreads) {
        const int g = i / keep, j = i - g * keep;
        int c = kept_idx[((size_t)b * Hkv + kv) * keep + j];
        c = c < 0 ? 0 : (c >= D ? D - 1 : c);
        qs[i] = E::load(q, ((size_t)b * Hq + kv * G + g) * D + c);
    }
    if (tid < kMaxG) {
        ms[tid] = -INFINITY;
        ls[tid] = 0.0f;
    }

    // this thread's key elements of a tile: element f = tid + 256 i of the
    // tile's kTT x keep block is (row f / keep, channel f % keep)
    uint32_t rj[KR];
    {
        int r = tid / keep, j = tid - (tid / keep) * keep;
        const int dr = kThreads / keep, dj = kThreads - dr * keep;
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            rj[i] = ((uint32_t)r << 16) | (uint32_t)j;
            j += dj;
            r += dr;
            if (j >= keep) {
                j -= keep;
                ++r;
            }
        }
    }
    const int rs = Hkv * keep;                   // thin-row stride (elements)
    // value columns in quads; threads past TG * DQ (when DQ does not divide
    // 256) hold no tokens.  VR * TG >= kTT (the launcher's choice of VR).
    const int DQ = D >> 2, TG = kThreads / DQ;   // column quads, token groups
    const int cq = tid % DQ, tg = tid < TG * DQ ? tid / DQ : kTT;
    const size_t kbase = ((size_t)b * s_cap + t0) * rs + (size_t)kv * keep;
    const size_t vbase = (((size_t)b * s_cap + t0) * Hkv + kv) * (size_t)D;
    const int ntiles = (nt + kTT - 1) / kTT;

    using VQ = typename std::conditional<DT == THINK_F32, uint4, uint2>::type;
    uint32_t kr[KR];
    VQ vq[VR], vn[VR];
    // issue tile `tile`'s loads (an empty range past the last tile: zeros, no traffic)
    auto load_tile = [&](int tile, uint32_t (&kd)[KR], VQ (&vd)[VR]) {
        const int tb = tile * kTT;
        const int ntt = tile < ntiles ? min(kTT, nt - tb) : 0;
        const auto rk = make_rsrc(k_thin + kbase + (size_t)tb * rs,
                                  ntt > 0 ? (uint32_t)(((ntt - 1) * rs + keep) * e) : 0u);
        const auto rv = make_rsrc(v_cache + vbase + (size_t)tb * Hkv * D,
                                  ntt > 0 ? (uint32_t)(((ntt - 1) * Hkv * D + D) * e) : 0u);
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int r = (int)(rj[i] >> 16), j = (int)(rj[i] & 0xffffu);
            const uint32_t off = r < ntt ? (uint32_t)((r * rs + j) * e) : kOff;
            if constexpr (DT == THINK_F32)
                kd[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)off, 0, kNonTemporal);
            else
                kd[i] = __builtin_amdgcn_raw_buffer_load_b16(rk, (int)off, 0, kNonTemporal);
        }
#pragma unroll
        for (int i = 0; i < VR; ++i) {
            const int r = tg + i * TG;               // >= kTT for threads without tokens
            const uint32_t off = r < ntt ? (uint32_t)((r * Hkv * D + 4 * cq) * e) : kOff;
            if constexpr (DT == THINK_F32) {
                const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0,
                                                                        kNonTemporal);
                vd[i] = make_uint4(w.x, w.y, w.z, w.w);
            } else {
                const unsigned long long w =
                        __builtin_bit_cast(unsigned long long,
                                           __builtin_amdgcn_raw_buffer_load_b64(rv, (int)off, 0,
                                                                                kNonTemporal));
                vd[i] = make_uint2((uint32_t)w, (uint32_t)(w >> 32));
            }
        }
    };
    load_tile(0, kr, vq);

    float o[GM][4];                              // GM >= G: 4 or 16
#pragma unroll
    for (int g = 0; g < GM; ++g) o[g][0] = o[g][1] = o[g][2] = o[g][3] = 0.0f;

    for (int tile = 0; tile < ntiles; ++tile) {
        const int ntt = min(kTT, nt - tile * kTT);
        __syncthreads();                         // LDS of the previous tile is free
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int r = (int)(rj[i] >> 16), j = (int)(rj[i] & 0xffffu);
            if (r < kTT) kt[r * ks + j] = elem_f32<DT>(kr[i]);
        }
        __syncthreads();
        load_tile(tile + 1, kr, vn);             // in flight while this tile computes

        // logits: token r = tid / 8, channels j = p, p + 8, ... (p = tid % 8)
        {
            const int r = tid >> 3, pp = tid & 7;
            LT acc[GM];
#pragma unroll
            for (int g = 0; g < GM; ++g) acc[g] = 0;
            for (int j = pp; j < keep; j += 8) {
                const LT x = (LT)kt[r * ks + j];
#pragma unroll
                for (int g = 0; g < GM; ++g)
                    if (g < G) acc[g] = fma((LT)qs[g * keep + j], x, acc[g]);
            }
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (g < G) {
                    LT a = acc[g];
                    a += __shfl_xor(a, 1);
                    a += __shfl_xor(a, 2);
                    a += __shfl_xor(a, 4);
                    if (pp == 0) lg[g * kTT + r] = a * (LT)scale;
                }
            }
        }
        __syncthreads();

        // online softmax, one wave per head
        for (int g = wave; g < G; g += kThreads / 64) {
            const bool ok = lane < ntt;
            const LT x = ok ? lg[g * kTT + lane] : (LT)-INFINITY;
            LT mx = x;
            for (int off = 32; off > 0; off >>= 1) {
                const LT y = __shfl_xor(mx, off);
                mx = y > mx ? y : mx;
            }
            const LT mo = ms[g];
            const LT mn = mx > mo ? mx : mo;
            const float a = mo == (LT)-INFINITY ? 0.0f : expf((float)(mo - mn));
            const float pe = ok ? expf((float)(x - mn)) : 0.0f;
            if (lane < kTT) pf[g * kTT + lane] = pe;
            float sum = pe;
            for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
            if (lane == 0) {
                ms[g] = mn;
                ls[g] = ls[g] * a + sum;
                al[g] = a;
            }
        }
        __syncthreads();

        // values
        float vf[VR][4];
#pragma unroll
        for (int i = 0; i < VR; ++i) {
            if constexpr (DT == THINK_F32) {
                vf[i][0] = __uint_as_float(vq[i].x);
                vf[i][1] = __uint_as_float(vq[i].y);
                vf[i][2] = __uint_as_float(vq[i].z);
                vf[i][3] = __uint_as_float(vq[i].w);
            } else {
                vf[i][0] = bf16_lo(vq[i].x);
                vf[i][1] = bf16_hi(vq[i].x);
                vf[i][2] = bf16_lo(vq[i].y);
                vf[i][3] = bf16_hi(vq[i].y);
            }
        }
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                const float a = al[g];
#pragma unroll
                for (int c = 0; c < 4; ++c) o[g][c] *= a;
#pragma unroll
                for (int i = 0; i < VR; ++i) {
                    const int r = tg + i * TG;
                    const float pv = r < kTT ? pf[g * kTT + r] : 0.0f;
#pragma unroll
                    for (int c = 0; c < 4; ++c) o[g][c] = fmaf(pv, vf[i][c], o[g][c]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < VR; ++i) vq[i] = vn[i];
    }

    // records: (m, l, m - fp32(m)) and o, the token groups added in order
    float* red = kt;
    if (tid < G) {
        float* r = partials + (((size_t)b * Hq + kv * G + tid) * nsplit + split) * rec;
        const LT m = ms[tid];
        r[0] = (float)m;
        r[1] = ls[tid];
        r[2] = (float)(m - (LT)(float)m);        // zero for bf16
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g < G) {
            __syncthreads();
#pragma unroll
            for (int c = 0; c < 4; ++c) red[tid * 4 + c] = o[g][c];
            __syncthreads();
            if (tid < DQ) {
                float s4[4] = {0.f, 0.f, 0.f, 0.f};
                for (int t = 0; t < TG; ++t)
#pragma unroll
                    for (int c = 0; c < 4; ++c) s4[c] += red[(t * DQ + tid) * 4 + c];
                float* r = partials + (((size_t)b * Hq + kv * G + g) * nsplit + split) * rec + 4;
                *reinterpret_cast<float4*>(r + 4 * tid) = make_float4(s4[0], s4[1], s4[2], s4[3]);
            }
        }
    }
}

// dynamic LDS of the general chunk pass
size_t decode_partial_lds(const think_dims& d, int keep) {
    const int G = d.n_q_heads / d.n_kv_heads;
    const size_t lt = d.dtype == THINK_F32 ? 8 : 4;
    const size_t kt = (size_t)kTT * (keep + 1) > (size_t)kThreads * 4 ? (size_t)kTT * (keep + 1)
                                                                      : (size_t)kThreads * 4;
    return (size_t)kMaxG * kTT * lt + kMaxG * lt + 2 * kMaxG * 4 + (size_t)kMaxG * kTT * 4 +
           (size_t)G * keep * 4 + kt * 4;
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
    const size_t lds = decode_partial_lds(d, keep);
    // value rows per thread and tile: kTT tokens over 256 / (D / 4) token
    // groups, rounded up to a power of two
    const int tgs = kThreads / (d.head_dim / 4), need = (kTT + tgs - 1) / tgs;
    const int vr = need > 4 ? 8 : need > 2 ? 4 : need > 1 ? 2 : 1;
    const bool wide = keep > 64;                 // key elements per thread and tile: 8 or 32
    auto go = [&](auto dt, auto vrc, auto krc) {
        constexpr int DT = decltype(dt)::value, VR = decltype(vrc)::value,
                      KR = decltype(krc)::value;
        using T = typename Elem<DT>::T;
        if (G <= 4)
            k_decode_partial<DT, VR, KR, 4><<<grid, kThreads, lds, s>>>(
                    (const T*)q, (const T*)k_thin, (const T*)v_cache, seq_lens, kept_idx,
                    d.seq_capacity, d.n_kv_heads, G, d.head_dim, keep, scale, g.nsplit, g.rec,
                    partials, stash);
        else
            k_decode_partial<DT, VR, KR, kMaxG><<<grid, kThreads, lds, s>>>(
                    (const T*)q, (const T*)k_thin, (const T*)v_cache, seq_lens, kept_idx,
                    d.seq_capacity, d.n_kv_heads, G, d.head_dim, keep, scale, g.nsplit, g.rec,
                    partials, stash);
        return hipGetLastError();
    };
    auto by_k = [&](auto dt, auto vrc) {
        return wide ? go(dt, vrc, std::integral_constant<int, 32>{})
                    : go(dt, vrc, std::integral_constant<int, 8>{});
    };
    auto by_v = [&](auto dt) {
        switch (vr) {
            case 8: return by_k(dt, std::integral_constant<int, 8>{});
            case 4: return by_k(dt, std::integral_constant<int, 4>{});
            case 2: return by_k(dt, std::integral_constant<int, 2>{});
            default: return by_k(dt, std::integral_constant<int, 1>{});
        }
    };
    return d.dtype == THINK_BF16 ? by_v(std::integral_constant<int, THINK_BF16>{})
                                 : by_v(std::integral_constant<int, THINK_F32>{});
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
