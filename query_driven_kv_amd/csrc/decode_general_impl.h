// decode_general_impl.h - the general chunk pass of stage (d): any dtype, any
// head_dim that is a multiple of 8 up to 256, any keep, G <= 16.  Included by
// decode_general_f32.hip and decode_general_bf16.hip, which build one dtype
// each.
//
// Workgroup = (token chunk of 64..256, kv head, b), 256 threads; the G query heads of
// the group share every byte of K_thin and V it streams.  The chunk is walked
// in tiles of TT = 32 or 64 tokens, NB tiles in a ring of register buffers:
// while tile t computes, the loads of tiles t+1 .. t+NB-1 are in flight.
// Per tile:
//  * its thin key rows of this head (keep contiguous elements at the token
//    stride Hkv*keep) are loaded in units of KB bytes, consecutive lanes on
//    consecutive units: the largest of 16, 8 and 4 bytes that divides a row
//    (so every unit lies inside one row, aligned), else one element; stored
//    to LDS as fp32;
//  * its value rows (D contiguous elements, 16-byte aligned) are loaded as
//    4-element quads straight into registers;
//  * logits: LP = 256 / TT lanes per token; lane p sums the 4-channel chunks
//    p, p + LP, ... of the kept channels for all G heads (16-byte LDS reads of
//    the key row and of the gathered query), and the LP partial sums are
//    added with DPP lane moves;
//  * online softmax: one wave per head (lane = token), the wave maximum and
//    sum by DPP moves inside each 16-lane row and two cross-row exchanges;
//  * values: thread (column quad cq, token group tg) accumulates the G output
//    rows of its columns over its tokens, rescaled when the running maximum
//    moves; the token groups are added in order at the end.
// The prologue issues the kept-index loads with the length load, then the
// query gather and the ring's first tiles back to back, so the stream starts
// after one memory round trip past the indices.
// Loads are buffer loads bounded to the tile's valid rows, so padding rows
// (and the tiles past the chunk's end that the ring still issues) read as
// zero with no memory traffic, and their logits are masked.  Each workgroup
// writes one partial record (m, l, m - fp32(m), pad, o[D]) per query head.
#pragma once

#include <mutex>
#include <type_traits>

#include "decode_general.h"

namespace thinkkv {
namespace {

template <int DT>
__device__ __forceinline__ float elem_f32(uint32_t x) {
    if constexpr (DT == THINK_F32) return __uint_as_float(x);
    else return bf16_to_f32(x & 0xffffu);
}

// DPP lane moves inside 16-lane rows: xor 1 and xor 2 inside quads, the
// mirror of each half row (lane i <- 7 - i) and of each row (i <- 15 - i).
constexpr int kDppXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
            float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double x) {
    const long long u = __builtin_bit_cast(long long, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (long long)(unsigned)lo);
}

// sum over the LP (4 or 8) aligned lanes of a group, in every lane of it
template <int LP, typename T>
__device__ __forceinline__ T group_sum(T a) {
    a += dpp<kDppXor1>(a);
    a += dpp<kDppXor2>(a);
    if constexpr (LP == 8) a += dpp<kDppHalfMirror>(a);
    return a;
}

template <typename T>
__device__ __forceinline__ T max2(T a, T b) { return b > a ? b : a; }

// maximum and sum over the 64 lanes of the wave, in every lane
template <typename T>
__device__ __forceinline__ T wave_max(T x) {
    x = max2(x, dpp<kDppXor1>(x));
    x = max2(x, dpp<kDppXor2>(x));
    x = max2(x, dpp<kDppHalfMirror>(x));
    x = max2(x, dpp<kDppMirror>(x));
    x = max2(x, (T)__shfl_xor(x, 16));
    return max2(x, (T)__shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp<kDppXor1>(x);
    x += dpp<kDppXor2>(x);
    x += dpp<kDppHalfMirror>(x);
    x += dpp<kDppMirror>(x);
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// Ring depth from the registers one tile takes (key units + value quads).
template <int DT, int VR, int KB, int KR>
constexpr int ring_depth() {
    constexpr int regs = KR * (KB >= 4 ? KB / 4 : 1) + VR * (DT == THINK_F32 ? 4 : 2);
    return regs <= 8 ? 4 : regs <= 16 ? 3 : 2;
}

template <int DT, int TT, int VR, int KB, int KR, int GM>
__global__ __launch_bounds__(kGenThreads) void k_decode_general(
        const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ k_thin,
        const typename Elem<DT>::T* __restrict__ v_cache, const int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, int s_cap, int Hkv, int G, int D, int keep, int kp,
        int ks, float scale, int chunk, int nsplit, int rec, float* __restrict__ partials,
        int32_t* __restrict__ stash) {
    using LT = LogitT<DT>;
    constexpr int e = Elem<DT>::kBytes;
    constexpr int LP = kGenThreads / TT;         // logit lanes per token
    constexpr int KW = KB >= 4 ? KB / 4 : 1;     // registers per key unit
    constexpr int KE = KB / e;                   // elements per key unit
    constexpr int NB = ring_depth<DT, VR, KB, KR>();
    static_assert(NB >= 2 && NB <= 5, "ring depth");
    const int split = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = Hkv * G;

    // thread j < keep gathers kept channel j of the G query heads; its index
    // load is in flight with the length load
    const auto rsrc_idx = make_rsrc(kept_idx + ((size_t)b * Hkv + kv) * keep, (uint32_t)keep * 4u);
    const int cidx = __builtin_amdgcn_raw_buffer_load_b32(rsrc_idx, tid < keep ? tid * 4 : (int)kOff,
                                                          0, 0);
    const int len = clamp_len(seq_lens, b, s_cap);
    if (stash && split == 0 && kv == 0 && tid == 0) stash[b] = len;   // fused append
    const int t0 = split * chunk;
    if (t0 >= len) return;                       // the combine stops before this chunk
    const int nt = min(chunk, len - t0);

    extern __shared__ __align__(16) unsigned char smem[];
    LT* lg = reinterpret_cast<LT*>(smem);        // logits [kGenMaxG][TT]
    LT* ms = lg + kGenMaxG * TT;                 // running maxima [kGenMaxG]
    float* ls = reinterpret_cast<float*>(ms + kGenMaxG);   // running sums [kGenMaxG]
    float* al = ls + kGenMaxG;                   // this tile's rescale factors [kGenMaxG]
    float* pf = al + kGenMaxG;                   // probabilities [kGenMaxG][TT]
    float* qs = pf + kGenMaxG * TT;              // gathered query [G][kp], zero past keep
    float* kt = qs + G * kp;                     // key tile [TT][ks], zero past keep; then
                                                 // a reduction buffer [256][4]

    // this thread's key units of a tile: unit f = tid + 256 i of the tile's
    // TT x UR block is (row f / UR, unit f % UR), UR = keep * e / KB units a
    // row; rows >= TT mark slots past the block
    const int UR = keep * e / KB;
    uint32_t rj[KR];
    {
        int r = tid / UR, u = tid - (tid / UR) * UR;
        const int dr = kGenThreads / UR, du = kGenThreads - dr * UR;
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            rj[i] = ((uint32_t)(r < TT ? r : TT) << 16) | (uint32_t)u;
            u += du;
            r += dr;
            if (u >= UR) {
                u -= UR;
                ++r;
            }
        }
    }
    const int rs = Hkv * keep;                   // thin-row stride (elements)
    // value columns in quads; threads past TG * DQ (when DQ does not divide
    // 256) hold no tokens.  VR * TG >= TT (the launcher's choice of VR).
    const int DQ = D >> 2, TG = kGenThreads / DQ;   // column quads, token groups
    const int cq = tid % DQ, tg = tid < TG * DQ ? tid / DQ : TT;
    const size_t kbase = ((size_t)b * s_cap + t0) * rs + (size_t)kv * keep;
    const size_t vbase = (((size_t)b * s_cap + t0) * Hkv + kv) * (size_t)D;
    const int ntiles = (nt + TT - 1) / TT;

    using VQ = typename std::conditional<DT == THINK_F32, uint4, uint2>::type;
    uint32_t kb[NB][KR][KW];
    VQ vb[NB][VR];
    // issue tile `tile`'s loads (an empty range past the last tile: zeros, no traffic)
    auto load_tile = [&](int tile, uint32_t (&kd)[KR][KW], VQ (&vd)[VR]) {
        const int tb = tile * TT;
        const int ntt = tile < ntiles ? min(TT, nt - tb) : 0;
        const auto rk = make_rsrc(k_thin + kbase + (size_t)tb * rs,
                                  ntt > 0 ? (uint32_t)(((ntt - 1) * rs + keep) * e) : 0u);
        const auto rv = make_rsrc(v_cache + vbase + (size_t)tb * Hkv * D,
                                  ntt > 0 ? (uint32_t)(((ntt - 1) * Hkv * D + D) * e) : 0u);
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int r = (int)(rj[i] >> 16), u = (int)(rj[i] & 0xffffu);
            const uint32_t off = r < ntt ? (uint32_t)(r * rs * e + u * KB) : kOff;
            if constexpr (KB == 16) {
                const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0,
                                                                        kNonTemporal);
                kd[i][0] = w.x;
                kd[i][1] = w.y;
                kd[i][2] = w.z;
                kd[i][3] = w.w;
            } else if constexpr (KB == 8) {
                const unsigned long long w = __builtin_bit_cast(
                        unsigned long long,
                        __builtin_amdgcn_raw_buffer_load_b64(rk, (int)off, 0, kNonTemporal));
                kd[i][0] = (uint32_t)w;
                kd[i][1] = (uint32_t)(w >> 32);
            } else if constexpr (KB == 4) {
                kd[i][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, (int)off, 0, kNonTemporal);
            } else {
                kd[i][0] = __builtin_amdgcn_raw_buffer_load_b16(rk, (int)off, 0, kNonTemporal);
            }
        }
#pragma unroll
        for (int i = 0; i < VR; ++i) {
            const int r = tg + i * TG;               // >= TT for threads without tokens
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

    // the query elements the indices name, then the ring's first tiles, back
    // to back; the gathered query goes to LDS once its loads are in
    const auto rsrc_q = make_rsrc(q + ((size_t)b * Hq + (size_t)kv * G) * D, (uint32_t)(G * D * e));
    uint32_t qv[GM];
    {
        const int c = cidx < 0 ? 0 : (cidx >= D ? D - 1 : cidx);
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const int off = tid < keep && g < G ? (g * D + c) * e : (int)kOff;
            if constexpr (DT == THINK_F32)
                qv[g] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_q, off, 0, 0);
            else
                qv[g] = __builtin_amdgcn_raw_buffer_load_b16(rsrc_q, off, 0, 0);
        }
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) load_tile(u, kb[u], vb[u]);
    for (int i = tid; i < TT * (kp - keep); i += kGenThreads) {
        const int r = i / (kp - keep);
        kt[r * ks + keep + (i - r * (kp - keep))] = 0.0f;
    }
    for (int i = tid; i < G * (kp - keep); i += kGenThreads) {
        const int g = i / (kp - keep);
        qs[g * kp + keep + (i - g * (kp - keep))] = 0.0f;
    }
#pragma unroll
    for (int g = 0; g < GM; ++g)
        if (tid < keep && g < G) qs[g * kp + tid] = elem_f32<DT>(qv[g]);
    if (tid < kGenMaxG) {
        ms[tid] = -INFINITY;
        ls[tid] = 0.0f;
    }

    float o[GM][4];                              // GM >= G: 4 or 16
#pragma unroll
    for (int g = 0; g < GM; ++g) o[g][0] = o[g][1] = o[g][2] = o[g][3] = 0.0f;

    // one tile from ring slot U; the slot before it (free since the previous
    // tile) takes the loads of the tile NB - 1 ahead.  The loads are issued
    // whether or not `tile` exists (past the end they are empty), so every
    // path through the loop issues the same loads in the same order and the
    // waits before each use count exactly the NB - 1 tiles still in flight.
    // LDS reuse across tiles needs no barrier of its own: kt was last read by
    // the logits, lg by the softmax and pf / al by the values of the previous
    // tile, each followed by a barrier before this tile writes them.
    auto step = [&](int tile, auto uc) {
        constexpr int U = decltype(uc)::value;
        constexpr int P = (U + NB - 1) % NB;
        load_tile(tile + NB - 1, kb[P], vb[P]);
        if (tile >= ntiles) return;
#pragma unroll
        for (int i = 0; i < KR; ++i) {
            const int r = (int)(rj[i] >> 16), u = (int)(rj[i] & 0xffffu);
            if (r < TT) {
                float* dst = kt + r * ks + u * KE;
                if constexpr (KE == 1) {
                    dst[0] = elem_f32<DT>(kb[U][i][0]);
                } else {
#pragma unroll
                    for (int w = 0; w < KW; ++w) {
                        if constexpr (DT == THINK_F32) {
                            dst[w] = __uint_as_float(kb[U][i][w]);
                        } else {
                            dst[2 * w] = bf16_lo(kb[U][i][w]);
                            dst[2 * w + 1] = bf16_hi(kb[U][i][w]);
                        }
                    }
                }
            }
        }
        __syncthreads();

        const int ntt = min(TT, nt - tile * TT);
        // logits: token r = tid / LP; lane p = tid % LP takes the 4-channel
        // chunks p, p + LP, ... (kp / 4 chunks, zero past keep)
        {
            const int r = tid / LP, pp = tid % LP;
            LT acc[GM];
#pragma unroll
            for (int g = 0; g < GM; ++g) acc[g] = 0;
            const float* krow = kt + r * ks;
#pragma unroll 2
            for (int c = 4 * pp; c < kp; c += 4 * LP) {
                const float4 x = *reinterpret_cast<const float4*>(krow + c);
#pragma unroll
                for (int g = 0; g < GM; ++g) {
                    if (g < G) {
                        const float4 y = *reinterpret_cast<const float4*>(qs + g * kp + c);
                        LT a = acc[g];
                        a = fma((LT)y.x, (LT)x.x, a);
                        a = fma((LT)y.y, (LT)x.y, a);
                        a = fma((LT)y.z, (LT)x.z, a);
                        acc[g] = fma((LT)y.w, (LT)x.w, a);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (g < G) {
                    const LT a = group_sum<LP>(acc[g]);
                    if (pp == 0) lg[g * TT + r] = a * (LT)scale;
                }
            }
        }
        __syncthreads();

        // online softmax, one wave per head
        for (int g = wave; g < G; g += kGenThreads / 64) {
            const bool ok = lane < ntt;
            const LT x = ok ? lg[g * TT + lane] : (LT)-INFINITY;
            const LT mx = wave_max(x);
            const LT mo = ms[g];
            const LT mn = mx > mo ? mx : mo;
            const float a = mo == (LT)-INFINITY ? 0.0f : expf((float)(mo - mn));
            const float pe = ok ? expf((float)(x - mn)) : 0.0f;
            if (lane < TT) pf[g * TT + lane] = pe;
            const float sum = wave_sum(pe);
            if (lane == 0) {
                ms[g] = mn;
                ls[g] = ls[g] * a + sum;
                al[g] = a;
            }
        }
        __syncthreads();

        // values
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                const float a = al[g];
#pragma unroll
                for (int c = 0; c < 4; ++c) o[g][c] *= a;
#pragma unroll
                for (int i = 0; i < VR; ++i) {
                    const int r = tg + i * TG;
                    const float pv = r < TT ? pf[g * TT + r] : 0.0f;
                    float vf[4];
                    if constexpr (DT == THINK_F32) {
                        vf[0] = __uint_as_float(vb[U][i].x);
                        vf[1] = __uint_as_float(vb[U][i].y);
                        vf[2] = __uint_as_float(vb[U][i].z);
                        vf[3] = __uint_as_float(vb[U][i].w);
                    } else {
                        vf[0] = bf16_lo(vb[U][i].x);
                        vf[1] = bf16_hi(vb[U][i].x);
                        vf[2] = bf16_lo(vb[U][i].y);
                        vf[3] = bf16_hi(vb[U][i].y);
                    }
#pragma unroll
                    for (int c = 0; c < 4; ++c) o[g][c] = fmaf(pv, vf[c], o[g][c]);
                }
            }
        }
    };
    for (int tile = 0; tile < ntiles; tile += NB) {
        step(tile, std::integral_constant<int, 0>{});
        step(tile + 1, std::integral_constant<int, 1>{});
        if constexpr (NB > 2) step(tile + 2, std::integral_constant<int, 2 % NB>{});
        if constexpr (NB > 3) step(tile + 3, std::integral_constant<int, 3 % NB>{});
        if constexpr (NB > 4) step(tile + 4, std::integral_constant<int, 4 % NB>{});
    }

    // records: (m, l, m - fp32(m)) and o, the token groups added in order
    __syncthreads();                             // the last tile's reads of kt are done
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

}  // namespace

template <int DT>
using GeneralKernel = void (*)(const typename Elem<DT>::T*, const typename Elem<DT>::T*,
                               const typename Elem<DT>::T*, const int32_t*, const int32_t*, int,
                               int, int, int, int, int, int, float, int, int, int, float*,
                               int32_t*);

// The instance for a tile shape (nullptr for a shape no instance covers).
// Only the (TT, VR, KB, KR) combinations that keep <= head_dim <= 256 can
// reach are built.  32-token tiles: 16-byte key units number
// ceil(keep * e / 128) a thread, at most VR (fp32) or VR / 2 (bf16); 8- and
// 4-byte units (taken at KR 4, 8 or 16) at most 2 VR; one-element units
// ceil(keep / 8), at most 4 * VR (8 when VR <= 2).  64-token tiles are chosen
// only with 16-byte units, KR <= 2 and VR <= 4 (VR 8 for bf16).
template <int DT>
GeneralKernel<DT> general_kernel(const GeneralTile& t) {
    auto pick = [&](auto ttc, auto vrc, auto kbc, auto krc) -> GeneralKernel<DT> {
        constexpr int TT = decltype(ttc)::value, VR = decltype(vrc)::value,
                      KB = decltype(kbc)::value, KR = decltype(krc)::value;
        if (t.gm == 4) return k_decode_general<DT, TT, VR, KB, KR, 4>;
        return k_decode_general<DT, TT, VR, KB, KR, kGenMaxG>;
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I4 = std::integral_constant<int, 4>;
    using I8 = std::integral_constant<int, 8>;
    using I16 = std::integral_constant<int, 16>;
    using I32 = std::integral_constant<int, 32>;
    using I64 = std::integral_constant<int, 64>;
    using KE = std::integral_constant<int, Elem<DT>::kBytes>;
    auto tile32 = [&](auto vrc) -> GeneralKernel<DT> {
        constexpr int VR = decltype(vrc)::value;
        constexpr int kmax16 = DT == THINK_F32 ? VR : (VR > 1 ? VR / 2 : 1);
        constexpr int kmax84 = 2 * VR < 4 ? 4 : 2 * VR;
        constexpr int kmax1 = VR > 2 ? 4 * VR : 8;
        if (t.kb == 16) {
            if (t.kr > kmax16) return nullptr;
            if constexpr (kmax16 >= 8) if (t.kr == 8) return pick(I32{}, vrc, I16{}, I8{});
            if constexpr (kmax16 >= 4) if (t.kr == 4) return pick(I32{}, vrc, I16{}, I4{});
            if constexpr (kmax16 >= 2) if (t.kr == 2) return pick(I32{}, vrc, I16{}, I2{});
            return pick(I32{}, vrc, I16{}, I1{});
        }
        if (t.kb == 8 || (t.kb == 4 && DT == THINK_BF16)) {
            if (t.kr > kmax84) return nullptr;
            auto by_kr = [&](auto kbc) -> GeneralKernel<DT> {
                if constexpr (kmax84 >= 16) if (t.kr == 16) return pick(I32{}, vrc, kbc, I16{});
                if constexpr (kmax84 >= 8) if (t.kr == 8) return pick(I32{}, vrc, kbc, I8{});
                return pick(I32{}, vrc, kbc, I4{});
            };
            if (t.kb == 8) return by_kr(I8{});
            if constexpr (DT == THINK_BF16) return by_kr(I4{});
            return nullptr;
        }
        if (t.kr > kmax1) return nullptr;
        if constexpr (kmax1 >= 32) if (t.kr == 32) return pick(I32{}, vrc, KE{}, I32{});
        if constexpr (kmax1 >= 16) if (t.kr == 16) return pick(I32{}, vrc, KE{}, I16{});
        return pick(I32{}, vrc, KE{}, I8{});
    };
    auto tile64 = [&](auto vrc) -> GeneralKernel<DT> {
        if (t.kb != 16 || t.kr > 2) return nullptr;
        return t.kr == 2 ? pick(I64{}, vrc, I16{}, I2{}) : pick(I64{}, vrc, I16{}, I1{});
    };
    if (t.tt == 64) {
        switch (t.vr) {
            case 8:                              // bf16 only (8 quads of 8 bytes)
                if constexpr (DT == THINK_BF16) return tile64(I8{});
                return nullptr;
            case 4: return tile64(I4{});
            case 2: return tile64(I2{});
            case 1: return tile64(I1{});
            default: return nullptr;
        }
    }
    switch (t.vr) {
        case 8: return tile32(I8{});
        case 4: return tile32(I4{});
        case 2: return tile32(I2{});
        default: return tile32(I1{});
    }
}

// Workgroups of the call's instance that one compute unit holds at once
// (registers and LDS), or 0 when it cannot be asked (no device).  Answers are
// kept per (instance, LDS bytes, device) so a call asks the runtime once.
template <int DT>
int general_blocks_per_cu(const think_dims& d, int keep) {
    const GeneralTile t = general_tile(d, keep);
    const GeneralKernel<DT> fn = general_kernel<DT>(t);
    const size_t lds = general_lds_bytes(d, keep, t);
    int dev = 0;
    if (!fn || hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();                 // leave no error behind for the next call
        return 0;
    }
    struct Entry {
        const void* fn;
        size_t lds;
        int dev, n;
    };
    static std::mutex mu;
    static Entry cache[128];
    static int used = 0;
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == reinterpret_cast<const void*>(fn) && cache[i].lds == lds &&
            cache[i].dev == dev)
            return cache[i].n;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn),
                                                     kGenThreads, lds) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (used < 128) cache[used++] = Entry{reinterpret_cast<const void*>(fn), lds, dev, n};
    return n;
}

template <int DT>
hipError_t launch_general(const think_dims& d, int chunk, int nsplit, int rec, const void* q,
                          const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                          const int32_t* kept_idx, int keep, float scale, float* partials,
                          int32_t* stash, hipStream_t s) {
    using T = typename Elem<DT>::T;
    const GeneralTile t = general_tile(d, keep);
    const GeneralKernel<DT> fn = general_kernel<DT>(t);
    if (!fn) return hipErrorInvalidValue;
    fn<<<dim3(nsplit, d.n_kv_heads, d.batch), kGenThreads, general_lds_bytes(d, keep, t), s>>>(
            (const T*)q, (const T*)k_thin, (const T*)v_cache, seq_lens, kept_idx, d.seq_capacity,
            d.n_kv_heads, d.n_q_heads / d.n_kv_heads, d.head_dim, keep, t.kp, t.ks, scale, chunk,
            nsplit, rec, partials, stash);
    return hipGetLastError();
}

}  // namespace thinkkv
