// decode_mfma.hip - bf16 matrix-core kernel for stage (d), head_dim 128 or 64.
//
// "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework, last step: attention runs on the thinner key cache
// while the values stay unpruned.  Per (b, q head h), kv = h / G:
//   l_t = scale * sum_j q[b,h,idx_j] * K_thin[b,t,kv,j],  out = softmax(l) . V[b,:,kv,:]
//
// Work decomposition.  Workgroup = (token chunk, kv head, b), 4 waves; each
// wave walks its quarter of the chunk 32 tokens at a time.  Chunk sizes follow
// the lengths on the device: one sequence (or more than 64) spreads its tokens
// over its nsplit chunks; a batch of 2..64 deals its B * nsplit chunk slots in
// proportion to length (balanced_slots).  Ragged batches and partly filled
// caches stay balanced.  The G <= 16 query heads of the group share every
// K_thin / V byte the wave loads.
//
// Both products run on v_mfma_f32_16x16x32_bf16 (16x16 output, K = 32):
//   logits  C[t][g] = sum_j K_thin[t][j] * qS[j][g]
//           A = K_thin rows: lane (l%16 = token, l/16 = channel octet) takes 16
//               contiguous bytes of its row (one aligned load, or assembled
//               from aligned chunks when keep is not a multiple of 8);
//               B = gathered query,
//               loaded once per wave (zero for g >= G or j >= keep).
//           C lands as lane (l%16 = g, l/16 = token quad, reg = token).
//   values  O[g][d] = sum_t P[g][t] * V[t][d]
//           A = P: exactly the registers the logits produced (lane l%16 = g,
//               8 tokens per lane), rounded to bf16 - no data movement;
//           B = V: lane (l%16 = d octet, l/16 = token quad) loads the 16-byte
//               V rows of its 8 tokens; 8 output tiles, tile c taking element c
//               of each row, re-paired per token with 16-bit permutes.  At
//               head_dim 64 the lanes of octets 8..15 read zeros and their
//               output columns are dropped (the same instruction stream moves
//               half the value bytes).
// The token order inside one 32-token step is a permutation shared by A and
// B of the value product, so no transposition through LDS is needed.
//
// Online softmax per wave (fp32), the 4 waves merged in LDS, one partial
// record (m, l, o[128]) per (b, h, chunk) for the combine kernel.  (Merging
// in the last-finishing workgroup instead needs a device-scope release per
// workgroup, an L2 write-back on this part, which costs more than the
// second launch; measured: 69 -> 89 us per 128K call.)  K_thin and V are
// read once per call: the loads are marked non-temporal, except K_thin when
// a kv head's thin row is not whole 128-byte lines (SL): then the lines it
// shares with the neighbouring heads are kept in L2 for their workgroups,
// which are numbered to run next to it on the same XCD.
// Loads are raw buffer loads whose per-step descriptors end at the last
// valid token: padding tokens (t >= len_b) read as zero and their logits are
// set to -inf, so a NaN in padding cannot leak in; no load sits behind a
// branch.
#include <type_traits>

#include "think_common.h"

namespace thinkkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kQS = 128;      // LDS row stride of the gathered query (keep <= 128)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ f32x4 mfma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Element c (0..7) of each of the 8 V rows of this lane, as one B operand.
template <int C>
__device__ __forceinline__ uint4 v_column(const uint4 (&v)[8]) {
    constexpr int w = C >> 1;
    uint32_t x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t d = w == 0 ? v[i].x : w == 1 ? v[i].y : w == 2 ? v[i].z : v[i].w;
        x[i] = d;
    }
    uint4 r;
    if (C & 1) {
        r.x = (x[0] >> 16) | (x[1] & 0xffff0000u);
        r.y = (x[2] >> 16) | (x[3] & 0xffff0000u);
        r.z = (x[4] >> 16) | (x[5] & 0xffff0000u);
        r.w = (x[6] >> 16) | (x[7] & 0xffff0000u);
    } else {
        r.x = (x[0] & 0xffffu) | (x[1] << 16);
        r.y = (x[2] & 0xffffu) | (x[3] << 16);
        r.z = (x[4] & 0xffffu) | (x[5] << 16);
        r.w = (x[6] & 0xffffu) | (x[7] << 16);
    }
    return r;
}

// K_thin octets (8 channels, 16 bytes of one head row).  KAL = 8 (keep a
// multiple of 8): head rows are 16-byte aligned and an octet is one aligned
// dwordx4.  KAL = 0 (any other keep): each lane loads the 16-byte aligned
// chunks 4*jb + q4 of its token row (lanes q4 = 0 one more, chunk 4*KB); the
// octet of block jb spans that chunk and the next one, which the lane 16
// above holds, so a lane rotation brings it in and a per-lane byte shift (the
// row's offset inside its first chunk, the same in every step) cuts the octet
// out, and the last block's channels past keep are masked.  Every K_thin load
// is an aligned dwordx4.
template <int KB, int KAL>
struct Frag {
    uint4 k[2][KAL == 0 ? KB + 1 : KB];  // token half x 32-channel block (KAL 0: x chunk)
    uint4 v[8];                          // V rows of this lane's 8 tokens (16 bytes each)
};

// Lane-constant parts of the loads of one 32-token step (byte offsets from
// the step's K_thin / V descriptor bases).  Blocks before the last lie
// inside every kept row (keep > 32 * (KB - 1)), so their chunks are a fixed
// distance above the first; only the last block's chunk and the extra one
// are checked per lane.  V rows of the lane's tokens differ by wave-uniform
// offsets, passed separately.
template <int KB>
struct LaneOffsets {
    uint32_t k0[2];      // chunk q4 of the lane's token row (chunk 4*jb + q4 is 64*jb above)
    uint32_t kt[2][2];   // chunks of the last block and the extra one; kOff when not needed
    uint32_t kr[2];      // KAL 0: the token row's byte offset inside its first chunk
    uint4 kmask;         // KAL 0: channel mask of the last block's octet
    uint32_t v0;         // V: this lane's channel octet in token row 4*q4
};

// `delta` is the K_thin descriptor base's distance below the step's first
// row of this head, which puts the base on a 16-byte boundary.  A chunk is
// loaded if it starts before the row's last kept channel ends (it then lies
// inside the descriptor's range, which is rounded up to 16 bytes); for
// KAL = 8 that is exactly "the octet holds kept channels".
template <int KB, int D>
__device__ __forceinline__ LaneOffsets<KB> lane_offsets(int keep, size_t kt_row, size_t v_row,
                                                        int n16, int q4, uint32_t delta) {
    LaneOffsets<KB> lo;
    const int j0 = (KB - 1) * 32 + 8 * q4;       // the last block's octet
    uint32_t mw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const int j = j0 + 2 * w;
        mw[w] = (j < keep ? 0x0000ffffu : 0u) | (j + 1 < keep ? 0xffff0000u : 0u);
    }
    lo.kmask = make_uint4(mw[0], mw[1], mw[2], mw[3]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t row = (uint32_t)((16 * h + n16) * kt_row * 2) + delta;
        const uint32_t r = row & 15u, al = row & ~15u;
        lo.kr[h] = r;
        lo.k0[h] = al + 16u * q4;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int jb = KB - 1 + e;
            const uint32_t k = 4u * jb + q4;
            const bool need = 16u * k < r + 2u * (uint32_t)keep && (jb < KB || q4 == 0);
            lo.kt[h][e] = need ? al + 16u * k : kOff;
        }
    }
    // head_dim 64: lanes n16 >= 8 hold no column octet and read zeros
    lo.v0 = 8 * n16 < D ? (uint32_t)((4 * q4 * v_row + 8 * n16) * 2) : kOff;
    return lo;
}

// K_thin load of one 16-byte chunk: streaming (not kept in the caches) when
// each kv head's thin row is whole 128-byte lines; kept in L2 when SL (rows
// that share their first and last lines with the neighbouring heads, which
// other workgroups on the same XCD read at about the same time).
template <bool SL>
__device__ __forceinline__ uint4 ldb_k(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, SL ? 0 : kNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Issue the loads of one 32-token step: rk / rv cover this kv head's rows of
// the step's valid tokens only, so every other read returns zero.  vs[i] is
// the wave-uniform offset of token row (i & 3) + 16 * (i >> 2) above row 0.
template <int KB, int KAL, bool SL>
__device__ __forceinline__ void load_step(Frag<KB, KAL>& f, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, const LaneOffsets<KB>& lo,
                                          const uint32_t (&vs)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int jb = 0; jb < KB - 1; ++jb) f.k[h][jb] = ldb_k<SL>(rk, lo.k0[h] + 64u * jb);
        f.k[h][KB - 1] = ldb_k<SL>(rk, lo.kt[h][0]);
        if constexpr (KAL == 0) f.k[h][KB] = ldb_k<SL>(rk, lo.kt[h][1]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)lo.v0, (int)vs[i],
                                                                kNonTemporal);
        f.v[i] = make_uint4(w.x, w.y, w.z, w.w);
    }
}

__device__ __forceinline__ uint32_t pick(bool c, uint32_t a, uint32_t b) { return c ? a : b; }

// Bytes [r, r + 16) of the 32-byte window (lo, hi), r in [0, 16): two dword
// selects (by 8 and by 4 bytes) and a byte funnel shift.  Written as scalar
// selects so that no indexed private array is formed.
__device__ __forceinline__ uint4 window16(const uint4& lo, const uint4& hi, uint32_t r) {
    const bool s8 = (r & 8u) != 0, s4 = (r & 4u) != 0;
    const uint32_t rb = r & 3u;
    const uint32_t u0 = pick(s8, lo.z, lo.x), u1 = pick(s8, lo.w, lo.y), u2 = pick(s8, hi.x, lo.z),
                   u3 = pick(s8, hi.y, lo.w), u4 = pick(s8, hi.z, hi.x), u5 = pick(s8, hi.w, hi.y);
    const uint32_t a0 = pick(s4, u1, u0), a1 = pick(s4, u2, u1), a2 = pick(s4, u3, u2),
                   a3 = pick(s4, u4, u3), a4 = pick(s4, u5, u4);
    return make_uint4(__builtin_amdgcn_alignbyte(a1, a0, rb),
                      __builtin_amdgcn_alignbyte(a2, a1, rb),
                      __builtin_amdgcn_alignbyte(a3, a2, rb),
                      __builtin_amdgcn_alignbyte(a4, a3, rb));
}

// x of the lane 16 above (wrapping within the wave).
__device__ __forceinline__ uint4 from_lane_plus16(const uint4& x, int lane) {
    const int src = ((lane + 16) & 63) << 2;
    return make_uint4(__builtin_amdgcn_ds_bpermute(src, (int)x.x),
                      __builtin_amdgcn_ds_bpermute(src, (int)x.y),
                      __builtin_amdgcn_ds_bpermute(src, (int)x.z),
                      __builtin_amdgcn_ds_bpermute(src, (int)x.w));
}

// Logits, online softmax and the value product of one 32-token step.
template <int KB, int KAL>
__device__ __forceinline__ void compute_step(const Frag<KB, KAL>& f, const LaneOffsets<KB>& lo,
                                             int nt, float scale, const uint4 (&qB)[KB], int q4,
                                             f32x4 (&O)[8], float& m, float& l) {
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (KAL == 0) {
        // chunk 4*jb + q4 + 1 is in the lane 16 above: its chunk of block jb,
        // or of block jb + 1 (chunk 0) when q4 = 3
        const int lane = threadIdx.x & 63;
        const bool wrap = q4 == 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 y[KB + 1];
#pragma unroll
            for (int jb = 0; jb <= KB; ++jb) y[jb] = from_lane_plus16(f.k[h][jb], lane);
#pragma unroll
            for (int jb = 0; jb < KB; ++jb) {
                const uint4 nx = make_uint4(
                        pick(wrap, y[jb + 1].x, y[jb].x), pick(wrap, y[jb + 1].y, y[jb].y),
                        pick(wrap, y[jb + 1].z, y[jb].z), pick(wrap, y[jb + 1].w, y[jb].w));
                const uint4 o = window16(f.k[h][jb], nx, lo.kr[h]);
                const uint4 a = jb < KB - 1 ? o
                                            : make_uint4(o.x & lo.kmask.x, o.y & lo.kmask.y,
                                                         o.z & lo.kmask.z, o.w & lo.kmask.w);
                if (h == 0)
                    c0 = mfma(a, qB[jb], c0);
                else
                    c1 = mfma(a, qB[jb], c1);
            }
        }
    } else {
#pragma unroll
        for (int jb = 0; jb < KB; ++jb) {
            c0 = mfma(f.k[0][jb], qB[jb], c0);
            c1 = mfma(f.k[1][jb], qB[jb], c1);
        }
    }
    // c0[r]: token 4*q4 + r of the step, c1[r]: token 16 + 4*q4 + r (nt of
    // the 32 are valid); head g = lane % 16
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        x[r] = 4 * q4 + r < nt ? c0[r] * scale : -INFINITY;
        x[4 + r] = 16 + 4 * q4 + r < nt ? c1[r] * scale : -INFINITY;
    }
    // online softmax for head g (the step's first token is valid: mx is finite)
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 8; ++r) mx = fmaxf(mx, x[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const float alpha = expf(m - mn);
    uint32_t pw[4];
    float ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float p0 = expf(x[2 * r] - mn), p1 = expf(x[2 * r + 1] - mn);
        pw[r] = pack_bf16(p0, p1);
        ps += bf16_lo(pw[r]) + bf16_hi(pw[r]);   // sum what the value product uses
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * alpha + ps;
    m = mn;
    // O rows are heads g = 4*q4 + i: fetch those heads' rescale factors
    float aO[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aO[i] = __shfl(alpha, 4 * q4 + i);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[c][i] *= aO[i];
    // values: A = P (k slot 8*q4+i <-> token ts + 4*q4 + (i&3) + 16*(i>>2))
    const uint4 pa = make_uint4(pw[0], pw[1], pw[2], pw[3]);
    O[0] = mfma(pa, v_column<0>(f.v), O[0]);
    O[1] = mfma(pa, v_column<1>(f.v), O[1]);
    O[2] = mfma(pa, v_column<2>(f.v), O[2]);
    O[3] = mfma(pa, v_column<3>(f.v), O[3]);
    O[4] = mfma(pa, v_column<4>(f.v), O[4]);
    O[5] = mfma(pa, v_column<5>(f.v), O[5]);
    O[6] = mfma(pa, v_column<6>(f.v), O[6]);
    O[7] = mfma(pa, v_column<7>(f.v), O[7]);
}

template <int KB, int KAL, bool SL, int D>
__global__ __launch_bounds__(kThreads, (KAL == 8 && KB <= 2) ? 3 : 2) void k_decode_mfma(
        const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_thin,
        const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ seq_lens,
        const int32_t* __restrict__ kept_idx, int s_cap, int Hkv, int G, int keep, float scale,
        int chunk, int nsplit, int rec, int mode, float* __restrict__ partials,
        int32_t* __restrict__ stash) {
    int split = blockIdx.x, kv = blockIdx.y, zb = blockIdx.z;
    if constexpr (SL) {
        // Workgroups go to the XCDs in turn by linear id; renumber so that the
        // Hkv workgroups of one token range run one after another on one XCD,
        // where the thin-row lines they share stay in its L2.
        const int nx = gridDim.x, nz = gridDim.z;
        if ((nx * nz) % 8 == 0) {
            const int L = (int)blockIdx.x + nx * ((int)blockIdx.y + Hkv * (int)blockIdx.z);
            const int xcd = L % 8, idx = L / 8;
            kv = idx % Hkv;
            const int r = (idx / Hkv) * 8 + xcd;
            split = r % nx;
            zb = r / nx;
        }
    }
    const int tid = threadIdx.x;
    // fused append: the first workgroup of each sequence records the length
    // this pass reads, for the combine (which then advances seq_lens)
    if (stash && split == 0 && kv == 0 && tid == 0) {
        const int n = seq_lens[zb];
        stash[zb] = n < 0 ? 0 : (n > s_cap ? s_cap : n);
    }
    const int Hq = Hkv * G;
    const int lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, q4 = lane >> 4;

    __shared__ __align__(16) uint16_t s_q[16 * kQS];           // gathered query [g][j]
    __shared__ float s_o[kWaves * 16 * D];       // per-wave O [w][g][d]
    __shared__ float s_m[kWaves * 16], s_l[kWaves * 16];

    // Prologue, ordered so the stream starts after one memory round trip:
    // the sequence length and this thread's kept-channel indices are loaded
    // together; then the query elements they name and the first two steps'
    // K_thin/V fragments are issued back to back, and only then does the
    // workgroup wait for the query to build the MFMA operand.
    constexpr int kGather = 16 * KB * 32 / kThreads;
    // Balanced slots (2 <= B <= 64): this workgroup is chunk slot
    // split + nsplit * zb of its kv head; every wave reads the B
    // lengths (a bounded buffer load: lanes past B read zero) and finds the
    // sequence that owns the slot and its token range.  The kept indices of
    // sequence zb are loaded meanwhile, as a guess that holds for all
    // but the slots near a share boundary; a wrong guess loads them again.
    // A slot no sequence fills exits, uniformly for the workgroup.
    // Otherwise the workgroup is chunk `split` of sequence zb.
    //
    // The gather reads through buffer descriptors bounded to this kv head's
    // kept indices and its G query rows: slots past keep or past G read zero
    // in hardware, so every load is unconditional and none waits on another.
    // A chunk that starts past the length still runs (all its stream loads
    // are empty) and writes a record the combine never reads; an early exit
    // here would put the length load in front of the gather.
    const int nb = gridDim.z, slot = split + nsplit * zb;
    int b = zb, len_raw = 0, lr = 0, len = 0, cb = 0, t0 = 0;
    if (mode == kBalanced)
        lr = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(seq_lens, (uint32_t)nb * 4u), lane * 4,
                                                  0, 0);
    else
        len_raw = seq_lens[b];
    int cidx[kGather];
    auto load_idx = [&](int bb) {
        const auto rsrc_idx =
                make_rsrc(kept_idx + ((size_t)bb * Hkv + kv) * keep, (uint32_t)keep * 4u);
#pragma unroll
        for (int r = 0; r < kGather; ++r) {
            const int j = (tid + r * kThreads) % (KB * 32);
            cidx[r] = __builtin_amdgcn_raw_buffer_load_b32(rsrc_idx, j * 4, 0, 0);
        }
    };
    load_idx(b);
    // both loads are in flight before either is waited on
    asm volatile("" ::"s"(len_raw), "v"(lr), "v"(cidx[0]));
    if (mode == kBalanced) {
        const int li = lr < 0 ? 0 : (lr > s_cap ? s_cap : lr);
        const SeqSlots ss = balanced_slots(li, nsplit * nb, kDecodeUnit, kDecodeMinChunk);
        const unsigned long long own = __ballot(ss.n > 0 && slot < ss.first + ss.n);
        if (own == 0) return;
        const int owner = __builtin_amdgcn_readfirstlane(__ffsll((long long)own) - 1);
        const int j = slot - __builtin_amdgcn_readfirstlane(__shfl(ss.first, owner));
        if (j >= __builtin_amdgcn_readfirstlane(__shfl(ss.used, owner))) return;
        len = __builtin_amdgcn_readfirstlane(__shfl(li, owner));
        cb = __builtin_amdgcn_readfirstlane(__shfl(ss.chunk, owner));
        t0 = j * cb;
        if (owner != b) {
            b = owner;
            load_idx(b);
        }
    } else {
        len = len_raw < 0 ? 0 : (len_raw > s_cap ? s_cap : len_raw);
        cb = seq_chunk(len, chunk, nsplit);
        t0 = split * cb;
    }
    const auto rsrc_q =
            make_rsrc(q + ((size_t)b * Hq + (size_t)kv * G) * D, (uint32_t)(G * D * 2));
    uint16_t qv[kGather];
#pragma unroll
    for (int r = 0; r < kGather; ++r) {
        const int i = tid + r * kThreads;
        const int g = i / (KB * 32), j = i - g * (KB * 32);
        const int c = cidx[r] < 0 ? 0 : (cidx[r] >= D ? D - 1 : cidx[r]);
        const int off = j < keep ? (g * D + c) * 2 : (int)kOff;
        qv[r] = __builtin_amdgcn_raw_buffer_load_b16(rsrc_q, off, 0, 0);
    }

    const int tw = cb / kWaves;
    const int ws = t0 + __builtin_amdgcn_readfirstlane(wave) * tw;   // wave-uniform
    const int we = min(ws + tw, len);
    const size_t kt_row = (size_t)Hkv * keep;
    const size_t v_row = (size_t)Hkv * D;
    // this wave's first rows of kv head kv; the valid bytes of a step starting
    // at token ts end at the last valid token's row.  Steps advance by 32 rows
    // of 2*Hkv*keep bytes, a multiple of 64, so the row's offset from a 16-byte
    // boundary is the same in every step: the descriptor base starts `delta`
    // bytes below the row, on that boundary (k_thin itself is 16-byte
    // aligned, so the bytes read below the row and past the range's end stay
    // within the 16-byte blocks of valid rows; for KAL = 8 delta is 0).
    const uint16_t* kw = k_thin + ((size_t)b * s_cap + ws) * kt_row + (size_t)kv * keep;
    const uint16_t* vw = v_cache + ((size_t)b * s_cap + ws) * v_row + (size_t)kv * D;
    const uint32_t delta = (uint32_t)(reinterpret_cast<uintptr_t>(kw) & 15u);
    const LaneOffsets<KB> lo = lane_offsets<KB, D>(keep, kt_row, v_row, n16, q4, delta);
    uint32_t vs[8];                              // V rows of tokens (i & 3) + 16 * (i >> 2)
#pragma unroll
    for (int i = 0; i < 8; ++i) vs[i] = (uint32_t)(((i & 3) + 16 * (i >> 2)) * v_row * 2);
    // descriptors of the step starting at token ts: empty once ts >= we (a
    // wave past the length issues only empty loads, which read zeros without
    // touching memory)
    auto rsrc_k = [&](int ts) {
        const int nt = min(32, we - ts);
        // a dword reads as zero unless it ends inside the range, so the range
        // is rounded up to whole 16-byte chunks (the extra bytes share the
        // last valid chunk and are masked)
        const uint32_t bytes =
                nt > 0 ? ((uint32_t)(((nt - 1) * kt_row + keep) * 2) + delta + 15u) & ~15u : 0u;
        return make_rsrc(reinterpret_cast<const char*>(kw + (size_t)(ts - ws) * kt_row) - delta,
                         bytes);
    };
    auto rsrc_v = [&](int ts) {
        const int nt = min(32, we - ts);
        const uint32_t bytes = nt > 0 ? (uint32_t)(((nt - 1) * v_row + D) * 2) : 0u;
        return make_rsrc(vw + (size_t)(ts - ws) * v_row, bytes);
    };

    // Two fragment buffers: the loads of step s+1 are in flight while step s
    // computes.  Both buffers are loaded unconditionally (a step past the end
    // has an empty descriptor), so the wait before each compute covers only
    // that buffer's own loads.
    Frag<KB, KAL> fa, fb;
    load_step<KB, KAL, SL>(fa, rsrc_k(ws), rsrc_v(ws), lo, vs);
    load_step<KB, KAL, SL>(fb, rsrc_k(ws + 32), rsrc_v(ws + 32), lo, vs);

#pragma unroll
    for (int r = 0; r < kGather; ++r) {
        const int i = tid + r * kThreads;
        const int g = i / (KB * 32), j = i - g * (KB * 32);
        s_q[g * kQS + j] = qv[r];
    }
    __syncthreads();
    uint4 qB[KB];                                // B operand: lane holds qS[jb*32+8*q4+i][g=n16]
#pragma unroll
    for (int jb = 0; jb < KB; ++jb)
        qB[jb] = *reinterpret_cast<const uint4*>(&s_q[n16 * kQS + jb * 32 + 8 * q4]);

    f32x4 O[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) O[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.0f;

    for (int ts = ws; ts < we; ts += 64) {
        compute_step<KB, KAL>(fa, lo, min(32, we - ts), scale, qB, q4, O, m, l);
        load_step<KB, KAL, SL>(fa, rsrc_k(ts + 64), rsrc_v(ts + 64), lo, vs);
        if (ts + 32 < we)
            compute_step<KB, KAL>(fb, lo, min(32, we - ts - 32), scale, qB, q4, O, m, l);
        load_step<KB, KAL, SL>(fb, rsrc_k(ts + 96), rsrc_v(ts + 96), lo, vs);
    }

    // ---- merge the 4 waves (a wave past len_b has m = -inf, l = 0, O = 0)
    if (q4 == 0) {
        s_m[wave * 16 + n16] = m;
        s_l[wave * 16 + n16] = l;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * q4 + i;
            if (g < G && 8 * n16 < D) s_o[(wave * 16 + g) * D + 8 * n16 + c] = O[c][i];
        }
    __syncthreads();
    for (int e = tid; e < G * D; e += kThreads) {
        const int g = e / D, d = e - g * D;
        float M = s_m[g];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w * 16 + g]);
        float L = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = expf(s_m[w * 16 + g] - M);
            L = fmaf(f, s_l[w * 16 + g], L);
            o = fmaf(f, s_o[(w * 16 + g) * D + d], o);
        }
        float* r = partials + (mode == kBalanced
                                       ? ((size_t)(kv * G + g) * nsplit * nb + slot) * rec
                                       : (((size_t)b * Hq + kv * G + g) * nsplit + split) * rec);
        r[4 + d] = o;
        if (d == 0) {
            r[0] = M;
            r[1] = L;
        }
    }

}

template <int KB, int D>
hipError_t launch_kb(int kal, dim3 grid, hipStream_t s, const uint16_t* q, const uint16_t* kt,
                     const uint16_t* v, const int32_t* lens, const int32_t* idx, int s_cap,
                     int Hkv, int G, int keep, float scale, int chunk, int nsplit, int rec,
                     int mode, float* part, int32_t* stash) {
    // thin head rows of whole 128-byte lines stream; others share lines with
    // their neighbours (keep 51 at 128K tokens: 81 -> 68 us per call)
    const bool shared_lines = (keep * 2) % 128 != 0;
    if (kal == 8 && !shared_lines)
        k_decode_mfma<KB, 8, false, D><<<grid, kThreads, 0, s>>>(
                q, kt, v, lens, idx, s_cap, Hkv, G, keep, scale, chunk, nsplit, rec, mode, part,
                stash);
    else if (kal == 8)
        k_decode_mfma<KB, 8, true, D><<<grid, kThreads, 0, s>>>(
                q, kt, v, lens, idx, s_cap, Hkv, G, keep, scale, chunk, nsplit, rec, mode, part,
                stash);
    else
        k_decode_mfma<KB, 0, true, D><<<grid, kThreads, 0, s>>>(
                q, kt, v, lens, idx, s_cap, Hkv, G, keep, scale, chunk, nsplit, rec, mode, part,
                stash);
    return hipGetLastError();
}

}  // namespace

bool mfma_decode_supported(const think_dims& d, int keep) {
    return d.dtype == THINK_BF16 && (d.head_dim == 128 || d.head_dim == 64) &&
           d.n_q_heads / d.n_kv_heads <= 16 && keep >= 1 && keep <= d.head_dim;
}

hipError_t launch_decode_mfma(const think_dims& d, const DecodeGeom& g, const void* q,
                              const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                              const int32_t* kept_idx, int keep, float scale, float* partials,
                              int32_t* stash, hipStream_t s) {
    const int G = d.n_q_heads / d.n_kv_heads;
    const int kal = keep % 8 == 0 ? 8 : 0;
    const int KB = (keep + 31) / 32;
    dim3 grid(g.nsplit, d.n_kv_heads, d.batch);
    auto qp = (const uint16_t*)q;
    auto kp = (const uint16_t*)k_thin;
    auto vp = (const uint16_t*)v_cache;
    auto go = [&](auto kb, auto dc) {
        return launch_kb<decltype(kb)::value, decltype(dc)::value>(
                kal, grid, s, qp, kp, vp, seq_lens, kept_idx, d.seq_capacity, d.n_kv_heads, G,
                keep, scale, g.chunk, g.nsplit, g.rec, g.mode, partials, stash);
    };
    if (d.head_dim == 64) {                      // keep <= 64: one or two channel blocks
        using D64 = std::integral_constant<int, 64>;
        return KB == 1 ? go(std::integral_constant<int, 1>{}, D64{})
                       : go(std::integral_constant<int, 2>{}, D64{});
    }
    using D128 = std::integral_constant<int, 128>;
    switch (KB) {
        case 1: return go(std::integral_constant<int, 1>{}, D128{});
        case 2: return go(std::integral_constant<int, 2>{}, D128{});
        case 3: return go(std::integral_constant<int, 3>{}, D128{});
        default: return go(std::integral_constant<int, 4>{}, D128{});
    }
}

}  // namespace thinkkv
