// think_common.h - internal helpers shared by the gfx950 kernels and the
// host-side ABI layer.  Not part of the public interface (see include/think.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "think.h"

namespace thinkkv {

// ---------------------------------------------------------------------------
// Element access.  bf16 is carried as its 16-bit pattern; widening to fp32 is
// exact, narrowing rounds to nearest even (inputs are finite).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int DT> struct Elem;
template <> struct Elem<THINK_F32> {
    using T = float;
    static constexpr int kBytes = 4;
    static constexpr int kPerVec = 4;   // elements per 16-byte vector
    __device__ static float load(const T* p, size_t i) { return p[i]; }
    __device__ static void store(T* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<THINK_BF16> {
    using T = uint16_t;
    static constexpr int kBytes = 2;
    static constexpr int kPerVec = 8;
    __device__ static float load(const T* p, size_t i) { return bf16_to_f32(p[i]); }
    __device__ static void store(T* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Unpack one 16-byte vector into fp32 values.
__device__ __forceinline__ void unpack(const uint4& v, float (&x)[4], Elem<THINK_F32>) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack(const uint4& v, float (&x)[8], Elem<THINK_BF16>) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// 16-byte streaming load marked non-temporal: data read once per call is
// not kept in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg_stream(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer loads: a wave-uniform descriptor (base, size in bytes) lives in
// SGPRs and each lane supplies a 32-bit byte offset.  An offset at or past
// the size reads as zero in hardware, so ranges are masked without branches
// (a load behind a branch makes the compiler drain every load in flight at
// the join).
constexpr int kRsrcWord3 = 0x00020000;          // raw buffer, 32-bit data format
constexpr int kNonTemporal = 2;                 // streaming: read once per call
constexpr uint32_t kOff = 0x80000000u;          // an offset past any descriptor

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}
__device__ __forceinline__ uint4 ldb_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ int clamp_len(const int32_t* seq_lens, int b, int s_cap) {
    int n = seq_lens[b];
    return n < 0 ? 0 : (n > s_cap ? s_cap : n);
}

// Tokens per chunk of one sequence in the matrix-core decode: a sequence's
// `len` tokens are spread over all `nsplit` chunk slots in whole 128-token
// units (4 waves x one 32-token step), at least 512 and at most `cap_chunk`
// (the chunk at full capacity), so a sequence shorter than the capacity still
// keeps every one of its workgroups streaming.  The chunk pass and the
// combine both derive the chunk from the length this way, so they agree on
// which slots hold records.
constexpr int kDecodeUnit = 128, kDecodeMinChunk = 512;
__device__ __forceinline__ int seq_chunk(int len, int cap_chunk, int nsplit) {
    int c = (int)(((unsigned)len + (unsigned)nsplit - 1u) / (unsigned)nsplit);
    c = (c + kDecodeUnit - 1) & ~(kDecodeUnit - 1);
    c = c < kDecodeMinChunk ? kDecodeMinChunk : c;
    return c > cap_chunk ? cap_chunk : c;
}

// Token-range slots of a batch of 2..64 sequences, shared in proportion to
// length.  The batch's nslots = B * nsplit slots are dealt so that every
// non-empty sequence gets one slot plus its share of the rest by length
// (boundaries floor(M * prefix / total), M = nslots - non-empty count, so the
// counts add up to nslots exactly), and its chunk is its length over its slot
// count in whole `unit`-token units (at least `min_chunk`; both powers of
// two).  Every slot then carries about the same number of tokens however
// ragged the batch is.  Called by all 64 lanes of a wave; lane i < B passes
// sequence i's clamped length (0 past B) and gets sequence i's slot count,
// first slot, chunk and used slots.  The kernel that fills the slots and the
// one that reads them both compute this, so they agree.
struct SeqSlots {
    int n;       // slots dealt to the sequence
    int first;   // its first slot
    int chunk;   // tokens per slot
    int used;    // slots that hold tokens: ceil(len / chunk) <= n
};
__device__ __forceinline__ SeqSlots balanced_slots(int len, int nslots, int unit, int min_chunk) {
    const int lane = threadIdx.x & 63;
    const int nonempty = __popcll(__ballot(len > 0));
    long long inc = len;                          // inclusive prefix of the lengths
    for (int o = 1; o < 64; o <<= 1) {
        const long long y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    const long long total = __shfl(inc, 63);
    SeqSlots r{0, 0, min_chunk, 0};
    if (len > 0) {
        // M * prefix < 2^48 and total < 2^35: the quotients are exact to well
        // within 1/total, so the floors are those of the integer division
        const double M = (double)(nslots - nonempty), T = (double)total;
        r.n = 1 + (int)floor(M * (double)inc / T) - (int)floor(M * (double)(inc - len) / T);
    }
    int ninc = r.n;                               // inclusive prefix of the slot counts
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(ninc, o);
        if (lane >= o) ninc += y;
    }
    r.first = ninc - r.n;
    if (r.n > 0) {
        int c = (len + r.n - 1) / r.n;
        c = (c + unit - 1) & ~(unit - 1);
        r.chunk = c < min_chunk ? min_chunk : c;
        r.used = (len + r.chunk - 1) / r.chunk;
    }
    return r;
}

// How the decode's chunk slots are laid out (DecodeGeom::mode).
enum DecodeMode {
    kFixedChunk = 0,   // general kernel: fixed chunk, records [B][Hq][nsplit]
    kSeqChunk = 1,     // matrix-core kernel: per-sequence chunk (seq_chunk), same records
    kBalanced = 2      // matrix-core kernel, 2 <= B <= 64: balanced_slots, records [Hq][B*nsplit]
};

inline int elem_bytes(int dtype) { return dtype == THINK_F32 ? 4 : 2; }

// ---------------------------------------------------------------------------
// Launch geometry, shared by the workspace-size queries and the launchers so
// that both always agree.
// ---------------------------------------------------------------------------
struct ScoreGeom {
    int nvec;          // 16-byte vectors per token row (Hkv*D*e/16)
    int ncg;           // column groups of <= 256 vectors
    int tpw;           // tokens per workgroup
    int nsplit;        // token splits per sequence
    bool keep_in_llc;  // read K with plain loads (it fits the last-level cache)
    size_t q2_offset;  // byte offset of the window-query sums in the workspace
    size_t ws_bytes;   // fp32 partials [B][nsplit][Hkv*D], then Q2 [B][Hq][D] fp64
};
ScoreGeom score_geom(const think_dims& d);

struct DecodeGeom {
    int chunk;        // tokens per workgroup (matrix-core kernel: at full capacity)
    int nsplit;       // splits per sequence
    int rec;          // floats per partial record: m, l, 2 pad, o[D]
    bool mfma;        // bf16 matrix-core kernel
    int mode;         // DecodeMode
    size_t stash_offset;  // byte offset of the lengths the chunk pass used (fused append)
    size_t ws_bytes;  // B * Hq * nsplit records of rec fp32, then B int32 lengths
};
DecodeGeom decode_geom(const think_dims& d, int keep);

// Decode-time append fused into the decode (think_append_decode_attn): the
// chunk pass attends over the cached tokens and stashes the lengths it used;
// the combine adds the new token as one more softmax term, writes its rows
// into the caches and advances the lengths.
struct AppendArgs {
    const void* q;             // [B, Hq, D]
    const void* k_new;         // [B, Hkv, D]
    const void* v_new;         // [B, Hkv, D]
    const int32_t* kept_idx;   // [B, Hkv, keep]
    void* k_thin;              // [B, S_cap, Hkv, keep], row len_b written
    void* v_cache;             // [B, S_cap, Hkv, D], row len_b written
    int32_t* seq_lens;         // advanced to len_b + 1 (below capacity)
    const int32_t* stash;      // the lengths the chunk pass read
    int keep;
    int n_kv_heads;
    float scale;
};

// Prefill-write state: fp64 sums of squares per (b, slot, channel).
struct K2Geom {
    int nvec;        // 16-byte vectors per token row
    int ncg;         // column groups of <= 256 vectors
    int nslots;      // row ranges per chunk (state slots per sequence)
    size_t bytes;    // state [B][nslots][Hkv*D] fp64
};
K2Geom k2_geom(const think_dims& d);

struct CompactGeom {
    int tile;        // tokens per workgroup
    size_t lds;      // dynamic LDS bytes
};
CompactGeom compact_geom(const think_dims& d, int keep);

// Single-read score + select + compaction (one launch, K held in
// registers between the phases).  Workspace: fp32 partials [<= 512 tiles][R],
// then Q2 [B][Hq][D] fp64, then the tile flags [512], the selection flags
// [B][Hkv] (64-bit) and an error word.
constexpr int kSrMaxWorkgroups = 512;
struct SingleReadGeom {
    size_t part_bytes;
    size_t q2_offset;
    size_t bar_offset;
    size_t err_offset;  // 64-bit word: the tag of the latest launch if one of its waits ran out
    size_t ws_bytes;
    bool shape_ok;     // the shape suits the kernel (the device decides the rest)
};
struct SrPlan {
    int nv;            // 16-byte vectors per thread
    int wps;           // workgroups per sequence
    int rpw;           // token rows per workgroup
    size_t lds;        // dynamic LDS bytes
};
SingleReadGeom single_read_geom(const think_dims& d, int keep);
// test hook: this thread's single-read launches give up every wait
void set_single_read_test_give_up(bool on);
bool single_read_plan(const think_dims& d, int keep, const SingleReadGeom& g, SrPlan* plan);
hipError_t launch_single_read(const think_dims& d, const SingleReadGeom& g, const SrPlan& plan,
                              const void* k_cache, const int32_t* seq_lens,
                              const void* q_obs, int W, float* scores, int keep,
                              int32_t* kept_idx, int32_t* near_tie, void* k_thin,
                              void* workspace, hipStream_t s);

// ---------------------------------------------------------------------------
// Launchers (return hipGetLastError() after enqueueing).
// ---------------------------------------------------------------------------
hipError_t launch_score(const think_dims& d, const ScoreGeom& g, const void* k_cache,
                        const int32_t* seq_lens, const void* q_obs, int W, float* scores,
                        void* workspace, int keep, int32_t* kept_idx, int32_t* near_tie,
                        hipStream_t s);   // kept_idx NULL: scores only
hipError_t launch_select(const think_dims& d, const float* scores, int keep, int32_t* kept_idx,
                         int32_t* near_tie, hipStream_t s);
hipError_t launch_compact(const think_dims& d, const CompactGeom& g, const void* k_cache,
                          const int32_t* seq_lens, const int32_t* kept_idx, int keep,
                          void* k_thin, hipStream_t s);
hipError_t launch_prefill_write(const think_dims& d, const K2Geom& g, const void* k_rows,
                                const void* v_rows, int t0, int n_rows, const int32_t* seq_lens,
                                void* k_cache, void* v_cache, double* state, hipStream_t s);
hipError_t launch_score_k2(const think_dims& d, int nslots, const double* state, const void* q_obs,
                           int W, float* scores, int keep, int32_t* kept_idx, int32_t* near_tie,
                           hipStream_t s);
hipError_t launch_append(const think_dims& d, const void* k_new, const void* v_new,
                         int32_t* seq_lens, const int32_t* kept_idx, int keep, void* k_thin,
                         void* v_cache, hipStream_t s);
// stash: NULL, or where the chunk pass stores the lengths it read (fused append)
hipError_t launch_decode_partial(const think_dims& d, const DecodeGeom& g, const void* q,
                                 const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                                 const int32_t* kept_idx, int keep, float scale, float* partials,
                                 int32_t* stash, hipStream_t s);
// The whole decode: the chunk pass, then the merge kernel into out.
hipError_t launch_decode(const think_dims& d, const DecodeGeom& g, const void* q,
                         const void* k_thin, const void* v_cache, const int32_t* seq_lens,
                         const int32_t* kept_idx, int keep, float scale, void* out,
                         void* workspace, hipStream_t s);
// Bytes of the per-device scratch array of the allocation-free decode, and its
// device address on the current device (looked up once per device).
constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
hipError_t static_scratch(void** ptr);
hipError_t launch_probe_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                               hipStream_t s);
// app: NULL, or the fused append (its stash replaces seq_lens as the lengths)
hipError_t launch_decode_combine(const think_dims& d, const DecodeGeom& g, const int32_t* seq_lens,
                                 void* out, const float* partials, const AppendArgs* app,
                                 hipStream_t s);

}  // namespace thinkkv
