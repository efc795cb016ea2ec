// decode_general.h - the general chunk pass of stage (d), declarations shared
// by decode.hip (geometry, dispatch, combine) and the two sources that build
// the kernel for fp32 and bf16 inputs (decode_general_f32.hip,
// decode_general_bf16.hip; the kernel itself is in decode_general_impl.h).
//
// "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
// Technical framework, last step: attention on the thinner key cache, values
// unpruned.  Per (b, q head h), kv = h / G:
//   l_t = scale * sum_j q[b,h,idx_j] * K_thin[b,t,kv,j],  out = softmax(l) . V[b,:,kv,:]
#pragma once

#include <type_traits>

#include "think_common.h"

namespace thinkkv {

constexpr int kGenThreads = 256;   // threads per workgroup
constexpr int kGenChunk = 256;     // tokens per workgroup (one chunk slot), halved down to 64
                                   // while the halved grid still fits the GPU's resident workgroups
constexpr int kGenMaxG = 16;       // query heads per kv head

// Logits and running maxima of fp32 inputs are kept in fp64: with fp32 inputs
// of large magnitude (a logit of a few hundred has an fp32 ulp of 3e-5) an
// fp32 logit alone would spend the fp32 accuracy bound on its rounding.  The
// record's maximum is stored as its fp32 rounding plus the fp32 residual (in
// the record's third word).  bf16 inputs keep fp32 throughout.
template <int DT>
using LogitT = typename std::conditional<DT == THINK_F32, double, float>::type;

// Tile shape of one call of the general chunk pass.
struct GeneralTile {
    int tt;    // tokens per tile: 32, or 64 when a tile's loads fit in few registers
    int vr;    // value quads per thread and tile
    int kb;    // key unit bytes: the largest of 16, 8 (and 4 for bf16) dividing keep * elem_bytes,
               // else one element
    int kr;    // key units per thread and tile
    int gm;    // head slots: 4 or 16
    int kp;    // keep rounded up to whole 4-channel chunks per logit lane
    int ks;    // LDS row stride (words) of the key tile
};

GeneralTile general_tile(const think_dims& d, int keep);
size_t general_lds_bytes(const think_dims& d, int keep, const GeneralTile& t);

// Tokens per chunk of the general pass for a call of these dims and keep.
int general_chunk(const think_dims& d, int keep);

// Workgroups of the call's general-pass instance one compute unit holds at
// once, 0 if the runtime cannot say (no device).
int general_blocks_per_cu_f32(const think_dims& d, int keep);
int general_blocks_per_cu_bf16(const think_dims& d, int keep);

// One launch of the general chunk pass (grid nsplit x Hkv x B, 256 threads,
// `chunk` tokens a workgroup), writing the same partial records as the
// matrix-core kernel.
hipError_t launch_decode_general_f32(const think_dims& d, int chunk, int nsplit, int rec,
                                     const void* q, const void* k_thin, const void* v_cache,
                                     const int32_t* seq_lens, const int32_t* kept_idx, int keep,
                                     float scale, float* partials, int32_t* stash, hipStream_t s);
hipError_t launch_decode_general_bf16(const think_dims& d, int chunk, int nsplit, int rec,
                                      const void* q, const void* k_thin, const void* v_cache,
                                      const int32_t* seq_lens, const int32_t* kept_idx, int keep,
                                      float scale, float* partials, int32_t* stash, hipStream_t s);

}  // namespace thinkkv
