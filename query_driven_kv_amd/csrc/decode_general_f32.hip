// decode_general_f32.hip - the general decode chunk pass built for f32 inputs
// (the kernel is in decode_general_impl.h; one source per dtype so the two
// sets of tile shapes compile in parallel).
#include "decode_general_impl.h"

namespace thinkkv {

hipError_t launch_decode_general_f32(const think_dims& d, int chunk, int nsplit, int rec,
                                     const void* q, const void* k_thin, const void* v_cache,
                                     const int32_t* seq_lens, const int32_t* kept_idx, int keep,
                                     float scale, float* partials, int32_t* stash, hipStream_t s) {
    return launch_general<THINK_F32>(d, chunk, nsplit, rec, q, k_thin, v_cache, seq_lens, kept_idx,
                                     keep, scale, partials, stash, s);
}

int general_blocks_per_cu_f32(const think_dims& d, int keep) {
    return general_blocks_per_cu<THINK_F32>(d, keep);
}

}  // namespace thinkkv
