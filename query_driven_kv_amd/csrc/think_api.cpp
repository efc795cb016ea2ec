// think_api.cpp - host side of the C ABI declared in include/think.h:
// argument validation (before anything is enqueued), workspace sizing,
// dispatch to the gfx950 kernels and HIP-error mapping.
#include <math.h>
#include <stdint.h>

#include "think_common.h"

namespace {

thread_local int g_last_hip_error = 0;

int check_dims(const think_dims* d) {
    if (!d) return THINK_ERR_NULL;
    if (d->dtype != THINK_F32 && d->dtype != THINK_BF16) return THINK_ERR_DTYPE;
    if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
        d->seq_capacity < 1)
        return THINK_ERR_SHAPE;
    if (d->n_q_heads % d->n_kv_heads != 0) return THINK_ERR_SHAPE;
    if (d->head_dim % 8 != 0 || d->head_dim > 256) return THINK_ERR_UNSUPPORTED;
    if (d->batch > 65535) return THINK_ERR_UNSUPPORTED;
    if (d->n_q_heads / d->n_kv_heads > 16) return THINK_ERR_UNSUPPORTED;
    if ((int64_t)d->n_kv_heads * d->head_dim * thinkkv::elem_bytes(d->dtype) > 32768)
        return THINK_ERR_UNSUPPORTED;
    if (d->seq_capacity > (1 << 28)) return THINK_ERR_UNSUPPORTED;
    if ((int64_t)d->batch * d->seq_capacity > INT32_MAX) return THINK_ERR_UNSUPPORTED;
    return THINK_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return THINK_OK;
    g_last_hip_error = (int)e;
    return THINK_ERR_HIP;
}

}  // namespace

extern "C" {

int think_abi_version(void) { return THINK_ABI_VERSION; }

int32_t think_keep_from_ratio(int32_t head_dim, double prune_ratio) {
    if (head_dim < 1 || !(prune_ratio >= 0.0) || !(prune_ratio <= 1.0)) return -1;
    double k = floor((double)head_dim * (1.0 - prune_ratio) + 0.5);
    if (k < 1.0) k = 1.0;
    if (k > head_dim) k = head_dim;
    return (int32_t)k;
}

size_t think_score_workspace_bytes(const think_dims* d) {
    if (check_dims(d) != THINK_OK) return 0;
    return thinkkv::score_geom(*d).ws_bytes;
}

size_t think_decode_workspace_bytes(const think_dims* d, int32_t keep) {
    if (check_dims(d) != THINK_OK || keep < 1 || keep > d->head_dim) return 0;
    return thinkkv::decode_geom(*d, keep).ws_bytes;
}

int think_score(const think_dims* d, const void* k_cache, const int32_t* seq_lens,
                const void* q_obs, int32_t obs_window, float* scores, void* workspace,
                size_t workspace_bytes, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_cache || !seq_lens || !q_obs || !scores) return THINK_ERR_NULL;
    if (obs_window < 1) return THINK_ERR_SHAPE;
    if (!aligned16(k_cache) || !aligned16(q_obs)) return THINK_ERR_UNSUPPORTED;
    const thinkkv::ScoreGeom g = thinkkv::score_geom(*d);
    if (!workspace || workspace_bytes < g.ws_bytes || !aligned16(workspace))
        return THINK_ERR_WORKSPACE;
    return hip_status(thinkkv::launch_score(*d, g, k_cache, seq_lens, q_obs, obs_window, scores,
                                            workspace, 0, nullptr, nullptr,
                                            (hipStream_t)stream));
}

int think_score_select(const think_dims* d, const void* k_cache, const int32_t* seq_lens,
                       const void* q_obs, int32_t obs_window, int32_t keep, float* scores,
                       int32_t* kept_idx, int32_t* near_tie, void* workspace,
                       size_t workspace_bytes, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_cache || !seq_lens || !q_obs || !kept_idx) return THINK_ERR_NULL;
    if (obs_window < 1) return THINK_ERR_SHAPE;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (!aligned16(k_cache) || !aligned16(q_obs)) return THINK_ERR_UNSUPPORTED;
    const thinkkv::ScoreGeom g = thinkkv::score_geom(*d);
    if (!workspace || workspace_bytes < g.ws_bytes || !aligned16(workspace))
        return THINK_ERR_WORKSPACE;
    return hip_status(thinkkv::launch_score(*d, g, k_cache, seq_lens, q_obs, obs_window, scores,
                                            workspace, keep, kept_idx, near_tie,
                                            (hipStream_t)stream));
}

int think_select(const think_dims* d, const float* scores, int32_t keep, int32_t* kept_idx,
                 int32_t* near_tie, void* stream) {
    if (!d) return THINK_ERR_NULL;
    if (d->batch < 1 || d->n_kv_heads < 1 || d->head_dim < 1) return THINK_ERR_SHAPE;
    if (d->head_dim % 8 != 0 || d->head_dim > 256 || d->batch > 65535 || d->n_kv_heads > 65535)
        return THINK_ERR_UNSUPPORTED;
    if (!scores || !kept_idx) return THINK_ERR_NULL;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    return hip_status(
        thinkkv::launch_select(*d, scores, keep, kept_idx, near_tie, (hipStream_t)stream));
}

int think_compact_k(const think_dims* d, const void* k_cache, const int32_t* seq_lens,
                    const int32_t* kept_idx, int32_t keep, void* k_thin, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_cache || !seq_lens || !kept_idx || !k_thin) return THINK_ERR_NULL;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (!aligned16(k_cache) || !aligned16(k_thin)) return THINK_ERR_UNSUPPORTED;
    const thinkkv::CompactGeom g = thinkkv::compact_geom(*d, keep);
    return hip_status(thinkkv::launch_compact(*d, g, k_cache, seq_lens, kept_idx, keep, k_thin,
                                              (hipStream_t)stream));
}

size_t think_score_compact_workspace_bytes(const think_dims* d, int32_t keep) {
    if (check_dims(d) != THINK_OK || keep < 1 || keep > d->head_dim) return 0;
    const size_t a = thinkkv::score_geom(*d).ws_bytes;
    const size_t b = thinkkv::single_read_geom(*d, keep).ws_bytes;
    return a > b ? a : b;
}

int think_score_compact_single_read(const think_dims* d, int32_t keep) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    thinkkv::SrPlan pl;
    return thinkkv::single_read_plan(*d, keep, thinkkv::single_read_geom(*d, keep), &pl) ? 1 : 0;
}

namespace {
// the window rows of the single-read launch are read through one 32-bit buffer range
bool window_fits(const think_dims* d, int32_t obs_window) {
    return (int64_t)d->batch * obs_window * d->n_q_heads * d->head_dim *
                   thinkkv::elem_bytes(d->dtype) < ((int64_t)1 << 31);
}
}  // namespace

int think_score_compact_status(const think_dims* d, int32_t obs_window, int32_t keep,
                               const void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (obs_window < 1) return THINK_ERR_SHAPE;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    const thinkkv::SingleReadGeom sg = thinkkv::single_read_geom(*d, keep);
    const thinkkv::ScoreGeom g = thinkkv::score_geom(*d);
    const size_t need = g.ws_bytes > sg.ws_bytes ? g.ws_bytes : sg.ws_bytes;
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return THINK_ERR_WORKSPACE;
    thinkkv::SrPlan pl;
    if (!window_fits(d, obs_window) || !thinkkv::single_read_plan(*d, keep, sg, &pl))
        return THINK_OK;
    hipStream_t s = (hipStream_t)stream;
    unsigned long long err = 0;
    st = hip_status(hipMemcpyAsync(&err, (const char*)workspace + sg.err_offset, sizeof(err),
                                   hipMemcpyDeviceToHost, s));
    if (st != THINK_OK) return st;
    st = hip_status(hipStreamSynchronize(s));
    if (st != THINK_OK) return st;
    return err ? THINK_ERR_WAIT : THINK_OK;
}

int think_single_read_test_give_up(int on) {
    static thread_local int cur = 0;
    const int prev = cur;
    cur = on != 0;
    thinkkv::set_single_read_test_give_up(cur != 0);
    return prev;
}

int think_score_select_compact(const think_dims* d, const void* k_cache, const int32_t* seq_lens,
                               const void* q_obs, int32_t obs_window, int32_t keep,
                               float* scores, int32_t* kept_idx, int32_t* near_tie,
                               void* k_thin, void* workspace, size_t workspace_bytes,
                               void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_cache || !seq_lens || !q_obs || !kept_idx || !k_thin) return THINK_ERR_NULL;
    if (obs_window < 1) return THINK_ERR_SHAPE;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (!aligned16(k_cache) || !aligned16(q_obs) || !aligned16(k_thin))
        return THINK_ERR_UNSUPPORTED;
    const thinkkv::SingleReadGeom sg = thinkkv::single_read_geom(*d, keep);
    const thinkkv::ScoreGeom g = thinkkv::score_geom(*d);
    const size_t need = g.ws_bytes > sg.ws_bytes ? g.ws_bytes : sg.ws_bytes;
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return THINK_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    thinkkv::SrPlan pl;
    if (window_fits(d, obs_window) && thinkkv::single_read_plan(*d, keep, sg, &pl))
        return hip_status(thinkkv::launch_single_read(*d, sg, pl, k_cache, seq_lens,
                                                      q_obs, obs_window, scores, keep, kept_idx,
                                                      near_tie, k_thin, workspace, s));
    st = hip_status(thinkkv::launch_score(*d, g, k_cache, seq_lens, q_obs, obs_window, scores,
                                          workspace, keep, kept_idx, near_tie, s));
    if (st != THINK_OK) return st;
    return hip_status(thinkkv::launch_compact(*d, thinkkv::compact_geom(*d, keep), k_cache,
                                              seq_lens, kept_idx, keep, k_thin, s));
}

namespace {

// Validation shared by the decode entry points, in the documented order:
// dims, required pointers, keep, alignment, workspace.
int check_decode(const think_dims* d, const void* q, const void* k_thin, const void* v_cache,
                 const int32_t* seq_lens, const int32_t* kept_idx, bool need_inputs,
                 const void* out, bool need_out, int32_t keep, const void* workspace,
                 size_t workspace_bytes, thinkkv::DecodeGeom* g, bool need_new = false,
                 const void* k_new = nullptr, const void* v_new = nullptr) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!seq_lens) return THINK_ERR_NULL;
    if (need_inputs && (!q || !k_thin || !v_cache || !kept_idx)) return THINK_ERR_NULL;
    if (need_out && !out) return THINK_ERR_NULL;
    if (need_new && (!k_new || !v_new)) return THINK_ERR_NULL;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (need_inputs && (!aligned16(k_thin) || !aligned16(v_cache) || !aligned16(q)))
        return THINK_ERR_UNSUPPORTED;
    if (need_new && (!aligned16(k_new) || !aligned16(v_new))) return THINK_ERR_UNSUPPORTED;
    *g = thinkkv::decode_geom(*d, keep);
    if (!workspace || workspace_bytes < g->ws_bytes || !aligned16(workspace))
        return THINK_ERR_WORKSPACE;
    return THINK_OK;
}

}  // namespace

int think_decode_attn(const think_dims* d, const void* q, const void* k_thin,
                      const void* v_cache, const int32_t* seq_lens, const int32_t* kept_idx,
                      int32_t keep, float softmax_scale, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    thinkkv::DecodeGeom g;
    int st = check_decode(d, q, k_thin, v_cache, seq_lens, kept_idx, true, out, true, keep,
                          workspace, workspace_bytes, &g);
    if (st != THINK_OK) return st;
    return hip_status(thinkkv::launch_decode(*d, g, q, k_thin, v_cache, seq_lens, kept_idx, keep,
                                             softmax_scale, out, workspace, (hipStream_t)stream));
}

int think_decode_attn_static(const think_dims* d, const void* q, const void* k_thin,
                             const void* v_cache, const int32_t* seq_lens,
                             const int32_t* kept_idx, int32_t keep, float softmax_scale,
                             void* out, void* stream) {
    // the validation of think_decode_attn, with the scratch array standing in
    // for the workspace
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!seq_lens || !q || !k_thin || !v_cache || !kept_idx || !out) return THINK_ERR_NULL;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (!aligned16(k_thin) || !aligned16(v_cache) || !aligned16(q)) return THINK_ERR_UNSUPPORTED;
    const thinkkv::DecodeGeom g = thinkkv::decode_geom(*d, keep);
    if (g.ws_bytes > thinkkv::kStaticScratchBytes) return THINK_ERR_WORKSPACE;
    void* ws = nullptr;
    st = hip_status(thinkkv::static_scratch(&ws));
    if (st != THINK_OK) return st;
    return hip_status(thinkkv::launch_decode(*d, g, q, k_thin, v_cache, seq_lens, kept_idx, keep,
                                             softmax_scale, out, ws, (hipStream_t)stream));
}

int think_decode_attn_partial(const think_dims* d, const void* q, const void* k_thin,
                              const void* v_cache, const int32_t* seq_lens,
                              const int32_t* kept_idx, int32_t keep, float softmax_scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
    thinkkv::DecodeGeom g;
    int st = check_decode(d, q, k_thin, v_cache, seq_lens, kept_idx, true, nullptr, false, keep,
                          workspace, workspace_bytes, &g);
    if (st != THINK_OK) return st;
    return hip_status(thinkkv::launch_decode_partial(*d, g, q, k_thin, v_cache, seq_lens, kept_idx,
                                                     keep, softmax_scale, (float*)workspace,
                                                     nullptr, (hipStream_t)stream));
}

int think_decode_attn_combine(const think_dims* d, const int32_t* seq_lens, int32_t keep,
                              void* out, const void* workspace, size_t workspace_bytes,
                              void* stream) {
    thinkkv::DecodeGeom g;
    int st = check_decode(d, nullptr, nullptr, nullptr, seq_lens, nullptr, false, out, true, keep,
                          workspace, workspace_bytes, &g);
    if (st != THINK_OK) return st;
    return hip_status(thinkkv::launch_decode_combine(*d, g, seq_lens, out, (const float*)workspace,
                                                     nullptr, (hipStream_t)stream));
}

int think_append_kv(const think_dims* d, const void* k_new, const void* v_new, int32_t* seq_lens,
                    const int32_t* kept_idx, int32_t keep, void* k_thin, void* v_cache,
                    void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_new || !v_new || !seq_lens || !kept_idx || !k_thin || !v_cache) return THINK_ERR_NULL;
    if (keep < 1 || keep > d->head_dim) return THINK_ERR_KEEP;
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_thin) || !aligned16(v_cache))
        return THINK_ERR_UNSUPPORTED;
    return hip_status(thinkkv::launch_append(*d, k_new, v_new, seq_lens, kept_idx, keep, k_thin,
                                             v_cache, (hipStream_t)stream));
}

int think_append_decode_attn(const think_dims* d, const void* q, const void* k_new,
                             const void* v_new, void* k_thin, void* v_cache, int32_t* seq_lens,
                             const int32_t* kept_idx, int32_t keep, float softmax_scale,
                             void* out, void* workspace, size_t workspace_bytes, void* stream) {
    thinkkv::DecodeGeom g;
    int st = check_decode(d, q, k_thin, v_cache, seq_lens, kept_idx, true, out, true, keep,
                          workspace, workspace_bytes, &g, true, k_new, v_new);
    if (st != THINK_OK) return st;
    int32_t* stash = (int32_t*)((char*)workspace + g.stash_offset);
    st = hip_status(thinkkv::launch_decode_partial(*d, g, q, k_thin, v_cache, seq_lens, kept_idx,
                                                   keep, softmax_scale, (float*)workspace, stash,
                                                   (hipStream_t)stream));
    if (st != THINK_OK) return st;
    thinkkv::AppendArgs ap{q, k_new, v_new, kept_idx, k_thin, v_cache, seq_lens, stash, keep,
                           d->n_kv_heads, softmax_scale};
    return hip_status(thinkkv::launch_decode_combine(*d, g, seq_lens, out, (const float*)workspace,
                                                     &ap, (hipStream_t)stream));
}

size_t think_k2_state_bytes(const think_dims* d) {
    if (check_dims(d) != THINK_OK) return 0;
    return thinkkv::k2_geom(*d).bytes;
}

int think_prefill_write_kv(const think_dims* d, const void* k_rows, const void* v_rows, int32_t t0,
                           int32_t n_rows, const int32_t* seq_lens, void* k_cache, void* v_cache,
                           void* k2_state, size_t k2_state_bytes, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!k_rows || !v_rows || !seq_lens || !k_cache || !v_cache) return THINK_ERR_NULL;
    if (t0 < 0 || n_rows < 0) return THINK_ERR_SHAPE;
    if (!aligned16(k_rows) || !aligned16(v_rows) || !aligned16(k_cache) || !aligned16(v_cache))
        return THINK_ERR_UNSUPPORTED;
    const thinkkv::K2Geom g = thinkkv::k2_geom(*d);
    if (!k2_state || k2_state_bytes < g.bytes || !aligned16(k2_state)) return THINK_ERR_WORKSPACE;
    if (n_rows == 0) return THINK_OK;
    return hip_status(thinkkv::launch_prefill_write(*d, g, k_rows, v_rows, t0, n_rows, seq_lens,
                                                    k_cache, v_cache, (double*)k2_state,
                                                    (hipStream_t)stream));
}

int think_score_select_k2(const think_dims* d, const void* k2_state, size_t k2_state_bytes,
                          const void* q_obs, int32_t obs_window, int32_t keep, float* scores,
                          int32_t* kept_idx, int32_t* near_tie, void* stream) {
    int st = check_dims(d);
    if (st != THINK_OK) return st;
    if (!q_obs || (!scores && !kept_idx)) return THINK_ERR_NULL;
    if (obs_window < 1) return THINK_ERR_SHAPE;
    if (kept_idx && (keep < 1 || keep > d->head_dim)) return THINK_ERR_KEEP;
    if (!aligned16(q_obs)) return THINK_ERR_UNSUPPORTED;
    const thinkkv::K2Geom g = thinkkv::k2_geom(*d);
    if (!k2_state || k2_state_bytes < g.bytes || !aligned16(k2_state)) return THINK_ERR_WORKSPACE;
    return hip_status(thinkkv::launch_score_k2(*d, g.nslots, (const double*)k2_state, q_obs,
                                               obs_window, scores, keep, kept_idx, near_tie,
                                               (hipStream_t)stream));
}

int think_probe_stream(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                       void* stream) {
    if ((read_bytes && !src) || (write_bytes && !dst)) return THINK_ERR_NULL;
    if ((src && !aligned16(src)) || (dst && !aligned16(dst))) return THINK_ERR_UNSUPPORTED;
    if (read_bytes >= ((size_t)1 << 40) || write_bytes >= ((size_t)1 << 40))
        return THINK_ERR_UNSUPPORTED;
    if (!read_bytes && !write_bytes) return THINK_OK;
    return hip_status(
            thinkkv::launch_probe_stream(src, read_bytes, dst, write_bytes, (hipStream_t)stream));
}

const char* think_status_string(int status) {
    switch (status) {
        case THINK_OK: return "ok";
        case THINK_ERR_NULL: return "a required pointer is NULL";
        case THINK_ERR_SHAPE: return "inconsistent or out-of-range dimensions";
        case THINK_ERR_KEEP: return "keep outside [1, head_dim]";
        case THINK_ERR_DTYPE: return "unknown dtype";
        case THINK_ERR_UNSUPPORTED: return "shape, alignment or size outside what the kernels handle";
        case THINK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case THINK_ERR_HIP: return "HIP launch failed";
        case THINK_ERR_WAIT: return "a single-read launch gave up waiting; its outputs are invalid";
        default: return "unknown status";
    }
}

int think_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
