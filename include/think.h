/*
 * think.h - C ABI of the MI355X (gfx950) hot path for query-driven key-cache
 * channel pruning.
 *
 * The four compute calls follow the order in which "ThinK: Thinner Key Cache
 * by Query-Driven Pruning" (Method details -> Technical framework) states the
 * method: measure each key channel's relevance to the queries, order the
 * channels and drop the least relevant, then run inference on the thinner key
 * cache.  The pages give no API, layout or formula; the readings taken here
 * are stated at each call.
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers owned by the caller.  Tensors are
 *    dense, row-major, batch-major, with 16-byte aligned base pointers.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    Calls enqueue work and return; they never synchronise the stream.
 *  - The library allocates no device memory and keeps no global state apart
 *    from a thread-local copy of the last HIP error.
 *  - Arguments are validated on the host before anything is enqueued.  On an
 *    error nothing is enqueued and a negative think_status is returned.
 *  - Outputs must not alias inputs.  Calls on different streams are
 *    independent and may run concurrently, with one exception: the
 *    single-read launch of think_score_select_compact, whose workgroups wait
 *    for one another, must not run concurrently with another such launch
 *    (two could each hold half the compute units while waiting for the
 *    other half).  Calls that share a workspace must be ordered by the
 *    caller.
 *  - `seq_lens` is device memory: int32 [B], each 1 <= len_b <= S_cap (the
 *    host cannot check device values; kernels clamp them to [0, S_cap], and a
 *    length of 0 yields zero scores / zero attention output for that batch).
 *  - All inputs must be finite.  Padding rows t >= len_b are never read.
 *  - No float atomics: every result is bitwise reproducible run to run.
 */
#ifndef THINK_H
#define THINK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define THINK_ABI_VERSION 6

#ifndef THINK_API
#define THINK_API __attribute__((visibility("default")))
#endif

typedef enum {
    THINK_OK = 0,
    THINK_ERR_NULL = -1,        /* a required pointer is NULL */
    THINK_ERR_SHAPE = -2,       /* inconsistent or out-of-range dimensions */
    THINK_ERR_KEEP = -3,        /* keep outside [1, head_dim] */
    THINK_ERR_DTYPE = -4,       /* unknown dtype code */
    THINK_ERR_UNSUPPORTED = -5, /* valid, but outside what the kernels handle */
    THINK_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than required */
    THINK_ERR_HIP = -7,         /* a HIP launch failed; see think_last_hip_error */
    THINK_ERR_WAIT = -8         /* a single-read launch gave up waiting: its outputs are invalid */
} think_status;

typedef enum { THINK_F32 = 0, THINK_BF16 = 1 } think_dtype;

/* Shape of one layer's cache.  Layouts:
 *   K, V        [B, S_cap, Hkv, D]      (key and value cache)
 *   Q_w         [B, W, Hq, D]           (observation-window queries)
 *   K_thin      [B, S_cap, Hkv, keep]   (compacted keys, dense, no padding)
 *   q, out      [B, Hq, D]              (decode query and attention output)
 * Query head h reads kv head h / G with G = Hq / Hkv (contiguous groups). */
typedef struct {
    int32_t batch;        /* B >= 1 */
    int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
    int32_t n_kv_heads;   /* Hkv >= 1 */
    int32_t head_dim;     /* D: a multiple of 8 in [8, 256] */
    int32_t seq_capacity; /* S_cap >= 1: token stride per sequence of K, V, K_thin */
    int32_t dtype;        /* think_dtype of K, V, Q_w, q, K_thin and out */
} think_dims;
/* Further limits (THINK_ERR_UNSUPPORTED): B <= 65535, Hq/Hkv <= 16,
 * Hkv*D*element_size <= 32 KiB, S_cap <= 2^28, B*S_cap < 2^31. */

/* Version of this ABI (THINK_ABI_VERSION of the built library). */
THINK_API int think_abi_version(void);

/* Channels kept at a pruning ratio r in [0, 1): round-half-up of D*(1-r),
 * clamped to [1, D].  (The pages prune a fixed fraction of channels; this
 * rounding gives 77 of 128 at 40 %, 51 at 60 %, 64 at 50 %.)  Returns -1 for
 * D < 1 or r outside [0, 1]. */
THINK_API int32_t think_keep_from_ratio(int32_t head_dim, double prune_ratio);

/* Bytes of device workspace think_score needs for these dims; 0 if invalid. */
THINK_API size_t think_score_workspace_bytes(const think_dims *d);
/* Bytes of device workspace think_decode_attn needs; 0 if invalid.  For
 * shapes the bf16 matrix-core kernel does not take (fp32, other head dims)
 * the size follows the token chunk, which is chosen from the current
 * device's compute units and the kernel's occupancy: ask on the device the
 * calls will run on (on a host without a device the answer assumes 256-token
 * chunks). */
THINK_API size_t think_decode_workspace_bytes(const think_dims *d, int32_t keep);

/*
 * Stage (a) - per-channel relevance of the key cache to the queries
 * ("ThinK", Method details -> Technical framework, first step; Key design (1):
 * relevance is read off the attention logits).  Reading: channel c of kv head
 * kv contributes the rank-1 term Q_w[:,c] K[:,c]^T to the logits; its score is
 * that term's Frobenius norm, summed over the G query heads of the group:
 *   scores[b,kv,c] = sqrt(sum_{t<len_b} K[b,t,kv,c]^2)
 *                    * sum_{g<G} sqrt(sum_{i<W} Q_w[b,i,kv*G+g,c]^2)
 * No causal mask; every token t < len_b counts.
 *   k_cache   [B,S_cap,Hkv,D] dtype    q_obs [B,W,Hq,D] dtype, W = obs_window >= 1
 *   scores    out, fp32 [B,Hkv,D]
 *   workspace >= think_score_workspace_bytes(d), 16-byte aligned, caller-owned.
 * Precision: fp32 squares summed in runs of at most 16 tokens, runs combined
 * in fp64 in a fixed order; relative error of each score below 1e-6.
 */
THINK_API int think_score(const think_dims *d, const void *k_cache, const int32_t *seq_lens,
                const void *q_obs, int32_t obs_window, float *scores, void *workspace,
                size_t workspace_bytes, void *stream);

/*
 * Stage (b) - keep the `keep` most relevant channels of every (b, kv) and
 * drop the rest ("ThinK", Technical framework, second step; original
 * abstract: prune the least significant channels).  Order: score descending,
 * ties to the lower channel index.  Output in ascending channel order.
 * Reads only batch, n_kv_heads and head_dim of d.
 *   scores    fp32 [B,Hkv,D] (non-negative, finite)
 *   kept_idx  out, int32 [B,Hkv,keep], strictly ascending
 *   near_tie  out, int32 [B,Hkv] or NULL: 1 when keep < D and the keep-th and
 *             (keep+1)-th scores s_a >= s_b satisfy s_a - s_b <= 1e-5 * s_a
 *             (evaluated in fp64), so a cutoff decision that rounding could
 *             flip is reported, not hidden.
 */
THINK_API int think_select(const think_dims *d, const float *scores, int32_t keep, int32_t *kept_idx,
                           int32_t *near_tie, void *stream);

/*
 * Stages (a) and (b) fused: the scores of think_score and the selection of
 * think_select in two launches instead of three (the selection runs in the
 * workgroup that finishes each (b, kv) row's scores).  Results are bitwise
 * those of think_score followed by think_select.  scores may be NULL (not
 * written); near_tie may be NULL.  Workspace as for think_score.
 */
THINK_API int think_score_select(const think_dims *d, const void *k_cache, const int32_t *seq_lens,
                                 const void *q_obs, int32_t obs_window, int32_t keep,
                                 float *scores, int32_t *kept_idx, int32_t *near_tie,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Stage (c) - the thinner key cache ("ThinK", title and Technical framework:
 * inference proceeds on the pruned key cache).  A byte copy:
 *   k_thin[b,t,kv,j] = k_cache[b,t,kv,kept_idx[b,kv,j]]   for t < len_b
 * Rows t >= len_b of k_thin are not written.  kept_idx entries must lie in
 * [0, D) (values outside are clamped into range, never read out of bounds).
 *   k_thin    out, [B,S_cap,Hkv,keep] dtype
 */
THINK_API int think_compact_k(const think_dims *d, const void *k_cache, const int32_t *seq_lens,
                    const int32_t *kept_idx, int32_t keep, void *k_thin, void *stream);

/*
 * Stages (a) + (b) + (c) in one call ("ThinK", Technical framework: score,
 * prune, store the pruned key cache).  Same arguments and outputs as
 * think_score_select followed by think_compact_k; scores and near_tie may be
 * NULL.  When the key cache fits in the device's register files (by capacity:
 * up to 256 KiB per compute unit, 64 MiB on a 256-CU part; the exact rule is
 * think_score_compact_single_read), one launch of one workgroup per compute
 * unit reads K once, holds it on chip while the channels are selected and
 * writes k_thin from there; otherwise the two-pass kernels run.  The
 * workgroups of that launch wait for one another, so it needs every compute
 * unit to become free in time: it must not run concurrently with another
 * single-read launch or share the device with a kernel that never finishes.
 * Its waits are bounded (about 4 s), so a violation ends rather than hangs;
 * the launch then records that it gave up, and think_score_compact_status
 * reports it (THINK_ERR_WAIT: kept_idx, near_tie, scores and k_thin of that
 * call are invalid).
 * Both paths give the same kept channels up to the near-tie flag (scores may
 * differ in the last fp32 place: the token sums are split differently) and,
 * for the same kept channels, the same k_thin bytes.
 *   workspace   >= think_score_compact_workspace_bytes(d, keep) bytes, 16-byte
 *               aligned, any previous contents.  The single-read launch keeps
 *               its flags there, tagged with a generation word that every
 *               launch advances, so the call may be captured in a graph and
 *               replayed; calls that share a workspace must not overlap in
 *               time.
 */
THINK_API int think_score_select_compact(const think_dims *d, const void *k_cache,
                                         const int32_t *seq_lens, const void *q_obs,
                                         int32_t obs_window, int32_t keep, float *scores,
                                         int32_t *kept_idx, int32_t *near_tie, void *k_thin,
                                         void *workspace, size_t workspace_bytes, void *stream);
THINK_API size_t think_score_compact_workspace_bytes(const think_dims *d, int32_t keep);
/* Outcome of the latest think_score_select_compact on `workspace` (same d,
 * obs_window, keep and workspace as that call).  Waits for `stream`, then returns THINK_OK
 * if its outputs are valid, or THINK_ERR_WAIT if its single-read launch gave
 * up waiting (the one-launch-at-a-time rule above was broken); argument
 * errors as for the call, THINK_ERR_HIP if the stream or the copy failed.  A
 * shape that runs the two-pass kernels never waits: THINK_OK without touching
 * the device.  Only meaningful after such a call on this workspace. */
THINK_API int think_score_compact_status(const think_dims *d, int32_t obs_window, int32_t keep,
                                         const void *workspace, size_t workspace_bytes,
                                         void *stream);
/* Test hook, not for production use: while `on` is nonzero, single-read
 * launches enqueued from the calling thread wait for a tag that is never
 * written and give up after a few polls, so that the give-up report can be
 * tested without stalling the device.  Their outputs are invalid.  Returns the
 * previous setting. */
THINK_API int think_single_read_test_give_up(int on);
/* 1 if think_score_select_compact takes the single-read launch for this shape
 * on the current device, 0 if it runs the two-pass kernels, negative status
 * for invalid dims or keep. */
THINK_API int think_score_compact_single_read(const think_dims *d, int32_t keep);

/*
 * Stage (d) - one decode step of attention on the pruned keys ("ThinK",
 * Technical framework, last step; token generation is bound by memory
 * bandwidth: "Keyformer: KV Cache Reduction through Key Tokens Selection for
 * Efficient Generative Inference", original abstract).  Per (b, q head h),
 * kv = h / G:
 *   qS[j] = q[b,h,kept_idx[b,kv,j]]
 *   l_t   = softmax_scale * sum_j qS[j] * k_thin[b,t,kv,j]      (t < len_b)
 *   out[b,h,:] = sum_t softmax(l)_t * v_cache[b,t,kv,:]
 * Values are not pruned.  The caller passes softmax_scale (1/sqrt(D) with the
 * unpruned D reproduces unpruned attention at keep == D).
 *   q         [B,Hq,D] dtype           out  [B,Hq,D] dtype (written)
 *   workspace >= think_decode_workspace_bytes(d, keep), 16-byte aligned,
 *             caller-owned scratch (per-chunk partial softmax records); calls
 *             sharing one workspace must be ordered (same stream).
 * Precision: fp32 accumulation (bf16 matrix-core products for bf16 inputs);
 * per row ||out - exact||_inf / ||exact||_inf <= 1e-5 (fp32), 2e-2 (bf16).
 */
THINK_API int think_decode_attn(const think_dims *d, const void *q, const void *k_thin,
                      const void *v_cache, const int32_t *seq_lens, const int32_t *kept_idx,
                      int32_t keep, float softmax_scale, void *out, void *workspace,
                      size_t workspace_bytes, void *stream);

/*
 * think_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and result (bitwise), with no workspace argument.  The
 * partial records live in a scratch array of 8 MiB that the library holds on
 * every GPU it runs on, from that GPU's first such call until the process
 * ends; the call itself allocates nothing.  All calls on one GPU share that
 * array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.  Returns THINK_ERR_WORKSPACE
 * when think_decode_workspace_bytes(d, keep) exceeds 8 MiB (then use
 * think_decode_attn); other errors as for think_decode_attn.
 */
THINK_API int think_decode_attn_static(const think_dims *d, const void *q, const void *k_thin,
                                       const void *v_cache, const int32_t *seq_lens,
                                       const int32_t *kept_idx, int32_t keep,
                                       float softmax_scale, void *out, void *stream);

/*
 * Split-phase form of think_decode_attn, same arguments and workspace.
 * think_decode_attn_partial runs the chunk pass: every (b, kv head, token
 * chunk) writes one partial softmax record per query head (running max,
 * sum and unnormalised output) into the workspace.  think_decode_attn_combine
 * merges the records of each (b, h) in ascending chunk order and writes out.
 * Calling the two on one stream is exactly think_decode_attn (bitwise); a
 * caller may instead run the merge on a second stream after an event so it
 * overlaps other work.  The merge reads only dims, seq_lens, keep and the
 * workspace the chunk pass of the same shape filled.
 */
THINK_API int think_decode_attn_partial(const think_dims *d, const void *q, const void *k_thin,
                                        const void *v_cache, const int32_t *seq_lens,
                                        const int32_t *kept_idx, int32_t keep, float softmax_scale,
                                        void *workspace, size_t workspace_bytes, void *stream);
THINK_API int think_decode_attn_combine(const think_dims *d, const int32_t *seq_lens, int32_t keep,
                                        void *out, const void *workspace, size_t workspace_bytes,
                                        void *stream);

/*
 * Decode-time append, the step after stage (d): inference continues on the
 * pruned cache ("ThinK", Technical framework, last step), so a generated
 * token's key is stored pruned with the kept set already chosen for its
 * (b, kv), and its value in full.  For every b with len_b < S_cap:
 *   k_thin[b,len_b,kv,j]  = k_new[b,kv,kept_idx[b,kv,j]]
 *   v_cache[b,len_b,kv,:] = v_new[b,kv,:]
 *   seq_lens[b]           = len_b + 1        (device memory, updated in place)
 * A sequence already at S_cap is left as it is (no row written, length
 * kept); the caller owns capacity.  A think_decode_attn that follows on the
 * same stream attends over len_b + 1 tokens, the new one included.
 *   k_new, v_new  [B,Hkv,D] dtype
 *   seq_lens      int32 [B], read and written
 *   k_thin        [B,S_cap,Hkv,keep] dtype, row len_b written
 *   v_cache       [B,S_cap,Hkv,D] dtype, row len_b written
 * kept_idx entries outside [0, D) are clamped into range.  A byte copy.
 */
THINK_API int think_append_kv(const think_dims *d, const void *k_new, const void *v_new,
                              int32_t *seq_lens, const int32_t *kept_idx, int32_t keep,
                              void *k_thin, void *v_cache, void *stream);

/*
 * think_append_kv followed by think_decode_attn, in two launches instead of
 * three (the append is folded into the decode's merge).  The decode attends
 * over the cached tokens and, below capacity, the new token (key k_new pruned
 * to the kept channels, value v_new) as well; the new token's rows are then
 * written and seq_lens advanced exactly as think_append_kv does.  A sequence
 * at capacity gets no append and attends over its cached tokens only.
 * Arguments as for the two calls; workspace >= think_decode_workspace_bytes
 * (d, keep).  The output is within the decode's precision bound of the two
 * calls' (the new token's logit is summed in a different order); the cache
 * rows and lengths are bitwise those of think_append_kv.
 */
THINK_API int think_append_decode_attn(const think_dims *d, const void *q, const void *k_new,
                                       const void *v_new, void *k_thin, void *v_cache,
                                       int32_t *seq_lens, const int32_t *kept_idx, int32_t keep,
                                       float softmax_scale, void *out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * Prefill-fused scoring, the step before stage (a).  Stage (a) reads the keys
 * only through K2[b,kv,c] = sum_{t<len_b} K[b,t,kv,c]^2, and the prompt's keys
 * pass through the cache write anyway, so the sums can be gathered there and
 * the score computed later without reading the key cache.
 *
 * think_prefill_write_kv writes one chunk of a prompt: for t < n_rows with
 * t0 + t < min(len_b, S_cap) (seq_lens = the prompts' lengths),
 *   k_cache[b,t0+t,:,:] = k_rows[b,t,:,:],  v_cache[b,t0+t,:,:] = v_rows[b,t,:,:]
 * and adds the squares of those key rows to k2_state.  Other rows are neither
 * written nor counted.
 *   k_rows, v_rows    [B,n_rows,Hkv,D] dtype, n_rows >= 0, t0 >= 0
 *   k2_state          >= think_k2_state_bytes(d), 16-byte aligned, caller-owned,
 *                     zero-filled before a prompt's first chunk; every call adds
 *                     its chunk (fixed-order fp64 sums, no atomics).  Calls that
 *                     share a state must be ordered (same stream).
 * think_score_select_k2 computes the scores of think_score from the state (no
 * key read) and, when kept_idx is not NULL, the selection of think_select:
 *   scores    out, fp32 [B,Hkv,D] or NULL (then kept_idx is required)
 *   kept_idx  out, int32 [B,Hkv,keep] or NULL;  near_tie as for think_select
 * After a prompt is written completely, the scores equal think_score on the
 * written cache up to rounding (each within 1e-6 relative of exact).
 */
THINK_API size_t think_k2_state_bytes(const think_dims *d);
THINK_API int think_prefill_write_kv(const think_dims *d, const void *k_rows, const void *v_rows,
                                     int32_t t0, int32_t n_rows, const int32_t *seq_lens,
                                     void *k_cache, void *v_cache, void *k2_state,
                                     size_t k2_state_bytes, void *stream);
THINK_API int think_score_select_k2(const think_dims *d, const void *k2_state,
                                    size_t k2_state_bytes, const void *q_obs, int32_t obs_window,
                                    int32_t keep, float *scores, int32_t *kept_idx,
                                    int32_t *near_tie, void *stream);

/*
 * Calibration helper, not part of the method: one launch that reads
 * read_bytes from src and writes write_bytes to dst (any values) as fast as
 * the device allows, so that a benchmark can state the single-launch ceiling
 * for a path's byte counts.  Device pointers, 16-byte aligned; a pointer may
 * be NULL only when its byte count is 0.  THINK_ERR_UNSUPPORTED for counts of
 * 1 TiB or more.
 */
THINK_API int think_probe_stream(const void *src, size_t read_bytes, void *dst,
                                 size_t write_bytes, void *stream);

/* Static description of a status code. */
THINK_API const char *think_status_string(int status);
/* The hipError_t of the last THINK_ERR_HIP on this thread (0 if none). */
THINK_API int think_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* THINK_H */
