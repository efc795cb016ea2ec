"""MI355X (gfx950) hot path of query-driven key-cache channel pruning (ThinK).

Thin Python layer over the C ABI of include/think.h.  Tensors are torch
device tensors (torch is used for device memory and streams only); each
function checks shapes, dtypes, devices and contiguity, builds the
think_dims descriptor, allocates the workspace when none is passed, and
calls the HIP library on the current torch stream.

Stages ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
Technical framework): think_score -> think_select -> think_compact_k ->
think_decode_attn.
"""
import ctypes

import torch

from . import _lib
from ._lib import THINK_BF16, THINK_F32, ThinkError, think_dims

__all__ = ["think_score", "think_score_select", "think_select", "think_compact_k",
           "think_decode_attn",
           "think_decode_attn_partial", "think_decode_attn_combine", "think_append_kv",
           "think_append_decode_attn", "think_k2_state_bytes", "think_prefill_write_kv", "think_score_select_k2",
           "think_score_select_compact", "think_score_compact_workspace_bytes",
           "think_score_compact_single_read", "think_score_compact_status",
           "think_single_read_test_give_up",
           "think_keep_from_ratio", "think_score_workspace_bytes", "think_decode_workspace_bytes",
           "think_abi_version", "make_dims", "ThinkError", "think_dims", "LIB_PATH"]

LIB_PATH = _lib.LIB_PATH
_DT = {torch.float32: THINK_F32, torch.bfloat16: THINK_BF16}


def _dtype_code(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16") from None


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _new(stream, *shape, dtype, device):
    """A tensor this layer allocates for a call (output or workspace).  The
    kernels run on `stream`; when that is not the current stream, the caching
    allocator is told, so that the block is not handed to another allocation
    while the call may still use it."""
    t = torch.empty(*shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(t.device):
        t.record_stream(stream)
    return t


def _workspace(stream, nbytes, device):
    return _new(stream, max(int(nbytes), 16), dtype=torch.uint8, device=device)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def make_dims(batch, n_q_heads, n_kv_heads, head_dim, seq_capacity, dtype):
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return think_dims(batch, n_q_heads, n_kv_heads, head_dim, seq_capacity, code)


def think_abi_version():
    return _lib.lib.think_abi_version()


def think_keep_from_ratio(head_dim, prune_ratio):
    return _lib.lib.think_keep_from_ratio(int(head_dim), float(prune_ratio))


def think_score_workspace_bytes(dims):
    return _lib.lib.think_score_workspace_bytes(ctypes.byref(dims))


def think_decode_workspace_bytes(dims, keep):
    return _lib.lib.think_decode_workspace_bytes(ctypes.byref(dims), int(keep))


def think_score_compact_workspace_bytes(dims, keep):
    return _lib.lib.think_score_compact_workspace_bytes(ctypes.byref(dims), int(keep))


def think_score_compact_single_read(dims, keep):
    """1: think_score_select_compact reads K once for this shape on the current
    device; 0: it runs the two-pass kernels."""
    r = _lib.lib.think_score_compact_single_read(ctypes.byref(dims), int(keep))
    if r < 0:
        _lib.check("think_score_compact_single_read", r)
    return r


def think_score_compact_status(dims, obs_window, keep, workspace, *, stream=None):
    """Outcome of the latest think_score_select_compact on `workspace` (waits
    for the stream): 0 (THINK_OK) if its outputs are valid, -8 (THINK_ERR_WAIT)
    if its single-read launch gave up waiting.  Other errors raise."""
    _dev(workspace)
    r = _lib.lib.think_score_compact_status(
        ctypes.byref(dims), int(obs_window), int(keep), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if r not in (0, -8):
        _lib.check("think_score_compact_status", r)
    return r


def think_single_read_test_give_up(on):
    """Test hook: while on, this thread's single-read launches give up every
    wait (their outputs are invalid).  Returns the previous setting."""
    return bool(_lib.lib.think_single_read_test_give_up(1 if on else 0))


def _i32(t, name):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")


def think_score(k_cache, seq_lens, q_obs, *, scores=None, workspace=None, stream=None):
    """Stage (a).  k_cache [B,S_cap,Hkv,D], seq_lens int32 [B] (device),
    q_obs [B,W,Hq,D] -> scores fp32 [B,Hkv,D]."""
    _dev(k_cache, seq_lens, q_obs, scores, workspace)
    _i32(seq_lens, "seq_lens")
    B, S, Hkv, D = k_cache.shape
    Bq, W, Hq, Dq = q_obs.shape
    if (Bq, Dq) != (B, D) or q_obs.dtype != k_cache.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape or dtype mismatch between k_cache, q_obs and seq_lens")
    dims = make_dims(B, Hq, Hkv, D, S, _dtype_code(k_cache))
    if scores is None:
        scores = _new(stream, B, Hkv, D, dtype=torch.float32, device=k_cache.device)
    elif scores.dtype != torch.float32 or tuple(scores.shape) != (B, Hkv, D):
        raise ValueError("scores must be float32 [B,Hkv,D]")
    need = think_score_workspace_bytes(dims)
    if workspace is None:
        workspace = _workspace(stream, need, k_cache.device)
    _lib.check("think_score", _lib.lib.think_score(
        ctypes.byref(dims), _p(k_cache), _p(seq_lens), _p(q_obs), W, _p(scores), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return scores


def think_score_select(k_cache, seq_lens, q_obs, keep, *, scores=None, kept_idx=None,
                       near_tie=None, workspace=None, stream=None):
    """Stages (a)+(b) fused.  Returns (scores fp32 [B,Hkv,D], kept_idx int32
    [B,Hkv,keep], near_tie int32 [B,Hkv]); bitwise think_score then think_select."""
    _dev(k_cache, seq_lens, q_obs, scores, kept_idx, near_tie, workspace)
    _i32(seq_lens, "seq_lens")
    B, S, Hkv, D = k_cache.shape
    Bq, W, Hq, Dq = q_obs.shape
    if (Bq, Dq) != (B, D) or q_obs.dtype != k_cache.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape or dtype mismatch between k_cache, q_obs and seq_lens")
    dims = make_dims(B, Hq, Hkv, D, S, _dtype_code(k_cache))
    dev = k_cache.device
    if scores is None:
        scores = _new(stream, B, Hkv, D, dtype=torch.float32, device=dev)
    if kept_idx is None:
        kept_idx = _new(stream, B, Hkv, max(int(keep), 0), dtype=torch.int32, device=dev)
    if near_tie is None:
        near_tie = _new(stream, B, Hkv, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _workspace(stream, think_score_workspace_bytes(dims), dev)
    _lib.check("think_score_select", _lib.lib.think_score_select(
        ctypes.byref(dims), _p(k_cache), _p(seq_lens), _p(q_obs), W, int(keep), _p(scores),
        _p(kept_idx), _p(near_tie), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return scores, kept_idx, near_tie


def think_select(scores, keep, *, kept_idx=None, near_tie=None, want_near_tie=True, stream=None):
    """Stage (b).  scores fp32 [B,Hkv,D] -> (kept_idx int32 [B,Hkv,keep], near_tie int32 [B,Hkv])."""
    _dev(scores, kept_idx, near_tie)
    if scores.dtype != torch.float32 or scores.dim() != 3:
        raise ValueError("scores must be float32 [B,Hkv,D]")
    B, Hkv, D = scores.shape
    dims = make_dims(B, Hkv, Hkv, D, 1, THINK_F32)
    if kept_idx is None:
        kept_idx = _new(stream, B, Hkv, max(int(keep), 0), dtype=torch.int32,
                        device=scores.device)
    if want_near_tie and near_tie is None:
        near_tie = _new(stream, B, Hkv, dtype=torch.int32, device=scores.device)
    _lib.check("think_select", _lib.lib.think_select(
        ctypes.byref(dims), _p(scores), int(keep), _p(kept_idx), _p(near_tie), _stream(stream)))
    return kept_idx, near_tie


def think_compact_k(k_cache, seq_lens, kept_idx, *, k_thin=None, stream=None):
    """Stage (c).  k_cache [B,S_cap,Hkv,D], kept_idx int32 [B,Hkv,keep] ->
    k_thin [B,S_cap,Hkv,keep] (rows t >= len_b untouched)."""
    _dev(k_cache, seq_lens, kept_idx, k_thin)
    _i32(seq_lens, "seq_lens")
    _i32(kept_idx, "kept_idx")
    B, S, Hkv, D = k_cache.shape
    keep = kept_idx.shape[-1]
    if tuple(kept_idx.shape) != (B, Hkv, keep):
        raise ValueError("kept_idx must be [B,Hkv,keep]")
    dims = make_dims(B, Hkv, Hkv, D, S, _dtype_code(k_cache))
    if k_thin is None:
        k_thin = _new(stream, B, S, Hkv, keep, dtype=k_cache.dtype, device=k_cache.device)
    elif tuple(k_thin.shape) != (B, S, Hkv, keep) or k_thin.dtype != k_cache.dtype:
        raise ValueError("k_thin must be [B,S_cap,Hkv,keep] of the cache dtype")
    _lib.check("think_compact_k", _lib.lib.think_compact_k(
        ctypes.byref(dims), _p(k_cache), _p(seq_lens), _p(kept_idx), keep, _p(k_thin),
        _stream(stream)))
    return k_thin


def think_score_select_compact(k_cache, seq_lens, q_obs, keep, *, scores=None, kept_idx=None,
                               near_tie=None, k_thin=None, workspace=None, stream=None,
                               check_status=False):
    """Stages (a)+(b)+(c) in one call (one read of K when it fits on chip).
    Returns (scores fp32 [B,Hkv,D], kept_idx int32 [B,Hkv,keep], near_tie
    int32 [B,Hkv], k_thin [B,S_cap,Hkv,keep]).  check_status=True waits for
    the call and raises ThinkError (THINK_ERR_WAIT) if its single-read launch
    gave up waiting."""
    _dev(k_cache, seq_lens, q_obs, scores, kept_idx, near_tie, k_thin, workspace)
    _i32(seq_lens, "seq_lens")
    B, S, Hkv, D = k_cache.shape
    Bq, W, Hq, Dq = q_obs.shape
    if (Bq, Dq) != (B, D) or q_obs.dtype != k_cache.dtype or tuple(seq_lens.shape) != (B,):
        raise ValueError("shape or dtype mismatch between k_cache, q_obs and seq_lens")
    dims = make_dims(B, Hq, Hkv, D, S, _dtype_code(k_cache))
    dev = k_cache.device
    keep = int(keep)
    if scores is None:
        scores = _new(stream, B, Hkv, D, dtype=torch.float32, device=dev)
    if kept_idx is None:
        kept_idx = _new(stream, B, Hkv, max(keep, 0), dtype=torch.int32, device=dev)
    if near_tie is None:
        near_tie = _new(stream, B, Hkv, dtype=torch.int32, device=dev)
    if k_thin is None:
        k_thin = _new(stream, B, S, Hkv, max(keep, 0), dtype=k_cache.dtype, device=dev)
    elif tuple(k_thin.shape) != (B, S, Hkv, keep) or k_thin.dtype != k_cache.dtype:
        raise ValueError("k_thin must be [B,S_cap,Hkv,keep] of the cache dtype")
    if workspace is None:
        workspace = _workspace(stream, think_score_compact_workspace_bytes(dims, keep), dev)
    _lib.check("think_score_select_compact", _lib.lib.think_score_select_compact(
        ctypes.byref(dims), _p(k_cache), _p(seq_lens), _p(q_obs), W, keep, _p(scores),
        _p(kept_idx), _p(near_tie), _p(k_thin), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    if check_status:
        _lib.check("think_score_select_compact",
                   think_score_compact_status(dims, W, keep, workspace, stream=stream))
    return scores, kept_idx, near_tie, k_thin


def think_decode_attn(q, k_thin, v_cache, seq_lens, kept_idx, softmax_scale, *, out=None,
                      workspace=None, stream=None):
    """Stage (d).  q [B,Hq,D], k_thin [B,S_cap,Hkv,keep], v_cache [B,S_cap,Hkv,D],
    kept_idx int32 [B,Hkv,keep] -> out [B,Hq,D] (dtype of q)."""
    _dev(q, k_thin, v_cache, seq_lens, kept_idx, out, workspace)
    _i32(seq_lens, "seq_lens")
    _i32(kept_idx, "kept_idx")
    B, Hq, D = q.shape
    _, S, Hkv, keep = k_thin.shape
    if (tuple(v_cache.shape) != (B, S, Hkv, D) or tuple(kept_idx.shape) != (B, Hkv, keep)
            or k_thin.dtype != q.dtype or v_cache.dtype != q.dtype):
        raise ValueError("shape or dtype mismatch between q, k_thin, v_cache and kept_idx")
    dims = make_dims(B, Hq, Hkv, D, S, _dtype_code(q))
    if out is None:
        out = _new(stream, B, Hq, D, dtype=q.dtype, device=q.device)
    need = think_decode_workspace_bytes(dims, keep)
    if workspace is None:
        workspace = _workspace(stream, need, q.device)
    _lib.check("think_decode_attn", _lib.lib.think_decode_attn(
        ctypes.byref(dims), _p(q), _p(k_thin), _p(v_cache), _p(seq_lens), _p(kept_idx), int(keep),
        float(softmax_scale), _p(out), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def _decode_dims(q, k_thin, v_cache, seq_lens, kept_idx):
    _dev(q, k_thin, v_cache, seq_lens, kept_idx)
    _i32(seq_lens, "seq_lens")
    _i32(kept_idx, "kept_idx")
    B, Hq, D = q.shape
    _, S, Hkv, keep = k_thin.shape
    if (tuple(v_cache.shape) != (B, S, Hkv, D) or tuple(kept_idx.shape) != (B, Hkv, keep)
            or k_thin.dtype != q.dtype or v_cache.dtype != q.dtype):
        raise ValueError("shape or dtype mismatch between q, k_thin, v_cache and kept_idx")
    return make_dims(B, Hq, Hkv, D, S, _dtype_code(q)), keep


def think_decode_attn_partial(q, k_thin, v_cache, seq_lens, kept_idx, softmax_scale, workspace,
                              *, stream=None):
    """Chunk pass of stage (d): per-chunk partial softmax records into `workspace`
    (uint8, >= think_decode_workspace_bytes).  Returns (dims, keep) for the merge."""
    dims, keep = _decode_dims(q, k_thin, v_cache, seq_lens, kept_idx)
    _dev(workspace)
    _lib.check("think_decode_attn_partial", _lib.lib.think_decode_attn_partial(
        ctypes.byref(dims), _p(q), _p(k_thin), _p(v_cache), _p(seq_lens), _p(kept_idx), int(keep),
        float(softmax_scale), _p(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return dims, keep


def think_decode_attn_combine(dims, keep, seq_lens, workspace, out, *, stream=None):
    """Merge pass of stage (d): merges the records the chunk pass left in `workspace`."""
    _dev(seq_lens, workspace, out)
    _lib.check("think_decode_attn_combine", _lib.lib.think_decode_attn_combine(
        ctypes.byref(dims), _p(seq_lens), int(keep), _p(out), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def think_append_kv(k_new, v_new, seq_lens, kept_idx, k_thin, v_cache, *, stream=None):
    """Decode-time append.  k_new, v_new [B,Hkv,D]; writes the pruned key into
    k_thin[b, len_b] and the value into v_cache[b, len_b] and advances
    seq_lens[b] in place (a full sequence is left as it is).  Returns seq_lens."""
    _dev(k_new, v_new, seq_lens, kept_idx, k_thin, v_cache)
    _i32(seq_lens, "seq_lens")
    _i32(kept_idx, "kept_idx")
    B, S, Hkv, D = v_cache.shape
    keep = kept_idx.shape[-1]
    if (tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or tuple(k_thin.shape) != (B, S, Hkv, keep) or tuple(kept_idx.shape) != (B, Hkv, keep)
            or len({k_new.dtype, v_new.dtype, k_thin.dtype, v_cache.dtype}) != 1):
        raise ValueError("shape or dtype mismatch between k_new, v_new, k_thin, v_cache, kept_idx")
    dims = make_dims(B, Hkv, Hkv, D, S, _dtype_code(v_cache))
    _lib.check("think_append_kv", _lib.lib.think_append_kv(
        ctypes.byref(dims), _p(k_new), _p(v_new), _p(seq_lens), _p(kept_idx), int(keep),
        _p(k_thin), _p(v_cache), _stream(stream)))
    return seq_lens


def think_append_decode_attn(q, k_new, v_new, k_thin, v_cache, seq_lens, kept_idx,
                             softmax_scale, *, out=None, workspace=None, stream=None):
    """think_append_kv then think_decode_attn in two launches: the decode
    attends over the cached tokens plus the new one (below capacity), whose
    rows are then written and seq_lens advanced in place.  Returns out."""
    _dev(q, k_new, v_new, k_thin, v_cache, seq_lens, kept_idx, out, workspace)
    _i32(seq_lens, "seq_lens")
    _i32(kept_idx, "kept_idx")
    B, Hq, D = q.shape
    _, S, Hkv, keep = k_thin.shape
    if (tuple(v_cache.shape) != (B, S, Hkv, D) or tuple(kept_idx.shape) != (B, Hkv, keep)
            or tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D)
            or len({q.dtype, k_new.dtype, v_new.dtype, k_thin.dtype, v_cache.dtype}) != 1):
        raise ValueError("shape or dtype mismatch between q, k_new, v_new, k_thin, v_cache, "
                         "kept_idx")
    dims = make_dims(B, Hq, Hkv, D, S, _dtype_code(q))
    if out is None:
        out = _new(stream, B, Hq, D, dtype=q.dtype, device=q.device)
    need = think_decode_workspace_bytes(dims, keep)
    if workspace is None:
        workspace = _workspace(stream, need, q.device)
    _lib.check("think_append_decode_attn", _lib.lib.think_append_decode_attn(
        ctypes.byref(dims), _p(q), _p(k_new), _p(v_new), _p(k_thin), _p(v_cache), _p(seq_lens),
        _p(kept_idx), int(keep), float(softmax_scale), _p(out), _p(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def think_k2_state_bytes(dims):
    return int(_lib.lib.think_k2_state_bytes(ctypes.byref(dims)))


def think_prefill_write_kv(k_rows, v_rows, t0, seq_lens, k_cache, v_cache, k2_state, *,
                           stream=None):
    """Prefill-fused scoring, write half.  k_rows, v_rows [B,n,Hkv,D] go to
    positions t0.. of k_cache / v_cache [B,S_cap,Hkv,D] (rows at or past len_b
    skipped) and their key squares are added to k2_state (uint8 device buffer of
    think_k2_state_bytes, zeroed before a prompt's first chunk)."""
    _dev(k_rows, v_rows, seq_lens, k_cache, v_cache, k2_state)
    _i32(seq_lens, "seq_lens")
    B, S, Hkv, D = k_cache.shape
    n = k_rows.shape[1]
    if (tuple(k_rows.shape) != (B, n, Hkv, D) or tuple(v_rows.shape) != (B, n, Hkv, D)
            or tuple(v_cache.shape) != (B, S, Hkv, D)
            or len({k_rows.dtype, v_rows.dtype, k_cache.dtype, v_cache.dtype}) != 1):
        raise ValueError("shape or dtype mismatch between k_rows, v_rows, k_cache and v_cache")
    dims = make_dims(B, Hkv, Hkv, D, S, _dtype_code(k_cache))
    _lib.check("think_prefill_write_kv", _lib.lib.think_prefill_write_kv(
        ctypes.byref(dims), _p(k_rows), _p(v_rows), int(t0), int(n), _p(seq_lens), _p(k_cache),
        _p(v_cache), _p(k2_state), k2_state.numel() * k2_state.element_size(), _stream(stream)))


def think_score_select_k2(dims, k2_state, q_obs, keep=None, *, scores=None, kept_idx=None,
                          near_tie=None, stream=None):
    """Scores (fp32 [B,Hkv,D]) from the prefill-write state, no key read; with
    `keep`, also the kept channels and near-tie flags.  Returns (scores, kept_idx,
    near_tie), the last two None without `keep`."""
    _dev(k2_state, q_obs, scores, kept_idx, near_tie)
    B, Hkv, D = dims.batch, dims.n_kv_heads, dims.head_dim
    W = q_obs.shape[1]
    if tuple(q_obs.shape) != (B, W, dims.n_q_heads, D) or _dtype_code(q_obs) != dims.dtype:
        raise ValueError("q_obs must be [B,W,Hq,D] of the dims' dtype")
    dev = q_obs.device
    if scores is None:
        scores = _new(stream, B, Hkv, D, dtype=torch.float32, device=dev)
    if keep is not None:
        if kept_idx is None:
            kept_idx = _new(stream, B, Hkv, keep, dtype=torch.int32, device=dev)
        if near_tie is None:
            near_tie = _new(stream, B, Hkv, dtype=torch.int32, device=dev)
    _lib.check("think_score_select_k2", _lib.lib.think_score_select_k2(
        ctypes.byref(dims), _p(k2_state), k2_state.numel() * k2_state.element_size(), _p(q_obs),
        int(W), int(keep or 0), _p(scores), _p(kept_idx), _p(near_tie), _stream(stream)))
    return scores, kept_idx, near_tie
