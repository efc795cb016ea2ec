"""Plain fp64 CPU oracle for query-driven key-cache channel pruning (ThinK).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this package.  The product library
(`query_driven_kv_amd`) never imports it and shares no code with it; the
oracle takes plain NumPy arrays and calls the C loops in `oracle.c`.

Method source: "ThinK: Thinner Key Cache by Query-Driven Pruning",
Method details -> Technical framework (score channels against the queries,
order them, prune the weakest, infer on the pruned key cache) and Key design
(1)-(2) / original abstract (relevance through attention weights; keep the
attention-weight loss small).  The score reading is documented in oracle.c.

Arrays: bf16 tensors are passed as uint16 bit patterns, fp32 as float32.
Every function returns fp64 results (scores, attention outputs) or int32
indices; none of them touches a GPU.

Parity unpinned: the grouped-query aggregation (sum of per-query-head norms
versus the stacked Frobenius norm), the 1/sqrt(D) softmax scale at keep < D
and the synthetic-data distributions are readings of silent passages; no
page value or mathematical identity fixes them (see the header of oracle.c).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_SO)
    i32, dbl, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_score.argtypes = [i32] * 6 + [vp, vp, vp, i32, vp]
    lib.oracle_score_rss.argtypes = [i32] * 6 + [vp, vp, vp, i32, vp]
    lib.oracle_score_materialised.argtypes = [i32] * 6 + [vp, vp, vp, i32, vp]
    lib.oracle_select.argtypes = [i32, i32, i32, vp, i32, vp, vp]
    lib.oracle_compact.argtypes = [i32] * 5 + [vp, vp, vp, i32, vp]
    lib.oracle_decode.argtypes = [i32] * 6 + [vp, vp, vp, vp, vp, i32, dbl, vp]
    lib.oracle_append.argtypes = [i32] * 5 + [vp, vp, vp, vp, i32, vp, vp]
    lib.oracle_prefill_write.argtypes = [i32] * 5 + [vp, vp, i32, i32, vp, vp, vp, vp]
    lib.oracle_score_from_k2.argtypes = [i32] * 5 + [vp, vp, i32, vp]
    lib.oracle_full_attn.argtypes = [i32] * 6 + [vp, vp, vp, vp, dbl, vp]
    lib.oracle_residual_materialised.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_residual_materialised.restype = dbl
    lib.oracle_residual_gram.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_residual_gram.restype = dbl
    lib.oracle_bruteforce.argtypes = [i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_bruteforce.restype = ctypes.c_long
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dt=None):
    return np.ascontiguousarray(np.asarray(a) if dt is None else np.asarray(a, dtype=dt))


def _check(rc, what):
    if rc == -2:
        raise ValueError(f"{what}: non-finite input")
    if rc != 0:
        raise ValueError(f"{what}: bad argument (rc={rc})")


def num_threads():
    return _load().oracle_num_threads()


def set_threads(n):
    _load().oracle_set_threads(int(n))


def _score_common(fn, k_cache, seq_lens, q_obs):
    k_cache, q_obs = _c(k_cache), _c(q_obs)
    lens = _c(seq_lens, np.int32)
    B, S, Hkv, D = k_cache.shape
    Bq, W, Hq, Dq = q_obs.shape
    if (Bq, Dq) != (B, D) or k_cache.dtype != q_obs.dtype or lens.shape != (B,):
        raise ValueError("shape/dtype mismatch")
    out = np.empty((B, Hkv, D), np.float64)
    rc = fn(B, S, Hq, Hkv, D, _dtype_code(k_cache), _ptr(k_cache), _ptr(lens),
            _ptr(q_obs), W, _ptr(out))
    _check(rc, fn.__name__)
    return out


def score(k_cache, seq_lens, q_obs):
    """Stage (a): s[b,kv,c] = ||K[b,:len_b,kv,c]|| * sum_g ||Q_w[b,:,kv*G+g,c]||.

    k_cache [B,S_cap,Hkv,D], q_obs [B,W,Hq,D] (float32 or bf16 bits),
    seq_lens [B].  Returns fp64 [B,Hkv,D]."""
    return _score_common(_load().oracle_score, k_cache, seq_lens, q_obs)


def score_rss(k_cache, seq_lens, q_obs):
    """The alternative grouped-query reading (stacked Frobenius norm); report only."""
    return _score_common(_load().oracle_score_rss, k_cache, seq_lens, q_obs)


def score_materialised(k_cache, seq_lens, q_obs):
    """Stage (a) by definition: ||Q_w[:,c] K[:,c]^T||_F formed explicitly (small inputs)."""
    return _score_common(_load().oracle_score_materialised, k_cache, seq_lens, q_obs)


def select(scores, keep):
    """Stage (b): top-`keep` channels per (b, kv) by (score desc, channel asc),
    written ascending, plus the near-tie flag.  scores: [B,Hkv,D] (any float;
    widened to fp64).  Returns (kept_idx int32 [B,Hkv,keep], near_tie int32 [B,Hkv])."""
    s = _c(scores, np.float64)
    B, Hkv, D = s.shape
    idx = np.empty((B, Hkv, keep), np.int32)
    tie = np.empty((B, Hkv), np.int32)
    _check(_load().oracle_select(B, Hkv, D, _ptr(s), int(keep), _ptr(idx), _ptr(tie)), "select")
    return idx, tie


def compact(k_cache, seq_lens, kept_idx, fill=None):
    """Stage (c): K_thin[b,t,kv,j] = K[b,t,kv,kept_idx[b,kv,j]] for t < len_b.

    Rows t >= len_b keep `fill` (zeros by default)."""
    k_cache = _c(k_cache)
    lens = _c(seq_lens, np.int32)
    idx = _c(kept_idx, np.int32)
    B, S, Hkv, D = k_cache.shape
    keep = idx.shape[-1]
    out = np.zeros((B, S, Hkv, keep), k_cache.dtype)
    if fill is not None:
        out[...] = fill
    _check(_load().oracle_compact(B, S, Hkv, D, _dtype_code(k_cache), _ptr(k_cache), _ptr(lens),
                                  _ptr(idx), keep, _ptr(out)), "compact")
    return out


def prefill_write(k_rows, v_rows, t0, seq_lens, k_cache, v_cache, k2):
    """Prefill-fused scoring, write half: rows t of the chunk go to positions
    t0+t < len_b of the caches and their squares are added to K2 (fp64
    [B,Hkv,D]).  Returns new copies (k_cache, v_cache, k2)."""
    k_rows, v_rows = _c(k_rows), _c(v_rows)
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    acc = np.array(k2, dtype=np.float64, copy=True)
    lens = _c(seq_lens, np.int32)
    B, S, Hkv, D = kc.shape
    n = k_rows.shape[1]
    if (k_rows.shape != (B, n, Hkv, D) or v_rows.shape != (B, n, Hkv, D) or acc.shape != (B, Hkv, D)
            or len({k_rows.dtype, v_rows.dtype, kc.dtype, vc.dtype}) != 1):
        raise ValueError("shape or dtype mismatch")
    _check(_load().oracle_prefill_write(B, S, Hkv, D, _dtype_code(kc), _ptr(k_rows), _ptr(v_rows),
                                        int(t0), n, _ptr(lens), _ptr(kc), _ptr(vc), _ptr(acc)),
           "prefill_write")
    return kc, vc, acc


def score_from_k2(k2, q_obs):
    """Stage (a) from gathered sums: sqrt(K2) * sum_g sqrt(sum_i Q_w^2); fp64 [B,Hkv,D]."""
    k2, q_obs = _c(k2, np.float64), _c(q_obs)
    B, Hkv, D = k2.shape
    Bq, W, Hq, Dq = q_obs.shape
    if (Bq, Dq) != (B, D) or Hq % Hkv:
        raise ValueError("shape mismatch")
    out = np.empty((B, Hkv, D), np.float64)
    _check(_load().oracle_score_from_k2(B, Hq, Hkv, D, _dtype_code(q_obs), _ptr(k2), _ptr(q_obs),
                                        W, _ptr(out)), "score_from_k2")
    return out


def append(k_new, v_new, seq_lens, kept_idx, k_thin, v_cache):
    """Decode-time append: for every b with len_b < S_cap, write the pruned new
    key K_thin[b,len_b,kv,j] = k_new[b,kv,kept_idx[b,kv,j]] and the new value
    V[b,len_b,kv,:] = v_new[b,kv,:], then len_b += 1.  Returns new copies
    (k_thin, v_cache, seq_lens); the inputs are not modified."""
    k_new, v_new = _c(k_new), _c(v_new)
    idx = _c(kept_idx, np.int32)
    kt, vc = np.array(k_thin, copy=True), np.array(v_cache, copy=True)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    B, S, Hkv, D = vc.shape
    keep = idx.shape[-1]
    if (k_new.shape != (B, Hkv, D) or v_new.shape != (B, Hkv, D) or kt.shape != (B, S, Hkv, keep)
            or k_new.dtype != vc.dtype or kt.dtype != vc.dtype or v_new.dtype != vc.dtype):
        raise ValueError("shape or dtype mismatch")
    _check(_load().oracle_append(B, S, Hkv, D, _dtype_code(vc), _ptr(k_new), _ptr(v_new),
                                 _ptr(lens), _ptr(idx), keep, _ptr(kt), _ptr(vc)), "append")
    return kt, vc, lens


def decode(q, k_thin, v_cache, seq_lens, kept_idx, scale):
    """Stage (d): softmax(scale * q[idx] . K_thin^T) V per q head; fp64 [B,Hq,D]."""
    q, k_thin, v_cache = _c(q), _c(k_thin), _c(v_cache)
    lens = _c(seq_lens, np.int32)
    idx = _c(kept_idx, np.int32)
    B, Hq, D = q.shape
    _, S, Hkv, keep = k_thin.shape
    if v_cache.shape != (B, S, Hkv, D) or idx.shape != (B, Hkv, keep):
        raise ValueError("shape mismatch")
    out = np.empty((B, Hq, D), np.float64)
    _check(_load().oracle_decode(B, S, Hq, Hkv, D, _dtype_code(q), _ptr(q), _ptr(k_thin),
                                 _ptr(v_cache), _ptr(lens), _ptr(idx), keep, float(scale),
                                 _ptr(out)), "decode")
    return out


def full_attn(q, k_cache, v_cache, seq_lens, scale):
    """Unpruned decode attention over the original keys; fp64 [B,Hq,D]."""
    q, k_cache, v_cache = _c(q), _c(k_cache), _c(v_cache)
    lens = _c(seq_lens, np.int32)
    B, Hq, D = q.shape
    _, S, Hkv, _ = k_cache.shape
    out = np.empty((B, Hq, D), np.float64)
    _check(_load().oracle_full_attn(B, S, Hq, Hkv, D, _dtype_code(q), _ptr(q), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(lens), float(scale), _ptr(out)),
           "full_attn")
    return out


def _mask(in_set, D):
    m = np.zeros(D, np.int32)
    m[np.asarray(list(in_set), dtype=np.int64)] = 1
    return m


def residual_materialised(Qw, K, in_set):
    """||Qw K^T - Qw[:,S] K[:,S]^T||_F by forming the error matrix. Qw [W,D], K [L,D]."""
    Qw, K = _c(Qw, np.float64), _c(K, np.float64)
    W, D = Qw.shape
    L = K.shape[0]
    return _load().oracle_residual_materialised(W, L, D, _ptr(Qw), _ptr(K), _ptr(_mask(in_set, D)))


def residual_gram(Qw, K, in_set):
    """The same residual through the Gram matrices of Qw and K."""
    Qw, K = _c(Qw, np.float64), _c(K, np.float64)
    W, D = Qw.shape
    L = K.shape[0]
    return _load().oracle_residual_gram(W, L, D, _ptr(Qw), _ptr(K), _ptr(_mask(in_set, D)))


def bruteforce(Qw, K, keep, candidate=None):
    """Exhaustive optimum of the residual over all keep-subsets (D <= 20).

    Returns dict(r_opt, opt_set, visited, r_candidate, candidate_rank)."""
    Qw, K = _c(Qw, np.float64), _c(K, np.float64)
    W, D = Qw.shape
    L = K.shape[0]
    cand = _mask(candidate, D) if candidate is not None else None
    r_opt = ctypes.c_double()
    r_c = ctypes.c_double()
    rank = ctypes.c_long()
    opt = np.zeros(D, np.int32)
    n = _load().oracle_bruteforce(W, L, D, _ptr(Qw), _ptr(K), int(keep), _ptr(cand),
                                  ctypes.byref(r_opt), _ptr(opt), ctypes.byref(r_c),
                                  ctypes.byref(rank))
    if n < 0:
        raise ValueError("bruteforce: bad argument")
    return dict(r_opt=r_opt.value, opt_set=sorted(np.nonzero(opt)[0].tolist()), visited=int(n),
                r_candidate=r_c.value if candidate is not None else None,
                candidate_rank=int(rank.value) if candidate is not None else None)
