"""The allocation-free decode (think_decode_attn_static), called through the C
ABI: its output equals think_decode_attn's (same kernels, bitwise) and lies
within the dtype's bound of the oracle, on calls in a row on the device's one
scratch array, each with a smaller input than the one before (bf16 on the
matrix-core kernel, then fp32 on the general one); a shape whose records
exceed the array is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import row_rel_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def _decode_pair(cfg, layer, step):
    import query_driven_kv_amd as qdk
    from query_driven_kv_amd import _lib
    L = kvsynth.make_layer(cfg, layer)
    k = to_dev(L["k_cache"])
    lens = to_dev(L["seq_lens"])
    s, idx, _ = qdk.think_score_select(k, lens, to_dev(L["q_obs"]), cfg.keep)
    thin = qdk.think_compact_k(k, lens, idx)
    v = to_dev(L["v_cache"])
    q = to_dev(kvsynth.decode_q(cfg, layer, step, L["channel_scale"]))
    scale = 1.0 / np.sqrt(cfg.head_dim)
    ref = qdk.think_decode_attn(q, thin, v, lens, idx, scale)
    B, Hq, D = q.shape
    dims = qdk.make_dims(B, Hq, cfg.n_kv_heads, D, cfg.seq_capacity,
                         qdk.THINK_BF16 if cfg.dtype == "bf16" else qdk.THINK_F32)
    out = torch.full_like(ref, float("nan"))
    P = ctypes.c_void_p
    rc = _lib.lib.think_decode_attn_static(
        ctypes.byref(dims), P(q.data_ptr()), P(thin.data_ptr()), P(v.data_ptr()),
        P(lens.data_ptr()), P(idx.data_ptr()), cfg.keep, ctypes.c_float(scale),
        P(out.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, _lib.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    o_ref = oracle.decode(kvsynth.decode_q(cfg, layer, step, L["channel_scale"]),
                          oracle.compact(L["k_cache"], L["seq_lens"], to_host(idx)),
                          L["v_cache"], L["seq_lens"], to_host(idx), np.float32(scale))
    return to_host(out), to_host(ref), o_ref


def test_static_scratch_decode_matches_the_workspace_call():
    big = kvsynth.CONFIGS["mistral-7b-gqa-32k"]
    small = kvsynth.custom("no-alloc-small", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           seq_capacity=700, obs_window=8, keep=51, dtype="bf16", lowrank=8,
                           ragged=(200, 700), cfg_id=77)
    general = kvsynth.custom("no-alloc-f32", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64,
                             seq_capacity=600, obs_window=8, keep=30, dtype="f32", lowrank=8,
                             ragged=(100, 600), cfg_id=78)
    for cfg, step in ((big, 0), (small, 1), (general, 2)):
        print(f"[no-alloc] {cfg.name}: B={cfg.batch} S={cfg.seq_capacity} keep={cfg.keep} "
              f"{cfg.dtype}", flush=True)
        got, ref, o_ref = _decode_pair(cfg, 0, step)
        np.testing.assert_array_equal(got.view(np.uint8), ref.view(np.uint8))
        err = row_rel_err(got, o_ref).max()
        bar = 2e-2 if cfg.dtype == "bf16" else 1e-5
        assert err <= bar, f"{cfg.name}: row error {err:.3e}"


def test_static_scratch_refuses_shapes_past_its_size():
    import query_driven_kv_amd as qdk
    from query_driven_kv_amd import _lib
    # fp32 records of a long many-head cache need more than the 8 MiB array
    dims = qdk.make_dims(1, 64, 64, 128, 1 << 20, qdk.THINK_F32)
    assert qdk.think_decode_workspace_bytes(dims, 64) > (8 << 20)
    t = torch.empty(16, device="cuda")
    P = ctypes.c_void_p(t.data_ptr())
    rc = _lib.lib.think_decode_attn_static(ctypes.byref(dims), P, P, P, P, P, 64,
                                           ctypes.c_float(0.1), P, None)
    assert rc == -6
