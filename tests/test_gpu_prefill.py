"""GPU parity of prefill-fused scoring against the oracle: a prompt is
written into the caches chunk by chunk with think_prefill_write_kv, then
think_score_select_k2 scores it from the gathered sums without reading the key
cache.  Checks: the caches equal the oracle's writes byte for byte (rows past
len_b keep their NaN sentinel); the scores are within 5e-6 relative of the
oracle's scores of the finished cache and of think_score on the same cache;
the selection equals the oracle's selection on the same fp32 scores bit for
bit; a second pass over the same chunks gives the same bits."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

SCORE_RTOL = 5e-6

CASES = [
    # seed, lens, Hq, Hkv, D, S_cap, chunk sizes, keep, dtype
    (60, [3000, 1234], 32, 8, 128, 3072, [512] * 6, 64, "bf16"),
    (61, [100, 1, 77], 6, 3, 64, 128, [13, 50, 1, 64], 20, "f32"),
    (62, [20000], 16, 2, 128, 20000, [4096] * 4 + [3616], 51, "bf16"),
    (63, [5, 700], 8, 8, 256, 700, [700], 100, "bf16"),          # one chunk, 4 KiB rows
]


def _run(qdk, dims, src_k, src_v, lens_d, chunks, nan, dtype_t):
    B, S, Hkv, D = src_k.shape
    kc = torch.full((B, S, Hkv, D), float("nan"), dtype=dtype_t, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    state = torch.zeros(qdk.think_k2_state_bytes(dims), dtype=torch.uint8, device="cuda")
    t0 = 0
    for n in chunks:
        qdk.think_prefill_write_kv(to_dev(np.ascontiguousarray(src_k[:, t0:t0 + n])),
                                   to_dev(np.ascontiguousarray(src_v[:, t0:t0 + n])), t0, lens_d,
                                   kc, vc, state)
        t0 += n
    return kc, vc, state


@pytest.mark.parametrize("case", CASES, ids=[f"prefill{c[0]}" for c in CASES])
def test_prefill_write_then_score_from_sums(case):
    import query_driven_kv_amd as qdk
    seed, lens, Hq, Hkv, D, S, chunks, keep, dtype = case
    B = len(lens)
    assert sum(chunks) == S
    print(f"[prefill] seed {seed}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} chunks={chunks} "
          f"keep={keep} {dtype}", flush=True)
    cfg = kvsynth.custom(f"prefill{seed}", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                         seq_capacity=S, obs_window=6, keep=keep, dtype=dtype, cfg_id=92,
                         lowrank=8 if D >= 64 else 0)
    L = kvsynth.make_layer(cfg, layer=seed)
    lens = np.asarray(lens, np.int32)
    nan = kvsynth.nan_value(dtype)
    src_k, src_v = L["k_cache"], L["v_cache"]
    for b in range(B):
        src_k[b, lens[b]:] = nan                 # a read past len_b would show up
        src_v[b, lens[b]:] = nan
    dtype_t = torch.bfloat16 if dtype == "bf16" else torch.float32
    dims = qdk.make_dims(B, Hq, Hkv, D, S, dtype_t)
    lens_d, qo = to_dev(lens), to_dev(L["q_obs"])

    kc, vc, state = _run(qdk, dims, src_k, src_v, lens_d, chunks, nan, dtype_t)
    s_k2, idx, tie = qdk.think_score_select_k2(dims, state, qo, keep)
    s_cache = qdk.think_score(kc, lens_d, qo)
    torch.cuda.synchronize()

    # the oracle writes the same chunks
    okc = np.full_like(src_k, nan)
    ovc = np.full_like(src_v, nan)
    ok2 = np.zeros((B, Hkv, D))
    t0 = 0
    for n in chunks:
        okc, ovc, ok2 = oracle.prefill_write(src_k[:, t0:t0 + n], src_v[:, t0:t0 + n], t0, lens,
                                             okc, ovc, ok2)
        t0 += n
    np.testing.assert_array_equal(to_host(kc).view(np.uint8), okc.view(np.uint8))
    np.testing.assert_array_equal(to_host(vc).view(np.uint8), ovc.view(np.uint8))

    ref = oracle.score(okc, lens, L["q_obs"])
    gs = to_host(s_k2).astype(np.float64)
    rel = np.abs(gs - ref) / np.maximum(ref, 1e-30)
    assert rel.max() <= SCORE_RTOL, f"score from sums rel err {rel.max():.3e}"
    np.testing.assert_allclose(gs, oracle.score_from_k2(ok2, L["q_obs"]), rtol=SCORE_RTOL, atol=0)
    rel2 = np.abs(gs - to_host(s_cache)) / np.maximum(ref, 1e-30)
    assert rel2.max() <= 2 * SCORE_RTOL
    o_idx, o_tie = oracle.select(gs, keep)
    np.testing.assert_array_equal(to_host(idx), o_idx)
    np.testing.assert_array_equal(to_host(tie), o_tie)
    print(f"[prefill] seed {seed}: score rel {rel.max():.2e}, vs cache path {rel2.max():.2e}",
          flush=True)

    # bitwise reproducible
    _, _, state2 = _run(qdk, dims, src_k, src_v, lens_d, chunks, nan, dtype_t)
    s2, _, _ = qdk.think_score_select_k2(dims, state2, qo, keep)
    torch.cuda.synchronize()
    assert torch.equal(state, state2)
    assert torch.equal(s_k2.view(torch.int32), s2.view(torch.int32))
