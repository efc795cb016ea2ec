"""The HIP path at the size limits, where the oracle cannot run over the whole
input: structured inputs whose results have closed forms that hold at any size.

Every key row equals one vector k, so for t < len_b
  score[b,kv,c] = sqrt(len_b) * |k_c| * sum_g ||Q_w[b,:,kv*G+g,c]||   (stage (a))
  K_thin rows all equal k[kept_idx]                                     (stage (c))
  every logit is equal, so attention is uniform and the output is the mean of
  the value rows, which repeat a 4-row pattern (len_b a multiple of 4) (stage (d))
The selection is checked against the oracle's selection of the same fp32 scores.
Cases: 16M tokens on the matrix-core decode path (4 GiB key and value caches),
4M tokens with head_dim 8 on the general path, and 65535 one-token sequences
(the batch limit)."""
import math

import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import to_host

pytestmark = pytest.mark.gpu


def _structured(B, S, Hkv, G, D, lens, seed):
    rng = np.random.default_rng(seed)
    kvec = kvsynth.to_bf16_bits((rng.choice([0.25, 0.5, 1.0, 1.5, 2.0, 3.0], size=(Hkv, D))
                                 * rng.choice([-1.0, 1.0], size=(Hkv, D))).astype(np.float32))
    pat = kvsynth.to_bf16_bits(rng.standard_normal((4, Hkv, D)).astype(np.float32))
    W = 3
    qo = kvsynth.to_bf16_bits(rng.standard_normal((B, W, Hkv * G, D)).astype(np.float32))
    q = kvsynth.to_bf16_bits(rng.standard_normal((B, Hkv * G, D)).astype(np.float32))
    dev = "cuda"
    kf = torch.from_numpy(kvsynth.as_float(kvec)).to(dev).to(torch.bfloat16)
    pf = torch.from_numpy(kvsynth.as_float(pat)).to(dev).to(torch.bfloat16)
    k = torch.empty(B, S, Hkv, D, dtype=torch.bfloat16, device=dev)
    k.copy_(kf.view(1, 1, Hkv, D).expand(B, S, Hkv, D))
    v = torch.empty_like(k)
    reps = S // 4
    v.view(B, reps, 4, Hkv, D).copy_(pf.view(1, 1, 4, Hkv, D).expand(B, reps, 4, Hkv, D))
    return kvec, pat, qo, q, k, v


def _check(B, S, Hkv, G, D, lens, keep, seed):
    import query_driven_kv_amd as qdk
    print(f"[limits] B={B} S={S} Hkv={Hkv} G={G} D={D} keep={keep} lens {sorted(set(lens))[:3]}",
          flush=True)
    assert all(n % 4 == 0 and 0 < n <= S for n in lens) and S % 4 == 0
    kvec, pat, qo, q, k, v = _structured(B, S, Hkv, G, D, lens, seed)
    lens_np = np.asarray(lens, np.int32)
    lens_d = torch.from_numpy(lens_np).cuda()
    to_bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    scores, idx, tie = qdk.think_score_select(k, lens_d, to_bf(qo), keep)
    thin = qdk.think_compact_k(k, lens_d, idx)
    out = qdk.think_decode_attn(to_bf(q), thin, v, lens_d, idx, 1.0 / math.sqrt(D))
    torch.cuda.synchronize()

    # (a) closed form of the score
    kv64 = kvsynth.as_float(kvec).astype(np.float64)                     # [Hkv, D]
    q64 = kvsynth.as_float(qo).astype(np.float64)                          # [B, W, Hq, D]
    qn = np.sqrt((q64 ** 2).sum(axis=1)).reshape(B, Hkv, G, D).sum(axis=2)
    ref = np.sqrt(lens_np.astype(np.float64))[:, None, None] * np.abs(kv64)[None] * qn
    gs = to_host(scores).astype(np.float64)
    rel = np.abs(gs - ref) / np.maximum(ref, 1e-300)
    assert rel.max() <= 5e-6, f"score rel err {rel.max():.3e}"
    # (b) the selection of those fp32 scores
    o_idx, o_tie = oracle.select(gs, keep)
    gi = to_host(idx)
    np.testing.assert_array_equal(gi, o_idx)
    np.testing.assert_array_equal(to_host(tie), o_tie)
    # (c) every valid thin row is k[kept_idx]
    want = torch.from_numpy(np.take_along_axis(kvec[None].repeat(B, 0), gi, axis=-1)
                            .view(np.int16)).cuda()
    th = thin.view(torch.int16)
    for b in sorted(set([0, B - 1])):
        n = int(lens_np[b])
        assert torch.equal(th[b, :n], want[b].unsqueeze(0).expand(n, Hkv, keep)), f"thin rows, b={b}"
    if B > 2:
        n0 = int(lens_np.min())
        assert torch.equal(th[:, :n0], want.unsqueeze(1).expand(B, n0, Hkv, keep))
    # (d) uniform attention: the mean of the 4 pattern rows
    mean = kvsynth.as_float(pat).astype(np.float64).mean(axis=0)            # [Hkv, D]
    exp = np.repeat(mean, G, axis=0)[None]                                  # [1, Hq, D]
    go = kvsynth.as_float(to_host(out)).astype(np.float64)
    err = np.abs(go - exp).max(axis=-1) / np.abs(exp).max(axis=-1)
    assert err.max() <= 2e-2, f"decode row error {err.max():.3e}"
    print(f"[limits] score rel {rel.max():.2e}, decode row err {err.max():.2e}", flush=True)


def test_sixteen_million_tokens_matrix_core_path():
    S = 1 << 24
    _check(1, S, 1, 4, 128, [S], keep=64, seed=70)


def test_four_million_tokens_general_path_ragged():
    S = 1 << 22
    _check(2, S, 2, 2, 8, [S, S - 1024], keep=3, seed=71)


def test_batch_limit():
    B = 65535
    _check(B, 4, 2, 2, 16, [4] * B, keep=5, seed=72)
