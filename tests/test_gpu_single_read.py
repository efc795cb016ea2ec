"""GPU parity of think_score_select_compact (stages a+b+c in one call) against
the oracle, on the same seeded inputs as the stage-by-stage tests.

Where the key cache fits on chip (think_score_compact_single_read == 1) the
call reads K once in a cooperative launch; elsewhere it runs the two-pass
kernels.  Every case states which route it expects, and checks:
 (i)   scores within 5e-6 relative of the oracle's fp64 scores
 (ii)  the oracle's selection on the GPU's fp32 scores == the GPU's indices and
       near-tie flags, bit-exact
 (iii) GPU indices == the oracle's selection on its own scores, except (b, kv)
       pairs the oracle flags as near ties
 (iv)  K_thin == oracle compaction with the GPU indices, bytewise; padding rows
       untouched
 (v)   against think_score_select + think_compact_k: the same indices wherever
       the oracle reports no near tie, and then the same K_thin bytes
 (vi)  a second call on a workspace full of random bytes (the first call's
       barrier words included) gives the same bits
"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import to_dev, to_host
from test_gpu_parity import EDGE, SCORE_RTOL, _custom

pytestmark = pytest.mark.gpu


def _qdk():
    import query_driven_kv_amd as qdk
    return qdk


def _run(qdk, k, lens, qo, keep, ws):
    B, S, Hkv, D = k.shape
    thin = torch.full((B, S, Hkv, keep), float("nan"), dtype=k.dtype, device=k.device)
    s, i, t, thin = qdk.think_score_select_compact(k, lens, qo, keep, k_thin=thin, workspace=ws)
    torch.cuda.synchronize()
    return dict(scores=to_host(s), idx=to_host(i), tie=to_host(t), thin=to_host(thin))


def check_single_read(cfg, L, keep, label, expect_single):
    qdk = _qdk()
    k, lens_d, qo = to_dev(L["k_cache"]), to_dev(L["seq_lens"]), to_dev(L["q_obs"])
    B, S, Hkv, D = k.shape
    dims = qdk.make_dims(B, cfg.n_q_heads, Hkv, D, S, qdk.THINK_BF16 if cfg.dtype == "bf16"
                         else qdk.THINK_F32)
    route = qdk.think_score_compact_single_read(dims, keep)
    print(f"[single-read] {label}: B={B} S={S} Hq={cfg.n_q_heads} Hkv={Hkv} D={D} keep={keep} "
          f"{cfg.dtype}: route {route}", flush=True)
    assert route == int(expect_single)
    nbytes = qdk.think_score_compact_workspace_bytes(dims, keep)
    gen = torch.Generator(device="cpu").manual_seed(B * 7919 + S)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen).to(k.device)
    g = _run(qdk, k, lens_d, qo, keep, ws)
    assert qdk.think_score_compact_status(dims, cfg.obs_window, keep, ws) == 0, "wait gave up"
    lens = L["seq_lens"]
    # (i)
    ref_s = oracle.score(L["k_cache"], lens, L["q_obs"])
    rel = np.abs(g["scores"].astype(np.float64) - ref_s) / np.maximum(ref_s, 1e-30)
    assert rel.max() <= SCORE_RTOL, f"score rel err {rel.max():.3e}"
    # (ii)
    o_idx, o_tie = oracle.select(g["scores"].astype(np.float64), keep)
    np.testing.assert_array_equal(g["idx"], o_idx)
    np.testing.assert_array_equal(g["tie"], o_tie)
    # (iii)
    r_idx, r_tie = oracle.select(ref_s, keep)
    diff = (g["idx"] != r_idx).any(axis=-1)
    assert not (diff & (r_tie == 0)).any(), "kept set differs outside a reported near tie"
    # (iv)
    sentinel = kvsynth.nan_value(cfg.dtype)
    ref_thin = oracle.compact(L["k_cache"], lens, g["idx"], fill=sentinel)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(g["thin"][b, :n].view(np.uint8),
                                      ref_thin[b, :n].view(np.uint8))
        assert np.isnan(kvsynth.as_float(g["thin"][b, n:])).all(), "padding rows were written"
    # (v)
    s2, i2, t2 = qdk.think_score_select(k, lens_d, qo, keep)
    thin2 = torch.full((B, S, Hkv, keep), float("nan"), dtype=k.dtype, device=k.device)
    qdk.think_compact_k(k, lens_d, i2, k_thin=thin2)
    torch.cuda.synchronize()
    i2, thin2 = to_host(i2), to_host(thin2)
    same = ~(g["idx"] != i2).any(axis=-1)                   # [B, Hkv]
    assert (same | (r_tie != 0)).all(), "single call and two calls disagree outside a near tie"
    for b, n in enumerate(lens):
        if same[b].all():
            np.testing.assert_array_equal(g["thin"][b, :n].view(np.uint8),
                                          thin2[b, :n].view(np.uint8))
    # (vi)
    ws2 = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=gen).to(k.device)
    g2 = _run(qdk, k, lens_d, qo, keep, ws2)
    g3 = _run(qdk, k, lens_d, qo, keep, ws2)               # the same workspace again
    for key in g:
        np.testing.assert_array_equal(g[key].view(np.uint8), g2[key].view(np.uint8))
        np.testing.assert_array_equal(g[key].view(np.uint8), g3[key].view(np.uint8))
    print(f"[single-read] {label}: score rel {rel.max():.2e}, near ties "
          f"{int(r_tie.sum())}", flush=True)


@pytest.mark.parametrize("name,single", [("tiny", True), ("llama2-7b-layer-4k", True),
                                         ("mistral-7b-gqa-32k", True),
                                         ("batched-ragged-16k", False)])
def test_full_configs(name, single):
    cfg = kvsynth.CONFIGS[name]
    L = kvsynth.make_layer(cfg, 0)
    check_single_read(cfg, L, cfg.keep, name, single)


# shapes of the stage-by-stage edge cases; the single-read route needs a row
# of 16-byte vectors that divides 512 and a key cache that fits on chip (one
# workgroup per compute unit, at most 32 vectors per thread of 512)
def _fits(c):
    e = 2 if c["dtype"] == "bf16" else 4
    nvec = c["n_kv_heads"] * c["head_dim"] * e // 16
    if 512 % nvec or c["n_q_heads"] // c["n_kv_heads"] * c["head_dim"] > 4096:
        return False
    ncu = min(torch.cuda.get_device_properties(0).multi_processor_count, 512)
    wps = ncu // c["batch"]
    if wps < 1 or c["n_kv_heads"] > wps:          # one selecting workgroup per (b, kv)
        return False
    rpw = -(-c["seq_capacity"] // wps)
    return rpw * nvec <= 32 * 512


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{c['seed']}" for c in EDGE])
def test_edge_shapes(case):
    c = dict(case)
    seed, lens = c.pop("seed"), c.pop("lens")
    cfg, L, _ = _custom(seed, lens, **c)
    check_single_read(cfg, L, cfg.keep, f"edge{seed}", _fits(case))


EXTRA = [
    # window of one query; 16 query heads per kv head at D = 256 (G*D = 4096)
    dict(seed=40, lens=[2000, 1999, 1], batch=3, n_q_heads=16, n_kv_heads=1, head_dim=256,
         seq_capacity=2000, keep=200, dtype="bf16", obs_window=1),
    # fp32 rows of 32 vectors, every tile short of its last rows
    dict(seed=41, lens=[1023, 700], batch=2, n_q_heads=8, n_kv_heads=8, head_dim=64,
         seq_capacity=1023, keep=31, dtype="f32"),
    # a key cache just past what fits (two passes)
    dict(seed=42, lens=[33000], batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
         seq_capacity=33000, keep=64, dtype="bf16", lowrank=8),
    # 32 sequences of 8 kv heads: exactly one selecting workgroup per (b, kv)
    # row fits (8 workgroups per sequence); 40 sequences do not (two passes)
    dict(seed=44, lens=[(i * 131) % 600 + 1 for i in range(32)], batch=32, n_q_heads=32,
         n_kv_heads=8, head_dim=128, seq_capacity=600, keep=64, dtype="bf16", lowrank=8),
    dict(seed=45, lens=[(i * 97) % 300 + 1 for i in range(40)], batch=40, n_q_heads=32,
         n_kv_heads=8, head_dim=128, seq_capacity=300, keep=64, dtype="bf16", lowrank=8),
    # more sequences than compute units (two passes)
    dict(seed=43, lens=[(i * 7) % 50 + 1 for i in range(300)], batch=300, n_q_heads=2,
         n_kv_heads=1, head_dim=128, seq_capacity=50, keep=64, dtype="bf16"),
]


@pytest.mark.parametrize("case", EXTRA, ids=[f"extra{c['seed']}" for c in EXTRA])
def test_extra_shapes(case):
    c = dict(case)
    seed, lens = c.pop("seed"), c.pop("lens")
    cfg, L, _ = _custom(seed, lens, **c)
    check_single_read(cfg, L, cfg.keep, f"extra{seed}", _fits(case))


def test_random_shapes():
    """Seeded random shapes through the one-call pruning: bf16 and fp32, head
    dims 8-256, batches of 1-40 with ragged lengths, every kind of keep and
    window; each states its route and passes the checks above."""
    rng = np.random.default_rng(909)
    for case in range(16):
        dtype = "f32" if case % 4 == 3 else "bf16"
        D = int(rng.choice([8, 32, 64, 128, 128, 256]))
        B = int(rng.choice([1, 1, 2, 5, 16, 40]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4]))
        while Hkv * D * (2 if dtype == "bf16" else 4) > 32768:
            Hkv //= 2
        S = int(rng.integers(1, 3000)) if B <= 5 else int(rng.integers(1, 400))
        keep = int(rng.integers(1, D + 1))
        lens = [int(x) for x in rng.integers(1, S + 1, B)]
        c = dict(batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv, head_dim=D, seq_capacity=S,
                 keep=keep, dtype=dtype, obs_window=int(rng.integers(1, 65)))
        cfg, L, _ = _custom(200 + case, lens, **c)
        check_single_read(cfg, L, keep, f"random{case}", _fits(c))


def test_give_up_is_reported_and_cleared():
    """A single-read launch whose waits give up says so through
    think_score_compact_status; the next launch on the same workspace clears the
    report and gives the normal result.  The give-up is forced from the host
    (the test hook makes every wait look for a tag that is never written and stop
    after a few polls), so every workgroup still finishes normally."""
    qdk = _qdk()
    cfg = kvsynth.CONFIGS["mistral-7b-gqa-32k"]
    L = kvsynth.make_layer(cfg, 0)
    k, lens_d, qo = to_dev(L["k_cache"]), to_dev(L["seq_lens"]), to_dev(L["q_obs"])
    B, S, Hkv, D = k.shape
    dims = qdk.make_dims(B, cfg.n_q_heads, Hkv, D, S, qdk.THINK_BF16)
    assert qdk.think_score_compact_single_read(dims, cfg.keep) == 1
    ws = torch.zeros(qdk.think_score_compact_workspace_bytes(dims, cfg.keep), dtype=torch.uint8,
                     device=k.device)
    good = _run(qdk, k, lens_d, qo, cfg.keep, ws)
    assert qdk.think_score_compact_status(dims, cfg.obs_window, cfg.keep, ws) == 0
    print("[single-read] give-up: forcing every wait to run out", flush=True)
    prev = qdk.think_single_read_test_give_up(True)
    try:
        _run(qdk, k, lens_d, qo, cfg.keep, ws)
    finally:
        qdk.think_single_read_test_give_up(prev)
    assert qdk.think_score_compact_status(dims, cfg.obs_window, cfg.keep, ws) == -8
    prev = qdk.think_single_read_test_give_up(True)
    try:
        with pytest.raises(qdk.ThinkError) as ei:
            qdk.think_score_select_compact(k, lens_d, qo, cfg.keep, workspace=ws,
                                           check_status=True)
    finally:
        qdk.think_single_read_test_give_up(prev)
    assert ei.value.status == -8
    again = _run(qdk, k, lens_d, qo, cfg.keep, ws)
    assert qdk.think_score_compact_status(dims, cfg.obs_window, cfg.keep, ws) == 0
    for key in good:
        np.testing.assert_array_equal(good[key].view(np.uint8), again[key].view(np.uint8))
    # a two-pass shape never waits
    c2 = kvsynth.CONFIGS["batched-ragged-16k"]
    d2 = qdk.make_dims(c2.batch, c2.n_q_heads, c2.n_kv_heads, c2.head_dim, c2.seq_capacity,
                       qdk.THINK_BF16)
    assert qdk.think_score_compact_single_read(d2, c2.keep) == 0
    ws2 = torch.zeros(qdk.think_score_compact_workspace_bytes(d2, c2.keep), dtype=torch.uint8,
                      device=k.device)
    assert qdk.think_score_compact_status(d2, c2.obs_window, c2.keep, ws2) == 0
