"""GPU parity: every stage of the HIP path against the fp64 oracle on the same
seeded inputs, stage by stage so a failure points at one kernel.

 (i)   scores within 5e-6 relative of the oracle's fp64 scores
 (ii)  think_select(GPU scores) == oracle select on the same fp32 scores, bit-exact
       (indices and near-tie flags)
 (iii) GPU indices == oracle select on the oracle's scores, except (b, kv)
       pairs the oracle flags as near ties (listed, never hidden)
 (iv)  think_compact_k == oracle compaction with the GPU indices, bytewise;
       padding rows of K_thin untouched
 (v)   think_decode_attn vs oracle decode (GPU indices, compacted keys):
       per-row max-abs relative error <= 1e-5 (fp32) / 2e-2 (bf16)
 (vi)  two runs bit-identical
Padding rows of every cache hold a NaN sentinel, so a read past len_b shows up.
"""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import row_rel_err, to_dev, to_host, tol_for

pytestmark = pytest.mark.gpu

SCORE_RTOL = 5e-6


def _qdk():
    import query_driven_kv_amd as qdk
    return qdk


def run_path(L, keep, q, scale):
    qdk = _qdk()
    k = to_dev(L["k_cache"])
    v = to_dev(L["v_cache"])
    lens = to_dev(L["seq_lens"])
    qo = to_dev(L["q_obs"])
    qd = to_dev(q)
    scores = qdk.think_score(k, lens, qo)
    idx, tie = qdk.think_select(scores, keep)
    # the fused entry point must give the same bits
    s2, i2, t2 = qdk.think_score_select(k, lens, qo, keep)
    assert torch.equal(scores.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(idx, i2) and torch.equal(tie, t2)
    B, S, Hkv, D = k.shape
    thin = torch.full((B, S, Hkv, keep), float("nan"), dtype=k.dtype, device=k.device)
    qdk.think_compact_k(k, lens, idx, k_thin=thin)
    out = qdk.think_decode_attn(qd, thin, v, lens, idx, scale)
    torch.cuda.synchronize()
    return dict(scores=to_host(scores), idx=to_host(idx), tie=to_host(tie), thin=to_host(thin),
                out=to_host(out))


def check_all(cfg, L, keep, q, scale, label):
    print(f"[parity] {label}: B={cfg.batch} S={cfg.seq_capacity} Hq={cfg.n_q_heads} "
          f"Hkv={cfg.n_kv_heads} D={cfg.head_dim} keep={keep} {cfg.dtype}", flush=True)
    g = run_path(L, keep, q, scale)
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
    near = list(zip(*np.nonzero(r_tie)))
    if near:
        print(f"[parity] {label}: near ties at (b, kv) {near}", flush=True)
    # (iv)
    sentinel = kvsynth.nan_value(cfg.dtype)
    ref_thin = oracle.compact(L["k_cache"], lens, g["idx"], fill=sentinel)
    for b, n in enumerate(lens):
        np.testing.assert_array_equal(g["thin"][b, :n].view(np.uint8), ref_thin[b, :n].view(np.uint8))
        assert np.isnan(kvsynth.as_float(g["thin"][b, n:])).all(), "padding rows of K_thin were written"
    # (v)
    ref_o = oracle.decode(q, ref_thin, L["v_cache"], lens, g["idx"], scale)
    err = row_rel_err(g["out"], ref_o)
    assert err.max() <= tol_for(cfg.dtype), f"decode row error {err.max():.3e}"
    print(f"[parity] {label}: score rel {rel.max():.2e}, decode row err {err.max():.2e}", flush=True)
    return g


@pytest.mark.parametrize("name", ["tiny", "llama2-7b-layer-4k", "mistral-7b-gqa-32k",
                                  "batched-ragged-16k"])
def test_full_config_parity(name):
    cfg = kvsynth.CONFIGS[name]
    L = kvsynth.make_layer(cfg, 0)
    q = kvsynth.decode_q(cfg, 0, 0, L["channel_scale"])
    scale = np.float32(1.0 / np.sqrt(cfg.head_dim))
    g1 = check_all(cfg, L, cfg.keep, q, scale, name)
    # (vi) determinism
    g2 = run_path(L, cfg.keep, q, scale)
    for key in g1:
        np.testing.assert_array_equal(g1[key].view(np.uint8), g2[key].view(np.uint8))


def test_llama3_128k_sampled_layers():
    """The 32-layer 128K workload at full per-layer size, in the launch
    configuration the benchmark times: layers 0 and 31, decode steps 0 and 127."""
    cfg = kvsynth.CONFIGS["llama3-8b-128k"]
    scale = np.float32(1.0 / np.sqrt(cfg.head_dim))
    for layer in (0, 31):
        L = kvsynth.make_layer(cfg, layer)
        for step in (0, 127):
            q = kvsynth.decode_q(cfg, layer, step, L["channel_scale"])
            check_all(cfg, L, cfg.keep, q, scale, f"llama3 layer {layer} step {step}")


def _custom(seed, lens, **kw):
    cfg = kvsynth.custom(f"edge{seed}", cfg_id=90, ragged=None, **kw)
    L = kvsynth.make_layer(cfg, layer=seed)
    lens = np.asarray(lens, np.int32)
    for b in range(cfg.batch):
        L["k_cache"][b, lens[b]:] = kvsynth.nan_value(cfg.dtype)
        L["v_cache"][b, lens[b]:] = kvsynth.nan_value(cfg.dtype)
    L["seq_lens"] = lens
    q = kvsynth.decode_q(cfg, seed, 0, L["channel_scale"])
    return cfg, L, q


EDGE = [
    # ragged tails, lengths of 1 and not multiples of any tile, odd keep
    dict(seed=1, lens=[1, 17, 255, 300], batch=4, n_q_heads=8, n_kv_heads=2, head_dim=128,
         seq_capacity=300, keep=77, dtype="bf16", lowrank=8),
    dict(seed=2, lens=[1000, 999], batch=2, n_q_heads=4, n_kv_heads=1, head_dim=128,
         seq_capacity=1001, keep=51, dtype="bf16", lowrank=8),
    dict(seed=3, lens=[513], batch=1, n_q_heads=16, n_kv_heads=1, head_dim=64, seq_capacity=513,
         keep=13, dtype="f32"),
    dict(seed=4, lens=[70, 3], batch=2, n_q_heads=4, n_kv_heads=4, head_dim=8, seq_capacity=77,
         keep=1, dtype="f32"),
    dict(seed=5, lens=[129], batch=1, n_q_heads=4, n_kv_heads=2, head_dim=256, seq_capacity=129,
         keep=256, dtype="bf16"),
    dict(seed=6, lens=[40], batch=1, n_q_heads=64, n_kv_heads=64, head_dim=256, seq_capacity=40,
         keep=100, dtype="bf16"),                 # widest row: 64*256*2 = 32 KiB
    dict(seed=7, lens=[2049, 4096, 1], batch=3, n_q_heads=12, n_kv_heads=3, head_dim=40,
         seq_capacity=4096, keep=5, dtype="f32"),
    # head_dim 128 bf16 (matrix-core kernel): even keep not a multiple of 8, every
    # channel kept, a single channel kept, groups of 8 and 16 query heads
    dict(seed=8, lens=[777, 1], batch=2, n_q_heads=16, n_kv_heads=2, head_dim=128,
         seq_capacity=800, keep=42, dtype="bf16", lowrank=16),
    dict(seed=9, lens=[300], batch=1, n_q_heads=16, n_kv_heads=1, head_dim=128,
         seq_capacity=300, keep=128, dtype="bf16"),
    dict(seed=10, lens=[129, 64, 1000], batch=3, n_q_heads=3, n_kv_heads=3, head_dim=128,
         seq_capacity=1000, keep=1, dtype="bf16"),
    dict(seed=11, lens=[5000, 2500], batch=2, n_q_heads=32, n_kv_heads=4, head_dim=128,
         seq_capacity=5000, keep=96, dtype="bf16", lowrank=32),
    # rows at every offset from a 16-byte boundary (odd Hkv*keep), one to three
    # 32-channel blocks; and the widest odd and even rows off dword boundaries
    dict(seed=12, lens=[1500, 31, 700], batch=3, n_q_heads=10, n_kv_heads=5, head_dim=128,
         seq_capacity=1500, keep=33, dtype="bf16", lowrank=8),
    dict(seed=13, lens=[2100], batch=1, n_q_heads=21, n_kv_heads=3, head_dim=128,
         seq_capacity=2100, keep=90, dtype="bf16", lowrank=8),
    dict(seed=14, lens=[999, 64], batch=2, n_q_heads=6, n_kv_heads=3, head_dim=128,
         seq_capacity=1000, keep=101, dtype="bf16", lowrank=8),
    dict(seed=15, lens=[640], batch=1, n_q_heads=8, n_kv_heads=1, head_dim=128,
         seq_capacity=640, keep=126, dtype="bf16", lowrank=8),
    # a cache filled far below its capacity: the chunk follows the length
    dict(seed=16, lens=[3000, 11], batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
         seq_capacity=20000, keep=64, dtype="bf16", lowrank=8),
    # 64 ragged sequences (chunk slots dealt by length), and 65 (past the batch
    # size that deals slots: per-sequence chunks)
    dict(seed=17, lens=[(i * 37) % 700 + 1 for i in range(64)], batch=64,
         n_q_heads=8, n_kv_heads=2, head_dim=128, seq_capacity=700, keep=51, dtype="bf16",
         lowrank=8),
    dict(seed=18, lens=[(i * 53) % 600 + 1 for i in range(65)], batch=65, n_q_heads=4,
         n_kv_heads=1, head_dim=128, seq_capacity=600, keep=64, dtype="bf16", lowrank=8),
    # a batch with aligned thin rows of one 32-channel block (three workgroups
    # per CU)
    dict(seed=20, lens=[4000, 2047, 1], batch=3, n_q_heads=12, n_kv_heads=2, head_dim=128,
         seq_capacity=4000, keep=24, dtype="bf16", lowrank=8),
    # one long sequence among 63 of 1-5 tokens: it takes almost every slot
    dict(seed=19, lens=[6000] + [1 + i % 5 for i in range(63)], batch=64, n_q_heads=4,
         n_kv_heads=1, head_dim=128, seq_capacity=6000, keep=77, dtype="bf16", lowrank=8),
]


@pytest.mark.parametrize("case", EDGE, ids=[f"edge{c['seed']}" for c in EDGE])
def test_edge_shapes(case):
    case = dict(case)
    seed, lens, keep = case.pop("seed"), case.pop("lens"), case.pop("keep")
    cfg, L, q = _custom(seed, lens, obs_window=7, keep=keep, **case)
    check_all(cfg, L, keep, q, np.float32(1.0 / np.sqrt(cfg.head_dim)), f"edge{seed}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_keep_all_reproduces_unpruned_attention(dtype):
    cfg, L, q = _custom(20, [333, 64], batch=2, n_q_heads=8, n_kv_heads=2, head_dim=64,
                        seq_capacity=333, keep=64, dtype=dtype, obs_window=5)
    scale = np.float32(1.0 / 8.0)
    g = check_all(cfg, L, 64, q, scale, f"keep=D {dtype}")
    assert (g["idx"] == np.arange(64)).all()
    full = oracle.full_attn(q, L["k_cache"], L["v_cache"], L["seq_lens"], scale)
    assert row_rel_err(g["out"], full).max() <= tol_for(dtype)


def test_exact_tie_goes_to_lower_channel_and_is_flagged():
    cfg, L, q = _custom(21, [200], batch=1, n_q_heads=2, n_kv_heads=1, head_dim=32,
                        seq_capacity=200, keep=16, dtype="bf16", obs_window=4)
    s = oracle.score(L["k_cache"], L["seq_lens"], L["q_obs"])[0, 0]
    order = np.lexsort((np.arange(32), -s))
    a, b = sorted(order[15:17])                 # straddle the cutoff at keep=16
    for key in ("k_cache", "q_obs"):
        L[key][..., b] = L[key][..., a]
    g = check_all(cfg, L, 16, q, np.float32(0.2), "exact tie")
    assert g["tie"][0, 0] == 1
    kept = set(g["idx"][0, 0].tolist())
    assert a in kept and b not in kept


def test_select_on_crafted_scores_matches_the_oracle():
    """think_select on scores drawn from a few fp32 values (many exact ties,
    +0 and -0, subnormals, the largest finite magnitude): kept channels and
    near-tie flags bit-exact against the oracle's selection of the same
    values, for head dims on both selection instances (128 and others)."""
    qdk = _qdk()
    rng = np.random.default_rng(77)
    tiny = np.float32(1e-40)                                   # subnormal
    pool = np.array([0.0, -0.0, tiny, 2 * tiny, 1.0, np.nextafter(np.float32(1), np.float32(2)),
                     2.5, 7.0, 3.0e38], dtype=np.float32)
    for D in (8, 64, 96, 128, 256):
        for keep in sorted({1, max(1, D // 3), D // 2, D - 1, D}):
            print(f"[select] D={D} keep={keep}", flush=True)
            s = pool[rng.integers(0, len(pool), size=(2, 5, D))]
            s[0, 0] = np.float32(2.5)                          # one value throughout
            s[1, 1] = np.where(rng.random(D) < 0.5, np.float32(0.0), np.float32(-0.0))
            idx, tie = qdk.think_select(to_dev(s), keep)
            torch.cuda.synchronize()
            o_idx, o_tie = oracle.select(s.astype(np.float64), keep)
            np.testing.assert_array_equal(to_host(idx), o_idx)
            np.testing.assert_array_equal(to_host(tie), o_tie)


def test_empty_sequences_in_a_ragged_batch_decode_to_zero():
    """Matrix-core decode with chunk slots dealt by length: empty sequences
    get no slot and a zero output; the others match the oracle one by one."""
    qdk = _qdk()
    lens = np.array([0, 900, 0, 5, 1300, 0, 1, 640, 0, 0, 77, 1024], np.int32)
    B, Hq, Hkv, D, S, keep = len(lens), 8, 2, 128, 1300, 51
    rng = np.random.default_rng(23)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    q = bf(rng.standard_normal((B, Hq, D)))
    thin = bf(rng.standard_normal((B, S, Hkv, keep)))
    v = bf(rng.standard_normal((B, S, Hkv, D)))
    idx = np.sort(np.stack([np.stack([rng.choice(D, keep, replace=False) for _ in range(Hkv)])
                            for _ in range(B)]), axis=-1).astype(np.int32)
    out = qdk.think_decode_attn(q.cuda(), thin.cuda(), v.cuda(), to_dev(lens), to_dev(idx), 0.1)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    h = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    for b in range(B):
        if lens[b] == 0:
            assert (got[b] == 0).all(), b
            continue
        ref = oracle.decode(h(q[b:b + 1]), h(thin[b:b + 1]), h(v[b:b + 1]), lens[b:b + 1],
                            idx[b:b + 1], np.float32(0.1))
        assert row_rel_err(out[b:b + 1], ref).max() <= 2e-2, b


def test_zero_length_sequence_gives_zero_scores_and_output():
    qdk = _qdk()
    cfg, L, q = _custom(22, [50, 50], batch=2, n_q_heads=2, n_kv_heads=2, head_dim=16,
                        seq_capacity=50, keep=8, dtype="f32", obs_window=3)
    lens = np.array([50, 0], np.int32)
    k, v, qo = to_dev(L["k_cache"]), to_dev(L["v_cache"]), to_dev(L["q_obs"])
    dl = to_dev(lens)
    s = qdk.think_score(k, dl, qo)
    idx, _ = qdk.think_select(s, 8)
    thin = torch.zeros(2, 50, 2, 8, dtype=k.dtype, device=k.device)
    qdk.think_compact_k(k, dl, idx, k_thin=thin)
    out = qdk.think_decode_attn(to_dev(q), thin, v, dl, idx, 0.25)
    torch.cuda.synchronize()
    assert (to_host(s)[1] == 0).all()
    assert (to_host(out)[1] == 0).all()
    assert (to_host(thin)[1] == 0).all()


def test_decode_workspace_reused_across_calls_and_shapes():
    """One workspace, filled with garbage first, serves consecutive calls of
    different shapes: no state survives between calls."""
    qdk = _qdk()
    cases = [(31, [4000, 2222], 4, 1, 64), (32, [700], 8, 2, 51), (33, [129, 1, 5000], 2, 2, 96)]
    ws = torch.full((1 << 22,), 0xA5, dtype=torch.uint8, device="cuda")
    for rep in range(2):
        for seed, lens, Hq, Hkv, keep in cases:
            cfg, L, q = _custom(seed, lens, batch=len(lens), n_q_heads=Hq * Hkv, n_kv_heads=Hkv,
                                head_dim=128, seq_capacity=max(lens), keep=keep, dtype="bf16",
                                obs_window=4, lowrank=8)
            rng = np.random.default_rng(seed)
            idx = np.sort(np.stack([np.stack([rng.choice(128, keep, replace=False) for _ in range(Hkv)])
                                    for _ in range(len(lens))]), axis=-1).astype(np.int32)
            thin = oracle.compact(L["k_cache"], L["seq_lens"], idx)
            dims = qdk.make_dims(len(lens), Hq * Hkv, Hkv, 128, max(lens), torch.bfloat16)
            assert qdk.think_decode_workspace_bytes(dims, keep) <= ws.numel()
            out = qdk.think_decode_attn(to_dev(q), to_dev(thin), to_dev(L["v_cache"]),
                                        to_dev(L["seq_lens"]), to_dev(idx), 0.1, workspace=ws)
            torch.cuda.synchronize()
            ref = oracle.decode(q, thin, L["v_cache"], L["seq_lens"], idx, np.float32(0.1))
            assert row_rel_err(out, ref).max() <= 2e-2, (rep, seed)


def test_split_phase_decode_is_bitwise_the_single_call():
    qdk = _qdk()
    for seed, lens, Hq, Hkv, D, keep, dtype in [(40, [3000, 17], 8, 2, 128, 64, "bf16"),
                                                (41, [900], 6, 3, 64, 20, "f32"),
                                                (42, [2048, 2047], 32, 8, 128, 77, "bf16"),
                                                (43, [30000], 32, 8, 128, 51, "bf16"),
                                                (44, [(i * 97) % 2000 + 1 for i in range(70)],
                                                 2, 1, 128, 96, "bf16")]:
        cfg, L, q = _custom(seed, lens, batch=len(lens), n_q_heads=Hq, n_kv_heads=Hkv,
                            head_dim=D, seq_capacity=max(lens), keep=keep, dtype=dtype,
                            obs_window=4)
        k, v, lensd, qd = to_dev(L["k_cache"]), to_dev(L["v_cache"]), to_dev(L["seq_lens"]), to_dev(q)
        s = qdk.think_score(k, lensd, to_dev(L["q_obs"]))
        idx, _ = qdk.think_select(s, keep)
        thin = qdk.think_compact_k(k, lensd, idx)
        one = qdk.think_decode_attn(qd, thin, v, lensd, idx, 0.125)
        dims = qdk.make_dims(len(lens), Hq, Hkv, D, max(lens), qd.dtype)
        ws = torch.empty(qdk.think_decode_workspace_bytes(dims, keep), dtype=torch.uint8, device="cuda")
        dims, kk = qdk.think_decode_attn_partial(qd, thin, v, lensd, idx, 0.125, ws)
        two = qdk.think_decode_attn_combine(dims, kk, lensd, ws, torch.empty_like(one))
        torch.cuda.synchronize()
        assert torch.equal(one.view(torch.int16) if one.dtype == torch.bfloat16 else one.view(torch.int32),
                           two.view(torch.int16) if two.dtype == torch.bfloat16 else two.view(torch.int32))


def test_random_decode_shapes_match_the_oracle():
    """Seeded random decode shapes on the bf16 matrix-core path: batch 1-70
    (one sequence, length-dealt slots, per-sequence chunks), every keep from
    1 to 128 over the draws, groups of 1-16 query heads, ragged lengths.
    Each output row within the bf16 bound of the oracle."""
    qdk = _qdk()
    rng = np.random.default_rng(2024)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    h = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    keeps = list(rng.permutation(np.arange(1, 129)))
    for case in range(64):
        B = int(rng.choice([1, 1, 2, 3, 5, 8, 13, 64, 70]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 7, 16]))
        S = int(rng.integers(1, 2600)) if B <= 8 else int(rng.integers(1, 300))
        keep = int(keeps[case % len(keeps)]) if case < 56 else int(rng.choice([64, 96, 128, 8]))
        lens = rng.integers(1, S + 1, B).astype(np.int32)
        print(f"[case {case}] B={B} Hkv={Hkv} G={G} S={S} keep={keep}", flush=True)
        q = bf(rng.standard_normal((B, Hkv * G, 128)))
        thin = bf(rng.standard_normal((B, S, Hkv, keep)))
        v = bf(rng.standard_normal((B, S, Hkv, 128)))
        idx = np.sort(np.stack([np.stack([rng.choice(128, keep, replace=False)
                                          for _ in range(Hkv)]) for _ in range(B)]),
                      axis=-1).astype(np.int32)
        out = qdk.think_decode_attn(q.cuda(), thin.cuda(), v.cuda(), to_dev(lens), to_dev(idx),
                                    0.09)
        torch.cuda.synchronize()
        ref = oracle.decode(h(q), h(thin), h(v), lens, idx, np.float32(0.09))
        err = row_rel_err(out, ref).max()
        assert err <= 2e-2, (case, B, Hkv, G, S, keep, err)


def test_random_full_path_shapes_match_the_oracle():
    """Seeded random shapes through score, selection, compaction and decode:
    bf16 and fp32, head_dim 8-256, ragged batches of 1-66 sequences, keep from
    1 to head_dim, windows of 1-40 queries."""
    rng = np.random.default_rng(77)
    for case in range(16):
        dtype = "bf16" if case % 4 else "f32"
        D = int(rng.choice([128, 128, 64, 256, 8, 40])) if dtype == "f32" else \
            int(rng.choice([128, 128, 128, 64, 256]))
        B = int(rng.choice([1, 2, 3, 7, 66]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 16]))
        while Hkv * D * (2 if dtype == "bf16" else 4) > 32768:
            Hkv //= 2
        S = int(rng.integers(1, 1200)) if B <= 7 else int(rng.integers(1, 120))
        keep = int(rng.integers(1, D + 1))
        lens = [int(x) for x in rng.integers(1, S + 1, B)]
        lens[0] = S
        cfg, L, q = _custom(100 + case, lens, batch=B, n_q_heads=Hkv * G, n_kv_heads=Hkv,
                            head_dim=D, seq_capacity=S, keep=keep, dtype=dtype,
                            obs_window=int(rng.integers(1, 41)))
        check_all(cfg, L, keep, q, np.float32(1.0 / np.sqrt(D)), f"random{case}")
