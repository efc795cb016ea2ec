"""GPU parity of the decode-time append against the oracle, several steps in
a row on the same seeded inputs: think_append_kv then think_decode_attn, and
the fused think_append_decode_attn (the append folded into the decode's
merge).  The thin-key and value caches and the lengths must match the
oracle's byte for byte after every step (the padding beyond the new length
still holds the NaN sentinel), and the attention over len_b + 1 tokens must be
within the decode tolerance.  Cases cover ragged batches (chunk slots dealt by
length), one long sequence, batches past the balanced range, odd keep, fp32,
empty sequences, a sequence that fills its last slot and one already at
capacity (left as it is, attending over its cached tokens only), and long
sequences whose merge runs in column slices (only the first slice writes the
new token's rows and advances the length)."""
import numpy as np
import pytest
import torch

import kvsynth
import oracle
from gpu_util import row_rel_err, to_dev, to_host, tol_for

pytestmark = pytest.mark.gpu

CASES = [
    # seed, lens, Hq, Hkv, D, S_cap, keep, dtype
    (50, [300, 17, 511], 8, 2, 128, 512, 64, "bf16"),     # matrix-core decode, ragged
    (51, [1000, 998], 4, 1, 128, 1000, 51, "bf16"),        # odd keep; one sequence full
    (52, [63, 40], 6, 3, 64, 66, 20, "f32"),               # general decode, fp32
    (53, [5, 2047], 32, 8, 128, 2048, 77, "bf16"),         # slot S_cap-1 filled by the first step
    (54, [0, 700, 0, 33], 8, 2, 128, 1024, 32, "bf16"),   # empty sequences
    (55, [9000], 32, 8, 128, 9216, 64, "bf16"),            # one long sequence
    (56, [0, 130], 4, 2, 32, 160, 9, "f32"),               # general decode, empty sequence
    (57, [(37 * i) % 300 for i in range(70)], 8, 2, 128, 300, 40, "bf16"),  # B past 64
    (58, [2, 1], 4, 1, 64, 2, 16, "bf16"),                 # capacity 2: both full by step 2
    (59, [39990], 32, 8, 128, 40000, 64, "bf16"),          # merge in four column slices
    (60, [6000], 8, 2, 256, 6100, 100, "f32"),             # general decode, sliced merge
]


@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("case", CASES, ids=[f"append{c[0]}" for c in CASES])
def test_append_then_decode(case, fused):
    import query_driven_kv_amd as qdk
    seed, lens, Hq, Hkv, D, S, keep, dtype = case
    B = len(lens)
    print(f"[append] seed {seed} fused={fused}: B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} "
          f"keep={keep} {dtype}", flush=True)
    cfg = kvsynth.custom(f"append{seed}", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                         seq_capacity=S, obs_window=4, keep=keep, dtype=dtype, cfg_id=91,
                         lowrank=8 if D >= 64 else 0)
    L = kvsynth.make_layer(cfg, layer=seed)
    lens = np.asarray(lens, np.int32)
    nan = kvsynth.nan_value(dtype)
    # an empty sequence takes its channel set from the one token the cache
    # held before it was emptied; its row 0 is padding again afterwards
    lens_sel = np.maximum(lens, 1)
    for b in range(B):
        L["k_cache"][b, lens_sel[b]:] = nan
        L["v_cache"][b, lens_sel[b]:] = nan
    s = oracle.score(L["k_cache"], lens_sel, L["q_obs"])
    idx, _ = oracle.select(s, keep)
    thin = oracle.compact(L["k_cache"], lens_sel, idx, fill=nan)
    v = L["v_cache"]
    for b in np.flatnonzero(lens == 0):
        thin[b, 0] = nan
        v[b, 0] = nan
    scale = np.float32(1.0 / np.sqrt(D))

    thin_d, v_d, lens_d, idx_d = to_dev(thin), to_dev(v), to_dev(lens), to_dev(idx)
    o_thin, o_v, o_lens = thin, v, lens
    for step in range(3):
        k_new, v_new = kvsynth.decode_kv(cfg, seed, step, L["channel_scale"])
        q = kvsynth.decode_q(cfg, seed, step, L["channel_scale"])
        if fused:
            out = qdk.think_append_decode_attn(to_dev(q), to_dev(k_new), to_dev(v_new), thin_d,
                                               v_d, lens_d, idx_d, scale)
        else:
            qdk.think_append_kv(to_dev(k_new), to_dev(v_new), lens_d, idx_d, thin_d, v_d)
            out = qdk.think_decode_attn(to_dev(q), thin_d, v_d, lens_d, idx_d, scale)
        torch.cuda.synchronize()
        o_thin, o_v, o_lens = oracle.append(k_new, v_new, o_lens, idx, o_thin, o_v)
        np.testing.assert_array_equal(to_host(lens_d), o_lens)
        np.testing.assert_array_equal(to_host(thin_d).view(np.uint8), o_thin.view(np.uint8))
        np.testing.assert_array_equal(to_host(v_d).view(np.uint8), o_v.view(np.uint8))
        ref = oracle.decode(q, o_thin, o_v, o_lens, idx, scale)
        err = row_rel_err(out, ref)
        assert err.max() <= tol_for(dtype), f"step {step}: decode row error {err.max():.3e}"
        print(f"[append] seed {seed} step {step}: lens {o_lens.tolist()}, "
              f"decode row err {err.max():.2e}", flush=True)
    assert (o_lens == np.minimum(lens + 3, S)).all()


def test_random_fused_append_decode_shapes_match_the_oracle():
    """Seeded random shapes through think_append_decode_attn, two steps each:
    bf16 (matrix-core decode at head_dim 128, general decode otherwise) and
    fp32, batches of 1-70 with empty, partial and full sequences, every kind
    of keep.  Caches and lengths byte for byte against the oracle's append,
    output rows within the decode bound of the oracle's decode over them."""
    import query_driven_kv_amd as qdk
    rng = np.random.default_rng(4242)
    for case in range(32):
        dtype = "f32" if case % 4 == 3 else "bf16"
        D = 128 if (dtype == "bf16" and case % 3) else int(rng.choice([8, 64, 128, 256]))
        B = int(rng.choice([1, 1, 2, 3, 8, 64, 70]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 7]))
        while Hkv * D * (2 if dtype == "bf16" else 4) > 32768:
            Hkv //= 2
        S = int(rng.integers(1, 2000)) if B <= 8 else int(rng.integers(1, 200))
        keep = int(rng.integers(1, D + 1))
        lens = rng.integers(0, S + 1, B).astype(np.int32)
        lens[0] = S if case % 2 else 0
        print(f"[fused case {case}] {dtype} B={B} Hkv={Hkv} G={G} D={D} S={S} keep={keep}",
              flush=True)
        sd = kvsynth.storage_dtype(dtype)

        def draw(*shape):
            x = rng.standard_normal(shape).astype(np.float32)
            return kvsynth.to_bf16_bits(x) if dtype == "bf16" else x

        thin, v = draw(B, S, Hkv, keep), draw(B, S, Hkv, D)
        idx = np.sort(np.stack([np.stack([rng.choice(D, keep, replace=False)
                                          for _ in range(Hkv)]) for _ in range(B)]),
                      axis=-1).astype(np.int32)
        thin_d, v_d, lens_d, idx_d = to_dev(thin), to_dev(v), to_dev(lens), to_dev(idx)
        scale = np.float32(1.0 / np.sqrt(D))
        o_thin, o_v, o_lens = thin, v, lens
        for step in range(2):
            q, k_new, v_new = draw(B, Hkv * G, D), draw(B, Hkv, D), draw(B, Hkv, D)
            assert q.dtype == sd
            out = qdk.think_append_decode_attn(to_dev(q), to_dev(k_new), to_dev(v_new), thin_d,
                                               v_d, lens_d, idx_d, scale)
            torch.cuda.synchronize()
            o_thin, o_v, o_lens = oracle.append(k_new, v_new, o_lens, idx, o_thin, o_v)
            np.testing.assert_array_equal(to_host(lens_d), o_lens)
            np.testing.assert_array_equal(to_host(thin_d).view(np.uint8), o_thin.view(np.uint8))
            np.testing.assert_array_equal(to_host(v_d).view(np.uint8), o_v.view(np.uint8))
            ref = oracle.decode(q, o_thin, o_v, o_lens, idx, scale)
            err = row_rel_err(out, ref).max()
            assert err <= tol_for(dtype), (case, step, err)
