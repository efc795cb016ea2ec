"""GPU parity of the decode chunk passes beyond the bf16 head_dim-128 shapes:
the general kernel (fp32 at every head_dim, bf16 at head_dims other than 64
and 128) over seeded random shapes that reach each of its tile classes, and
full-size 32K-token shapes of both chunk passes, every output row against the
oracle's decode on the same bytes.

Shape classes the random draws cover (the launcher picks them from dtype,
head_dim, keep and the query heads per kv head): 32- and 64-token tiles,
16-, 8- and 4-byte and one-element key units, 4 and 16 head slots, chunks of 256 tokens
halved while the grid fits one wave of resident workgroups.  Padding rows of
K_thin and V past each length hold NaN, so a read past len_b shows up.
Three more shapes reach the merge kernel's column slices and a pairwise
merge tree whose sub-group count is not a power of two.
Bar: per row max-abs error relative to the row's max-abs, 1e-5 (fp32) and
2e-2 (bf16), as for every decode."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import row_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _qdk():
    import query_driven_kv_amd as qdk
    return qdk


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _inputs(rng, dtype, B, S, Hq, Hkv, D, keep, lens, scale_in=1.0):
    """q, K_thin, V (NaN past each length) and sorted kept indices; torch CPU
    tensors in the dtype, plus the arrays the oracle reads."""
    q = rng.standard_normal((B, Hq, D), dtype=np.float32) * scale_in
    thin = rng.standard_normal((B, S, Hkv, keep), dtype=np.float32) * scale_in
    v = rng.standard_normal((B, S, Hkv, D), dtype=np.float32)
    for b in range(B):
        thin[b, lens[b]:] = np.nan
        v[b, lens[b]:] = np.nan
    idx = np.sort(np.stack([np.stack([rng.choice(D, keep, replace=False) for _ in range(Hkv)])
                            for _ in range(B)]), axis=-1).astype(np.int32)
    if dtype == "bf16":
        tq, tt, tv = _bf16(q), _bf16(thin), _bf16(v)
        return (tq, tt, tv, idx), (_bits(tq), _bits(tt), _bits(tv))
    tq, tt, tv = torch.from_numpy(q), torch.from_numpy(thin), torch.from_numpy(v)
    return (tq, tt, tv, idx), (q, thin, v)


def _check(dtype, B, S, Hq, Hkv, D, keep, lens, rng, label, scale_in=1.0):
    qdk = _qdk()
    lens = np.asarray(lens, np.int32)
    (tq, tt, tv, idx), (oq, ot, ov) = _inputs(rng, dtype, B, S, Hq, Hkv, D, keep, lens, scale_in)
    scale = np.float32(1.0 / np.sqrt(D))
    print(f"[decode] {label}: {dtype} B={B} S={S} Hq={Hq} Hkv={Hkv} D={D} keep={keep} "
          f"lens={lens.tolist()[:4]}", flush=True)
    out = qdk.think_decode_attn(tq.cuda(), tt.cuda(), tv.cuda(), to_dev(lens), to_dev(idx),
                                float(scale))
    torch.cuda.synchronize()
    ref = oracle.decode(oq, ot, ov, lens, idx, scale)
    err = row_rel_err(out, ref)
    bar = 1e-5 if dtype == "f32" else 2e-2
    # rows of empty sequences are zero on both sides
    assert np.all(np.isfinite(err)), label
    assert err.max() <= bar, (label, float(err.max()))
    return float(err.max())


def test_general_decode_random_shapes_match_the_oracle():
    rng = np.random.default_rng(4242)
    dims_bf16 = [8, 16, 24, 32, 40, 48, 72, 96, 136, 192, 256]
    dims_f32 = [8, 16, 32, 40, 64, 96, 128, 200, 256]
    worst = {}
    for case in range(48):
        dtype = "f32" if case % 2 else "bf16"
        D = int(rng.choice(dims_f32 if dtype == "f32" else dims_bf16))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        B = int(rng.choice([1, 1, 2, 3, 6]))
        S = int(rng.integers(1, 1600 if B <= 2 else 600))
        # keep: every fourth draw a multiple of 8 (16-byte units in both
        # dtypes where the row allows), else anything up to D
        if case % 4 == 0:
            keep = int(8 * rng.integers(1, D // 8 + 1))
        else:
            keep = int(rng.integers(1, D + 1))
        lens = rng.integers(0, S + 1, B).astype(np.int32)
        lens[0] = S
        e = _check(dtype, B, S, Hkv * G, Hkv, D, keep, lens, rng, f"random{case}")
        worst[dtype] = max(worst.get(dtype, 0.0), e)
    print(f"[decode] worst row error: {worst}", flush=True)


@pytest.mark.parametrize("shape", [
    # dtype, B, S, Hq, Hkv, D, keep
    ("f32", 1, 32768, 32, 8, 128, 64),      # general kernel, 16-byte key units
    ("bf16", 1, 32768, 16, 4, 256, 128),    # general kernel, halved chunks
    ("bf16", 1, 32768, 32, 8, 64, 32),      # matrix-core kernel, head_dim 64
    ("f32", 1, 4096, 32, 32, 128, 77),      # general kernel, one-element key units
], ids=["f32-d128-32k", "bf16-d256-32k", "bf16-d64-32k", "f32-mha-4k"])
def test_full_size_decode_matches_the_oracle(shape):
    dtype, B, S, Hq, Hkv, D, keep = shape
    rng = np.random.default_rng(S + D + keep)
    _check(dtype, B, S, Hq, Hkv, D, keep, [S] * B, rng, "full-size")


@pytest.mark.parametrize("shape", [
    # dtype, B, S, Hq, Hkv, D, keep: chunk slot counts whose merge has a
    # sub-group count that is not a power of two (the pairwise tree then
    # leaves an odd sub-group over in some rounds) and records split into
    # column slices
    ("bf16", 1, 65536, 28, 7, 128, 64),     # matrix-core pass, 74 slots a head
    ("f32", 1, 25600, 8, 2, 128, 48),       # general pass, about 100 slots a head
    ("bf16", 1, 20000, 12, 3, 72, 40),      # general pass, 18 column quads in two slices
], ids=["mfma-74-slots", "general-100-slots", "general-d72-slices"])
def test_merge_tree_and_column_slices_match_the_oracle(shape):
    dtype, B, S, Hq, Hkv, D, keep = shape
    rng = np.random.default_rng(S + Hkv)
    _check(dtype, B, S, Hq, Hkv, D, keep, [S - 37], rng, "merge-shape")
