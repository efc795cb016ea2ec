"""The C-ABI calls are capturable: they allocate nothing, never synchronise
and record no memset, so a whole pruning-and-decode step captured in a HIP
graph (through torch.cuda.graph) replays correctly.  The graph is replayed
several times with new inputs copied into its static buffers and eager work
and synchronisations in between, and every replay is compared bitwise with
the same calls run eagerly."""
import numpy as np
import pytest
import torch

import kvsynth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, D, S, keep, lengths
    (2, 8, 2, 128, 3000, 64, [3000, 1777]),     # chunk slots dealt by length
    (1, 32, 8, 128, 40000, 64, [39000]),        # merge in column slices
], ids=["ragged-pair", "long-sliced-merge"])
def test_pruning_and_decode_step_replays_in_a_graph(shape):
    import query_driven_kv_amd as qdk
    B, Hq, Hkv, D, S, keep, lengths = shape
    cfg = kvsynth.custom("graph", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, seq_capacity=S,
                         obs_window=8, keep=keep, dtype="bf16", lowrank=8, cfg_id=93)
    L = kvsynth.make_layer(cfg, layer=0)
    L["seq_lens"] = np.array(lengths, np.int32)
    k, v, qo = to_dev(L["k_cache"]), to_dev(L["v_cache"]), to_dev(L["q_obs"])
    lens = to_dev(L["seq_lens"])
    dims = qdk.make_dims(B, Hq, Hkv, D, S, torch.bfloat16)
    # static buffers
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    scores = torch.empty(B, Hkv, D, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, Hkv, keep, dtype=torch.int32, device="cuda")
    tie = torch.empty(B, Hkv, dtype=torch.int32, device="cuda")
    thin = torch.empty(B, S, Hkv, keep, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    ws_s = torch.empty(qdk.think_score_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(qdk.think_decode_workspace_bytes(dims, keep), dtype=torch.uint8, device="cuda")

    def step(qbuf, obuf):
        qdk.think_score_select(k, lens, qo, keep, scores=scores, kept_idx=idx, near_tie=tie,
                               workspace=ws_s)
        qdk.think_compact_k(k, lens, idx, k_thin=thin)
        qdk.think_decode_attn(qbuf, thin, v, lens, idx, D ** -0.5, out=obuf, workspace=ws_d)

    queries = [to_dev(kvsynth.decode_q(cfg, 0, s, L["channel_scale"])) for s in range(4)]
    q.copy_(queries[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm up off the capture stream
        step(q, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(q, out)
    torch.cuda.synchronize()

    ref = torch.empty_like(out)
    for rep in range(3):
        for s in (rep % 4, (rep + 1) % 4):
            q.copy_(queries[s])
            g.replay()
            got = out.clone()
            torch.cuda.synchronize()
            step(queries[s], ref)                  # eager, into its own output
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), (rep, s)
            x = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
            torch.cuda.synchronize()
            assert torch.isfinite(x)


def test_single_read_pruning_replays_in_a_graph():
    """The single-read pruning launch tags its flags with the call's value plus
    a generation word in the workspace that every launch advances, so replays
    of a captured call (frozen arguments) do not see the previous replay's
    flags.  New keys are copied into the static buffer before every replay,
    and eager calls on the same workspace run in between; every replay must
    give the eager call's bits."""
    import query_driven_kv_amd as qdk
    B, Hq, Hkv, D, S, keep = 1, 8, 2, 128, 4096, 51
    cfg = kvsynth.custom("graph-sr", batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                         seq_capacity=S, obs_window=8, keep=keep, dtype="bf16", lowrank=8,
                         cfg_id=94)
    dims = qdk.make_dims(B, Hq, Hkv, D, S, torch.bfloat16)
    assert qdk.think_score_compact_single_read(dims, keep) == 1
    layers = [kvsynth.make_layer(cfg, layer=l) for l in range(3)]
    keys = [to_dev(L["k_cache"]) for L in layers]
    k = torch.empty_like(keys[0])
    lens = to_dev(np.array([4000], np.int32))
    qo = to_dev(layers[0]["q_obs"])
    scores = torch.empty(B, Hkv, D, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, Hkv, keep, dtype=torch.int32, device="cuda")
    tie = torch.empty(B, Hkv, dtype=torch.int32, device="cuda")
    thin = torch.zeros(B, S, Hkv, keep, dtype=torch.bfloat16, device="cuda")
    ws = torch.randint(0, 256, (qdk.think_score_compact_workspace_bytes(dims, keep),),
                       dtype=torch.uint8).cuda()

    def call(kbuf, s_out, i_out, t_out, th_out):
        qdk.think_score_select_compact(kbuf, lens, qo, keep, scores=s_out, kept_idx=i_out,
                                       near_tie=t_out, k_thin=th_out, workspace=ws)

    k.copy_(keys[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(k, scores, idx, tie, thin)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(k, scores, idx, tie, thin)
    torch.cuda.synchronize()

    for rep in range(6):
        k.copy_(keys[rep % 3])
        g.replay()
        got = [t.clone() for t in (scores, idx, tie, thin)]
        torch.cuda.synchronize()
        ref = [torch.empty_like(t) for t in (scores, idx, tie, thin)]
        ref[3].zero_()
        call(keys[rep % 3], *ref)                    # eager, same workspace
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), rep
        print(f"[graph-sr] replay {rep} on layer {rep % 3}: equal to the eager call", flush=True)
