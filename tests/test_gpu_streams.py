"""Calls on a side stream: the Python layer allocates outputs and workspace for
a call whose kernels run on a stream that is not the current one, and tells
the caching allocator so (record_stream).  The pruning and decode calls made
on a side stream, with the current stream busy and freshly freed blocks about,
give the same bytes as on the current stream."""
import numpy as np
import pytest
import torch

import kvsynth
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def _calls(qdk, k, v, lens, qo, q, keep, scale, stream):
    out = {}
    out["s"], out["i"], out["t"], out["thin"] = qdk.think_score_select_compact(
        k, lens, qo, keep, stream=stream)
    out["o"] = qdk.think_decode_attn(q, out["thin"], v, lens, out["i"], scale, stream=stream)
    s2, i2, _ = qdk.think_score_select(k, lens, qo, keep, stream=stream)
    out["thin2"] = qdk.think_compact_k(k, lens, i2, stream=stream)
    out["s2"] = s2
    return out


@pytest.mark.parametrize("name", ["mistral-7b-gqa-32k", "batched-ragged-16k"])
def test_side_stream_matches_current_stream(name):
    import query_driven_kv_amd as qdk
    cfg = kvsynth.CONFIGS[name]
    L = kvsynth.make_layer(cfg, 0)
    k, v, qo, lens = (to_dev(L["k_cache"]), to_dev(L["v_cache"]), to_dev(L["q_obs"]),
                      to_dev(L["seq_lens"]))
    q = to_dev(kvsynth.decode_q(cfg, 0, 0, L["channel_scale"]))
    scale = 1.0 / np.sqrt(cfg.head_dim)
    ref = _calls(qdk, k, v, lens, qo, q, cfg.keep, scale, None)
    torch.cuda.synchronize()
    ref = {key: to_host(t) for key, t in ref.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    print(f"[streams] {name}: calls on a side stream", flush=True)
    for rep in range(3):
        got = _calls(qdk, k, v, lens, qo, q, cfg.keep, scale, side)
        # the current stream allocates and writes while the side stream runs:
        # blocks the wrappers freed must not be handed out under it
        junk = [torch.full((1 << 20,), 255, dtype=torch.uint8, device=k.device)
                for _ in range(16)]
        del junk
        side.synchronize()
        for key, t in got.items():
            a, r = to_host(t), ref[key]
            if key.startswith("thin"):          # rows past a length are never written
                for b, n in enumerate(L["seq_lens"]):
                    np.testing.assert_array_equal(
                        a[b, :n].view(np.uint8), r[b, :n].view(np.uint8),
                        err_msg=f"{key} differs on the side stream, rep {rep}, b {b}")
                continue
            np.testing.assert_array_equal(a.view(np.uint8), r.view(np.uint8),
                                          err_msg=f"{key} differs on the side stream, rep {rep}")
