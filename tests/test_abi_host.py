"""The C-ABI library without a GPU: it loads, exports every symbol that
include/think.h declares, and its host-side validation returns the documented
status codes before anything is enqueued (every call below fails validation,
so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "think.h")


@pytest.fixture(scope="module")
def L():
    from query_driven_kv_amd import _lib
    return _lib


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"THINK_API\s+[\w\s\*]+?\b(think_\w+)\s*\(", text)))


def test_header_declarations_are_all_exported(L):
    names = declared_functions()
    assert len(names) == 25
    assert sorted(L.EXPORTS) == names
    so = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n


def test_only_the_abi_is_exported(L):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    ours = {ln.split()[-1] for ln in out.splitlines() if "think" in ln}
    assert ours == set(declared_functions())


def test_version_and_keep_rounding(L):
    lib = L.lib
    assert lib.think_abi_version() == 6
    assert [lib.think_keep_from_ratio(128, r) for r in (0.4, 0.6, 0.5)] == [77, 51, 64]
    assert lib.think_keep_from_ratio(16, 0.5) == 8
    assert lib.think_keep_from_ratio(128, 0.0) == 128
    assert lib.think_keep_from_ratio(128, 1.0) == 1          # clamped to one channel
    assert lib.think_keep_from_ratio(5, 0.5) == 3            # half rounds up
    assert lib.think_keep_from_ratio(0, 0.5) == -1
    assert lib.think_keep_from_ratio(128, -0.1) == -1
    assert lib.think_keep_from_ratio(128, float("nan")) == -1


def dims(L, B=1, Hq=32, Hkv=8, D=128, S=32768, dt=1):
    return L.think_dims(B, Hq, Hkv, D, S, dt)


def test_workspace_sizes(L):
    lib = L.lib
    d = dims(L)
    ws = lib.think_score_workspace_bytes(ctypes.byref(d))
    assert ws > 0 and ws % 16 == 0
    assert ws < 32768 * 8 * 128 * 2 // 10        # partials stay a small fraction of |K|
    wd = lib.think_decode_workspace_bytes(ctypes.byref(d), 64)
    assert wd > 0 and wd % 16 == 0
    assert lib.think_decode_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.think_decode_workspace_bytes(ctypes.byref(d), 129) == 0
    assert lib.think_score_workspace_bytes(ctypes.byref(dims(L, Hq=30))) == 0
    assert lib.think_score_workspace_bytes(None) == 0


FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: every call fails validation first


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30), -2),                  # Hq not a multiple of Hkv
    (dict(B=0), -2),
    (dict(S=0), -2),
    (dict(dt=7), -4),
    (dict(D=12), -5),                   # head_dim not a multiple of 8
    (dict(D=264), -5),
    (dict(Hq=136, Hkv=8), -5),          # group of 17 query heads
    (dict(Hkv=65, Hq=65, D=256), -5),   # token row above 32 KiB
    (dict(B=65536), -5),
    (dict(B=16, S=1 << 28), -5),        # more than 2^31 token rows in all
])
def test_score_rejects_bad_dims(L, kw, status):
    d = dims(L, **kw)
    rc = L.lib.think_score(ctypes.byref(d), FAKE, FAKE, FAKE, 32, FAKE, FAKE, 1 << 30, None)
    assert rc == status
    assert L.lib.think_compact_k(ctypes.byref(d), FAKE, FAKE, FAKE, 8, FAKE, None) == status
    assert L.lib.think_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE,
                                   FAKE, 1 << 30, None) == status
    assert L.lib.think_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE,
                                 None) == status
    assert L.lib.think_prefill_write_kv(ctypes.byref(d), FAKE, FAKE, 0, 16, FAKE, FAKE, FAKE,
                                        FAKE, 1 << 30, None) == status
    assert L.lib.think_score_select_k2(ctypes.byref(d), FAKE, 1 << 30, FAKE, 8, 8, FAKE, FAKE,
                                       None, None) == status
    assert L.lib.think_k2_state_bytes(ctypes.byref(d)) == 0


def test_prefill_and_k2_score_validation(L):
    lib = L.lib
    d = dims(L)
    big = 1 << 30
    need = lib.think_k2_state_bytes(ctypes.byref(d))
    assert need > 0 and need % 16 == 0
    assert lib.think_k2_state_bytes(None) == 0
    w = lib.think_prefill_write_kv
    assert w(ctypes.byref(d), None, FAKE, 0, 8, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert w(ctypes.byref(d), FAKE, FAKE, 0, 8, None, FAKE, FAKE, FAKE, big, None) == -1
    assert w(ctypes.byref(d), FAKE, FAKE, -1, 8, FAKE, FAKE, FAKE, FAKE, big, None) == -2
    assert w(ctypes.byref(d), FAKE, FAKE, 0, -8, FAKE, FAKE, FAKE, FAKE, big, None) == -2
    assert w(ctypes.byref(d), FAKE, FAKE, 0, 8, FAKE, FAKE, FAKE, None, big, None) == -6
    assert w(ctypes.byref(d), FAKE, FAKE, 0, 8, FAKE, FAKE, FAKE, FAKE, need - 16, None) == -6
    assert w(ctypes.byref(d), ctypes.c_void_p(0x100008), FAKE, 0, 8, FAKE, FAKE, FAKE, FAKE, big,
             None) == -5
    assert w(ctypes.byref(d), FAKE, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, big, None) == 0  # nothing to do
    k = lib.think_score_select_k2
    assert k(ctypes.byref(d), FAKE, big, None, 8, 8, FAKE, FAKE, None, None) == -1
    assert k(ctypes.byref(d), FAKE, big, FAKE, 8, 8, None, None, None, None) == -1
    assert k(ctypes.byref(d), FAKE, big, FAKE, 0, 8, FAKE, FAKE, None, None) == -2
    assert k(ctypes.byref(d), FAKE, big, FAKE, 8, 0, FAKE, FAKE, None, None) == -3
    assert k(ctypes.byref(d), FAKE, big, FAKE, 8, 129, None, FAKE, None, None) == -3
    assert k(ctypes.byref(d), FAKE, 16, FAKE, 8, 8, FAKE, FAKE, None, None) == -6
    assert k(ctypes.byref(d), None, big, FAKE, 8, 8, FAKE, FAKE, None, None) == -6


def test_append_validation(L):
    lib = L.lib
    d = dims(L)
    assert lib.think_append_kv(None, FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, None) == -1
    for i in range(6):                                   # each required pointer
        args = [FAKE] * 6
        args[i] = None
        k_new, v_new, lens, idx, kt, vc = args
        assert lib.think_append_kv(ctypes.byref(d), k_new, v_new, lens, idx, 8, kt, vc,
                                   None) == -1
    for keep in (0, 129):
        assert lib.think_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, keep, FAKE, FAKE,
                                   None) == -3
    odd = ctypes.c_void_p(0x100008)
    assert lib.think_append_kv(ctypes.byref(d), odd, FAKE, FAKE, FAKE, 8, FAKE, FAKE, None) == -5
    assert lib.think_append_kv(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 8, FAKE, odd, None) == -5


def test_append_decode_validation(L):
    lib = L.lib
    d = dims(L)
    big = 1 << 30
    f = lib.think_append_decode_attn
    # q, k_new, v_new, k_thin, v_cache, seq_lens, kept_idx, keep, scale, out, ws, bytes, stream
    assert f(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE, FAKE, big, None) == -1
    for i in range(7):                                   # each required pointer but the workspace
        args = [FAKE] * 7
        args[i] = None
        q, kn, vn, kt, vc, lens, idx = args
        assert f(ctypes.byref(d), q, kn, vn, kt, vc, lens, idx, 8, 0.1, FAKE, FAKE, big,
                 None) == -1, i
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, None, FAKE, big,
             None) == -1
    for keep in (0, 129):
        assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, keep, 0.1, FAKE, FAKE,
                 big, None) == -3
    odd = ctypes.c_void_p(0x100008)
    assert f(ctypes.byref(d), FAKE, odd, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE, FAKE, big,
             None) == -5
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE, FAKE, 16,
             None) == -6
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE, None, big,
             None) == -6


def test_score_select_compact_validation(L):
    lib = L.lib
    d = dims(L)
    big = 1 << 30
    f = lib.think_score_select_compact
    # k_cache, seq_lens, q_obs, W, keep, scores, kept_idx, near_tie, k_thin, ws, bytes, stream
    assert f(None, FAKE, FAKE, FAKE, 32, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    for i in (0, 1, 2, 4, 6):                            # k_cache, seq_lens, q_obs, kept_idx, k_thin
        args = [FAKE] * 7
        args[i] = None
        k, lens, qo, sc, idx, tie, kt = args
        assert f(ctypes.byref(d), k, lens, qo, 32, 8, sc, idx, tie, kt, FAKE, big, None) == -1, i
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 0, 8, FAKE, FAKE, FAKE, FAKE, FAKE, big,
             None) == -2
    for keep in (0, 129):
        assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 32, keep, FAKE, FAKE, FAKE, FAKE, FAKE, big,
                 None) == -3
    odd = ctypes.c_void_p(0x100008)
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 8, FAKE, FAKE, FAKE, odd, FAKE, big,
             None) == -5
    need = lib.think_score_compact_workspace_bytes(ctypes.byref(d), 8)
    assert need >= lib.think_score_workspace_bytes(ctypes.byref(d))
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 8, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1,
             None) == -6
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 8, FAKE, FAKE, FAKE, FAKE, None, big,
             None) == -6
    assert lib.think_score_compact_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.think_score_compact_single_read(None, 8) == -1
    assert lib.think_score_compact_single_read(ctypes.byref(d), 0) == -3
    assert lib.think_score_compact_single_read(ctypes.byref(d), 8) in (0, 1)


def test_null_keep_window_workspace_and_alignment(L):
    lib = L.lib
    d = dims(L)
    big = 1 << 30
    assert lib.think_score(None, FAKE, FAKE, FAKE, 32, FAKE, FAKE, big, None) == -1
    assert lib.think_score(ctypes.byref(d), None, FAKE, FAKE, 32, FAKE, FAKE, big, None) == -1
    assert lib.think_score(ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, FAKE, big, None) == -2
    assert lib.think_score(ctypes.byref(d), FAKE, FAKE, FAKE, 32, FAKE, FAKE, 16, None) == -6
    assert lib.think_score(ctypes.byref(d), FAKE, FAKE, FAKE, 32, FAKE, None, big, None) == -6
    assert lib.think_score(ctypes.byref(d), ctypes.c_void_p(0x100002), FAKE, FAKE, 32, FAKE, FAKE,
                           big, None) == -5
    assert lib.think_score(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x100004), 32, FAKE, FAKE,
                           big, None) == -5
    assert lib.think_score_select(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x100008), 32, 8,
                                  None, FAKE, None, FAKE, big, None) == -5
    for keep in (0, 129):
        assert lib.think_select(ctypes.byref(d), FAKE, keep, FAKE, None, None) == -3
        assert lib.think_compact_k(ctypes.byref(d), FAKE, FAKE, FAKE, keep, FAKE, None) == -3
        assert lib.think_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, keep, 0.1, FAKE,
                                     FAKE, big, None) == -3
    assert lib.think_select(ctypes.byref(d), None, 8, FAKE, None, None) == -1
    assert lib.think_select(ctypes.byref(dims(L, D=12)), FAKE, 8, FAKE, None, None) == -5
    assert lib.think_compact_k(ctypes.byref(d), FAKE, FAKE, FAKE, 8, None, None) == -1
    assert lib.think_compact_k(ctypes.byref(d), FAKE, FAKE, FAKE, 8, ctypes.c_void_p(0x100008),
                               None) == -5
    assert lib.think_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1, FAKE,
                                 FAKE, 64, None) == -6
    assert lib.think_decode_attn(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, 8, 0.1, FAKE,
                                 FAKE, big, None) == -1
    assert lib.think_decode_attn_partial(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.1,
                                         FAKE, big, None) == -3
    assert lib.think_decode_attn_partial(ctypes.byref(d), FAKE, FAKE, None, FAKE, FAKE, 8, 0.1,
                                         FAKE, big, None) == -1
    assert lib.think_decode_attn_partial(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0.1,
                                         FAKE, 16, None) == -6
    assert lib.think_decode_attn_combine(ctypes.byref(d), FAKE, 8, None, FAKE, big, None) == -1
    assert lib.think_decode_attn_combine(ctypes.byref(d), FAKE, 8, FAKE, FAKE, 16, None) == -6
    assert lib.think_decode_attn_combine(ctypes.byref(dims(L, Hq=30)), FAKE, 8, FAKE, FAKE, big,
                                         None) == -2
    assert lib.think_score_select(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 0, FAKE, FAKE, None, FAKE,
                                  big, None) == -3
    assert lib.think_score_select(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 8, None, None, None, FAKE,
                                  big, None) == -1
    assert lib.think_score_select(ctypes.byref(d), FAKE, FAKE, FAKE, 0, 8, None, FAKE, None, FAKE,
                                  big, None) == -2
    assert lib.think_score_select(ctypes.byref(d), FAKE, FAKE, FAKE, 32, 8, None, FAKE, None, FAKE,
                                  16, None) == -6


def test_score_compact_status_validation(L):
    """The give-up query checks its arguments like the call it reports on and
    never touches the device for a bad argument."""
    lib = L.lib
    d = dims(L)
    big = 1 << 30
    assert lib.think_score_compact_status(None, 32, 8, FAKE, big, None) == -1
    assert lib.think_score_compact_status(ctypes.byref(d), 0, 8, FAKE, big, None) == -2
    assert lib.think_score_compact_status(ctypes.byref(d), 32, 0, FAKE, big, None) == -3
    assert lib.think_score_compact_status(ctypes.byref(d), 32, 8, None, big, None) == -6
    assert lib.think_score_compact_status(ctypes.byref(d), 32, 8, FAKE, 16, None) == -6
    assert lib.think_score_compact_status(ctypes.byref(dims(L, Hq=30)), 32, 8, FAKE, big,
                                          None) == -2


def test_single_read_test_hook_is_per_thread(L):
    import threading
    lib = L.lib
    assert lib.think_single_read_test_give_up(1) == 0
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.think_single_read_test_give_up(0)))
    t.start()
    t.join()
    assert seen == [0]                                    # another thread: its own setting
    assert lib.think_single_read_test_give_up(0) == 1


def test_probe_stream_validation(L):
    lib = L.lib
    assert lib.think_probe_stream(None, 16, None, 0, None) == -1
    assert lib.think_probe_stream(FAKE, 16, None, 16, None) == -1
    assert lib.think_probe_stream(ctypes.c_void_p(0x100008), 16, None, 0, None) == -5
    assert lib.think_probe_stream(FAKE, 1 << 40, None, 0, None) == -5
    assert lib.think_probe_stream(None, 0, None, 0, None) == 0       # nothing to do


def test_status_strings(L):
    for code in range(-8, 1):
        assert L.lib.think_status_string(code)
    assert L.lib.think_status_string(-99) == b"unknown status"
    assert L.lib.think_last_hip_error() == 0


def test_python_layer_checks_before_calling(L):
    import torch
    import query_driven_kv_amd as qdk
    with pytest.raises(ValueError):
        qdk.think_score(torch.zeros(1, 4, 2, 8), torch.zeros(1, dtype=torch.int32),
                        torch.zeros(1, 2, 2, 8))          # CPU tensors are refused
