"""The recent-token ring's host policy (tq_tail_policy) and the flush
workspace size, on the CPU: whole 32-token blocks leave the ring, oldest
first, only for sequences of at least min_compress_tokens tokens and only as
far as keep_recent tokens stay behind."""
import numpy as np
import pytest

import kv_cache_quantization_norm_amd as tq


def _rule(p, t, min_compress, keep):
    movable = t - keep
    return (movable // 32) * 32 if p + t >= min_compress and movable >= 32 else 0


def test_policy_matches_its_rule_on_random_states():
    rs = np.random.default_rng(7)
    for _ in range(20):
        n = int(rs.integers(1, 50))
        p = rs.integers(0, 2000, n)
        t = rs.integers(0, 400, n)
        mc, keep = int(rs.integers(0, 600)), int(rs.integers(0, 80))
        got = tq.tq_tail_policy(p, t, mc, keep)
        assert list(got) == [_rule(int(a), int(b), mc, keep) for a, b in zip(p, t)]


@pytest.mark.parametrize("p,t,mc,keep,want", [
    (0, 255, 256, 16, 0),      # shorter than the trigger: everything stays fp16
    (0, 256, 256, 16, 224),    # the trigger: all but keep_recent (rounded down to blocks) moves
    (224, 47, 256, 16, 0),     # 31 movable tokens: no whole block
    (224, 48, 256, 16, 32),    # one block
    (0, 32, 0, 0, 32),         # no trigger, no keep: whole blocks as they fill
    (5000, 16, 256, 16, 0),    # the ring holds only the kept tokens
])
def test_policy_cases(p, t, mc, keep, want):
    assert int(tq.tq_tail_policy([p], [t], mc, keep)[0]) == want


def test_policy_rejects_negative_values():
    with pytest.raises(tq.TQError):
        tq.tq_tail_policy([-1], [3], 256, 16)
    with pytest.raises(tq.TQError):
        tq.tq_tail_policy([0], [3], -1, 16)
    with pytest.raises(tq.TQError):
        tq.tq_tail_policy([0], [3], 256, -2)
    assert len(tq.tq_tail_policy([], [], 256, 16)) == 0


def test_flush_workspace_bytes():
    import ctypes
    fmt = tq.make_format(128, 4, 4)
    cs = tq.tq_cache(3, 2, 1024, None, None, None, None, None, None, None, None)
    rows = 5 * 64
    plane = (3 * rows * 2 * 128 * 2 + 255) // 256 * 256
    assert tq._lib.tq_tail_flush_workspace_bytes(ctypes.byref(fmt), ctypes.byref(cs), 5, 64) == 2 * plane + 8 * rows
    assert tq._lib.tq_tail_flush_workspace_bytes(ctypes.byref(fmt), ctypes.byref(cs), 0, 64) == 0
