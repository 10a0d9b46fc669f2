"""The decode work split (tq_decode_split, host): every chunk of every
problem that can hold tokens is dealt to exactly one workgroup, the pieces of
a workgroup's run land in distinct partial slots below the bound, the combine's
piece count per problem matches, and the workspace holds them."""
import math
import random

import pytest

import kv_cache_quantization_norm_amd as tq

SHAPES = [
    # (n_layers, batch, n_kv_heads, n_q_heads, max_seq_len)
    (28, 1, 4, 28, 8192),     # dense 28-layer decode: aligned runs
    (1, 43, 3, 6, 1100),      # 129 problems: balanced runs crossing problems
    (1, 40, 8, 16, 200),      # 320 short problems: several groups per workgroup
    (1, 1, 8, 64, 3000),
    (1, 1, 1, 1, 1024),
    (2, 2, 3, 3, 95),
    (1, 2, 1, 40, 257),       # G = 40: 5 head groups
    (1, 1, 1, 1, 0),
    (1, 1, 8, 64, 262144),
    (3, 7, 2, 10, 31),
]


def _random_shapes(n, seed=0):
    r = random.Random(seed)
    out = []
    for _ in range(n):
        h = r.choice([1, 2, 4, 8])
        out.append((r.randint(1, 6), r.randint(1, 48), h, h * r.choice([1, 2, 7, 8, 9, 20]), r.randint(0, 20000)))
    return out


def _check(shape):
    L, B, H, HQ, T = shape
    fmt = tq.make_format(128, 4, 4)
    sp = tq.tq_decode_split(fmt, L, B, H, HQ, T)
    P, cpp, cpw, nwg, seg_max = (sp[k] for k in ("problems", "chunks_per_problem", "chunks_per_wg",
                                                  "n_workgroups", "pieces_max"))
    n_hg = math.ceil(HQ // H / 8)
    assert P == L * B * H * n_hg
    live = math.ceil(max(T, 1) / 32)
    assert cpp >= live and cpw >= 1 and 1 <= nwg <= 256
    total = P * cpp
    assert (nwg - 1) * cpw < total <= nwg * cpw
    dealt = [0] * P          # live chunks dealt per problem
    slots = set()
    for w in range(nwg):
        lo, hi = w * cpw, min((w + 1) * cpw, total)
        g0 = lo
        while g0 < hi:        # the kernel's groups of at most two pieces
            pa = g0 // cpp
            a_end = min((pa + 1) * cpp, hi)
            b_end = min(a_end + cpp, hi) if a_end < hi else a_end
            for p, first, c0, c1 in ((pa, pa * cpp, g0, a_end),) + (((pa + 1, a_end, a_end, b_end),) if b_end > a_end else ()):
                seg = w - first // cpw
                assert 0 <= seg < seg_max and (p, seg) not in slots
                slots.add((p, seg))
                rel0 = c0 - p * cpp
                dealt[p] += max(0, min(c1 - p * cpp, live) - rel0) if rel0 < live else 0
            g0 = b_end
    assert dealt == [live] * P
    for p in range(P):        # the combine reads exactly the written slots
        first = p * cpp
        nseg = (first + cpp - 1) // cpw - first // cpw + 1
        assert all((p, s) in slots for s in range(nseg)) and (p, nseg) not in slots
    # prepared queries, partials and the counters (the in-kernel merge's one
    # per problem, then the step's append count per layer)
    align = lambda x: (x + 255) // 256 * 256
    need = (align(L * B * HQ * 2 * 128 * 4) + align(L * B * HQ * seg_max * (128 + 2) * 4)
            + align((P + L) * 4))
    assert tq.tq_decode_workspace_bytes(fmt, L, B, H, HQ, T) >= need
    return sp


@pytest.mark.parametrize("shape", SHAPES + _random_shapes(60))
def test_split_deals_every_chunk_once(shape):
    _check(shape)


def test_dense_decode_split_is_aligned():
    sp = _check((28, 1, 4, 28, 8192))
    # 112 problems of 256 chunks: two runs of 128 per problem, no crossing
    assert sp["chunks_per_wg"] == 128 and sp["n_workgroups"] == 224


def test_balanced_split_when_alignment_costs_too_much():
    sp = _check((1, 43, 3, 6, 1100))
    assert sp["chunks_per_problem"] == 35 and sp["chunks_per_wg"] == 18 and sp["n_workgroups"] == 251


def test_split_rejects_bad_sizes():
    fmt = tq.make_format(128, 4, 4)
    with pytest.raises(RuntimeError):
        tq.tq_decode_split(fmt, 1, 1, 4, 6, 10)


# The ragged split the decode kernel builds for itself (batch > 1) from the
# sequence lengths: each sequence's live chunks plus padding (32 chunks, plus
# 160 (w0 - live) / w0 for a sequence shorter than the mean range w0), laid
# out layer-major, then sequence, then KV head and head group; the decode
# workgroups take equal ranges of that sequence, at least half the static
# range long.  The constants restate the kernel's (kRaggedCrossChunks,
# kContainChunks).
CROSSING, CONTAIN = 32, 160


def _ragged_pieces_max(L, lens, H, HQ, T, nd=256):
    n_hg = math.ceil(HQ // H / 8)
    HG = H * n_hg
    cpp = math.ceil(max(T, 1) / 32)
    P = L * len(lens) * HG
    wgs = min(math.ceil(P * cpp / 8), nd)
    cpw_min = max(1, math.ceil(P * cpp / wgs) // 2)
    live = [min(math.ceil(n / 32), cpp) for n in lens]
    s = sum(live)
    if L * HG * s >= P * cpp:
        return None   # no sequence is short of max_len: the static split applies
    w0 = math.ceil(L * HG * s / nd)
    n = [lv + CROSSING + (CONTAIN * (w0 - lv) // w0 if lv < w0 else 0) if lv > 0 else 0 for lv in live]
    total = L * HG * sum(n)
    cpw = max(math.ceil(total / nd), cpw_min)
    worst, first = 0, 0
    for _layer in range(L):
        for nb in n:
            for _ in range(HG):
                if nb > 0:
                    worst = max(worst, (first + nb - 1) // cpw - first // cpw + 1)
                first += nb
    return worst


def _ragged_batches(count, seed=1):
    r = random.Random(seed)
    out = []
    for _ in range(count):
        T = r.choice([64, 1000, 4096, 32768, 100000])
        B = r.choice([2, 3, 16, 40, 200, 1024])
        mode = r.choice(["uniform", "short", "one_long", "zeros"])
        if mode == "uniform":
            lens = [r.randint(0, T) for _ in range(B)]
        elif mode == "short":
            lens = [r.randint(1, max(1, T // 50)) for _ in range(B)]
        elif mode == "one_long":
            lens = [T] + [r.randint(1, 64) for _ in range(B - 1)]
        else:
            lens = [0 if r.random() < 0.7 else r.randint(1, T) for _ in range(B)]
        h = r.choice([1, 4, 8])
        out.append((r.randint(1, 3), lens, h, h * r.choice([1, 7, 8]), T))
    return out


@pytest.mark.parametrize("case", _ragged_batches(60))
def test_ragged_split_pieces_fit_the_workspace(case):
    """Whatever the length mix, no problem of the kernel's ragged split leaves
    more pieces than the workspace has partial slots: the workspace holds
    queries, counters, L x B x Hq x (most pieces) partials of d + 2 floats and
    the per-workgroup wave-merge area after them."""
    L, lens, H, HQ, T = case
    worst = _ragged_pieces_max(L, lens, H, HQ, T)
    if worst is None:
        pytest.skip("every sequence fills max_len: static split")
    fmt = tq.make_format(128, 4, 4)
    B = len(lens)
    sp = tq.tq_decode_split(fmt, L, B, H, HQ, T)
    P = sp["problems"]
    align = lambda x: (x + 255) // 256 * 256
    need = (align(L * B * HQ * 2 * 128 * 4) + align((P + L + 1) * 4) + align(L * B * HQ * worst * (128 + 2) * 4)
            + align(sp["n_workgroups"] * 8 * 8 * 128 * 4))
    assert tq.tq_decode_workspace_bytes(fmt, L, B, H, HQ, T) >= need, (worst, sp)
