"""tq_decode_attention_noalloc: the decode entry point that allocates nothing
(its workspace is the library's static device scratch), through the C ABI,
against tq_decode_attention with a caller workspace and against the oracle,
on two calls in a row, the second with a smaller input (the scratch keeps the
first call's contents)."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _one_call(tq, w, layers_n):
    fmt, layers = pu.layer_groups(w)[0]
    layers = layers[:layers_n]
    starts, lens, cap, slots = pu.slots_of(w)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, layers)
    ora_caches = []
    for layer in layers:
        k, v = wl.gen_kv(w, layer)
        c, _ = pu.oracle_compress_layer(w, layer, fmt, k, v, slots, cap)
        ora_caches.append(c)
    dev = pu.upload_cache(ora_caches, fmt)
    Q = np.stack([wl.gen_q(w, layer) for layer in layers])
    n_layers, batch, hq, _ = Q.shape
    max_len = int(max(lens))
    qt = torch.from_numpy(Q).cuda().contiguous()
    st = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
    ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    ws = tq.workspace_for(tfmt, dev, batch, hq, max_len)
    ref = torch.full((n_layers, batch, hq, 128), float("nan"), device="cuda")
    got = torch.full_like(ref, float("nan"))
    tq.tq_decode_attention(tfmt, tables, dev, qt, st, ln, max_len, ref, ws)
    tq.tq_decode_attention_noalloc(tfmt, tables, dev, qt, st, ln, max_len, got)
    torch.cuda.synchronize()
    a, b = ref.cpu().numpy(), got.cpu().numpy()
    assert not np.isnan(b).any()
    # the dynamic dealing of chunks may move the last bits between two calls
    scale = max(1.0, float(np.max(np.abs(a))))
    assert float(np.max(np.abs(a - b))) <= 1e-5 * scale
    worst = 0.0
    for i, layer in enumerate(layers):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        o = attention.decode_attention(ora_caches[i], Q[i], starts, lens, pi, s, cbk, cbv)
        worst = max(worst, pu.check_outputs(b[i], o))
    return worst


def test_noalloc_decode_matches_workspace_decode_twice():
    import kv_cache_quantization_norm_amd as tq
    big = wl.reduced(wl.W5, (700, 0, 333, 1200, 64))
    small = wl.reduced(wl.W2, (300,), n_layers=2)
    _say("no-alloc decode, first call", big.name)
    e1 = _one_call(tq, big, 1)
    _say("no-alloc decode, second (smaller) call", small.name)
    e2 = _one_call(tq, small, 2)
    _say("oracle max-abs errors", f"{e1:.2e}", f"{e2:.2e}")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    import kv_cache_quantization_norm_amd as tq
    fmt = tq.make_format(128, 4, 4)
    need = tq.tq_decode_workspace_bytes(fmt, 64, 64, 8, 64, 1 << 20)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    tables = tq.Tables.create(fmt, [0])
    cache = tq.Cache.allocate(fmt, 1, 8, 32)
    cs = cache.struct()
    cs.n_layers = 64
    tb = tables.struct()
    import ctypes
    st = tq.raw_call("tq_decode_attention_noalloc", ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), 1, 64, 64,
                     1, 1, 1 << 20, 0.0, 1, None)
    assert st == tq.TQ_ERR_WORKSPACE
