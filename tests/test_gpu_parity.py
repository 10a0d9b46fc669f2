"""GPU parity: the HIP library against the float64 oracle, through the C ABI.

Compression: codes bit-exact except decisions within 1e-6 of their threshold
(at most a 1e-5 fraction of coordinates), norms to 1e-6 relative.
Decode: the oracle's own packed cache is uploaded and decoded on the GPU;
logits within 1e-3 of each row's largest magnitude, outputs within 2e-3
max-abs.  End to end: GPU compress + GPU decode against oracle compress +
oracle decode, same output bound.
"""
import math
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import attention, quant
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import kv_cache_quantization_norm_amd  # noqa: F401  (fails loudly if libtq.so is missing)
    yield


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _torch_dtype(w):
    return {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]


CASES = {
    "w1": wl.W1,
    "w2_4L_ragged": wl.reduced(wl.W2, (1000,), n_layers=4),
    "w3_6L_asym": wl.reduced(wl.W3, (700,), n_layers=6),
    "w4_h8_t3000": wl.reduced(wl.W4, (3000,)),
    "w5_ragged5": wl.reduced(wl.W5, (100, 0, 333, 64, 1)),
    "g20_k5v1": wl.Workload("g20_k5v1", 1, 2, 40, (257,), 5, 1, "f16", 0.3, 1, 5.0),
    "g1_k2v2": wl.Workload("g1_k2v2", 2, 3, 3, (95, 31), 2, 2, "f32", 0.0, 0, 1.0),
    # 129 problems: the decode split deals balanced chunk runs that cross from
    # one problem into the next (two pieces per workgroup)
    "split_cross_b43": wl.Workload("split_cross_b43", 1, 3, 6, wl.ragged_lengths(42, 600, 1100, seed=3) + (1100,),
                                   4, 4, "bf16", 0.5, 1, 10.0),
    # 320 short problems: several groups of pieces per workgroup
    "many_short_b40": wl.Workload("many_short_b40", 1, 8, 16, wl.ragged_lengths(39, 1, 200, seed=4) + (200,),
                                  3, 2, "f32", 0.3, 0, 1.0),
    # ragged split with problems far shorter than the mean range: the short
    # sequences' problems carry the largest padding (81 chunks against ranges
    # of 23), so ranges hold them whole and some ranges hold padding only
    # (pieces without tokens)
    "pad_contain_b4": wl.Workload("pad_contain_b4", 1, 8, 64, (8000, 300, 300, 8000), 4, 4, "bf16", 0.5, 2, 10.0),
    # 8-bit keys (7 Lloyd-Max bits + QJL) with 4-bit values, the wide key path
    "k8v4_ragged": wl.Workload("k8v4_ragged", 2, 2, 14, (300, 77), 8, 4, "bf16", 0.5, 1, 10.0),
    "k8v2_f32": wl.Workload("k8v2_f32", 1, 4, 32, (129,), 8, 2, "f32", 0.0, 0, 1.0),
    # 3-bit values: a coordinate's 32 codes fill 12 bytes, codes 10 and 21 of a
    # group straddle two dwords
    "k3v3_ragged": wl.Workload("k3v3_ragged", 2, 2, 14, (300, 45, 0, 129), 3, 3, "bf16", 0.5, 1, 10.0),
    "k4v3_t1000": wl.Workload("k4v3_t1000", 1, 4, 28, (1000,), 4, 3, "bf16", 0.5, 2, 10.0),
}


def _inputs(w, layers, fmt=None, sanitize=False):
    ks, vs = [], []
    for layer in layers:
        k, v = wl.gen_kv(w, layer)
        if sanitize:
            k, v, n = pu.sanitize_near_boundary(fmt, layer, k, v)
            _say("layer", layer, "zeroed near-boundary (token, head) pairs:", n)
        ks.append(k)
        vs.append(v)
    return np.stack(ks), np.stack(vs)


def _run_group(w, fmt, layers, dev_compress=True, sanitize=False):
    """Compress a group of layers on the GPU and with the oracle."""
    import kv_cache_quantization_norm_amd as tq
    starts, lens, cap, slots = pu.slots_of(w)
    K, V = _inputs(w, layers, fmt, sanitize)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, layers)
    ora_caches, ora_details = [], []
    for i, layer in enumerate(layers):
        c, det = pu.oracle_compress_layer(w, layer, fmt, K[i], V[i], slots, cap)
        ora_caches.append(c)
        ora_details.append(det)
    dev = None
    if dev_compress:
        dev = tq.Cache.allocate(tfmt, len(layers), w.n_kv_heads, cap)
        dt = _torch_dtype(w)
        kt = torch.from_numpy(K).to("cuda", dt).contiguous()
        vt = torch.from_numpy(V).to("cuda", dt).contiguous()
        st = torch.from_numpy(slots).cuda()
        if len(w.seq_lens) == 1:
            tq.tq_compress_kv(tfmt, tables, dev, kt, vt, layer0=0, slots=None, slot0=int(starts[0]))
        else:
            tq.tq_compress_kv(tfmt, tables, dev, kt, vt, layer0=0, slots=st)
        torch.cuda.synchronize()
    return tables, dev, ora_caches, ora_details, (starts, lens, cap, slots)


@pytest.mark.parametrize("case", list(CASES))
def test_compress_parity(case):
    w = CASES[case]
    _say("compress", case)
    total = dict(coords=0, k_mismatch=0, s_mismatch=0, v_mismatch=0, tokens_alt_codes=0)
    for fmt, layers in pu.layer_groups(w):
        tables, dev, ora_caches, ora_details, (starts, lens, cap, slots) = _run_group(w, fmt, layers)
        gpu_caches = pu.download_cache(dev, fmt)
        for i, layer in enumerate(layers):
            st = pu.compare_layer(gpu_caches[i], ora_caches[i], ora_details[i], fmt, slots, layer)
            for k in total:
                total[k] += st[k]
            # slots outside the sequences stay zero
            used = np.zeros(cap, bool)
            used[slots] = True
            for name in ("k_norm", "v_norm"):
                if name in gpu_caches[i]:
                    assert np.all(gpu_caches[i][name][:, ~used] == 0)
    _say("mismatches", total)
    assert pu.mismatch_rate(total) <= pu.MAX_MISMATCH_RATE, total


def _decode_gpu(fmt, tables, dev, Q, starts, lens, want_logits=True):
    import kv_cache_quantization_norm_amd as tq
    tfmt = pu.tq_format(fmt)
    n_layers, batch, hq, _ = Q.shape
    max_len = int(max(lens)) if len(lens) else 0
    qt = torch.from_numpy(Q).cuda().contiguous()
    st = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
    ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    ws = tq.workspace_for(tfmt, dev, batch, hq, max_len)
    out = torch.full((n_layers, batch, hq, 128), float("nan"), device="cuda")
    tq.tq_decode_attention(tfmt, tables, dev, qt, st, ln, max_len, out, ws)
    logits = None
    if want_logits:
        logits = torch.full((n_layers, batch, hq, max(max_len, 1)), float("nan"), device="cuda")
        tq.tq_score(tfmt, tables, dev, qt, st, ln, max_len, logits, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (logits.cpu().numpy() if logits is not None else None)


@pytest.mark.parametrize("case", list(CASES))
def test_decode_parity_on_oracle_cache(case):
    w = CASES[case]
    _say("decode", case)
    for fmt, layers in pu.layer_groups(w):
        tables, _, ora_caches, _, (starts, lens, cap, slots) = _run_group(w, fmt, layers, dev_compress=False)
        dev = pu.upload_cache(ora_caches, fmt)
        Q = np.stack([wl.gen_q(w, layer) for layer in layers])
        out, logits = _decode_gpu(fmt, tables, dev, Q, starts, lens)
        worst_l, worst_o = 0.0, 0.0
        for i, layer in enumerate(layers):
            pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
            ref, ref_logits = attention.decode_attention(ora_caches[i], Q[i], starts, lens, pi, s, cbk, cbv,
                                                         return_logits=True)
            worst_l = max(worst_l, pu.check_logits(logits[i], ref_logits, lens, w.n_q_heads))
            worst_o = max(worst_o, pu.check_outputs(out[i], ref))
            for b, n in enumerate(lens):
                if n == 0:
                    assert np.all(out[i, b] == 0)
        _say("format", fmt, "worst logit rel", f"{worst_l:.2e}", "worst out abs", f"{worst_o:.2e}")


@pytest.mark.parametrize("case", ["w1", "w2_4L_ragged", "w3_6L_asym", "w5_ragged5", "k8v4_ragged", "k3v3_ragged",
                                  "k4v3_t1000"])
def test_end_to_end(case):
    """GPU compress + GPU decode against oracle compress + oracle decode, on
    inputs with no decision within 1e-6 of its threshold (there the output is
    unique; near-threshold behaviour is covered by test_compress_parity)."""
    w = CASES[case]
    _say("end-to-end", case)
    for fmt, layers in pu.layer_groups(w):
        tables, dev, ora_caches, ora_details, (starts, lens, cap, slots) = _run_group(w, fmt, layers, sanitize=True)
        gpu_caches = pu.download_cache(dev, fmt)
        for i, layer in enumerate(layers):
            st = pu.compare_layer(gpu_caches[i], ora_caches[i], ora_details[i], fmt, slots, layer)
            assert st["k_mismatch"] == st["v_mismatch"] == st["s_mismatch"] == 0, st
        Q = np.stack([wl.gen_q(w, layer) for layer in layers])
        out, _ = _decode_gpu(fmt, tables, dev, Q, starts, lens, want_logits=False)
        for i, layer in enumerate(layers):
            pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
            ref = attention.decode_attention(ora_caches[i], Q[i], starts, lens, pi, s, cbk, cbv)
            pu.check_outputs(out[i], ref)


@pytest.mark.parametrize("case", ["w5_ragged5", "w3_6L_asym"])
def test_staged_decode_matches_one_call(case):
    """tq_decode_prepare + tq_decode_partials + tq_decode_combine on one stream
    give what tq_decode_attention gives.  The decode kernel deals chunks to its
    waves dynamically, so two calls can round differently in the last bits:
    the results agree to a relative 1e-5 of the output scale."""
    import kv_cache_quantization_norm_amd as tq
    w = CASES[case]
    _say("staged", case)
    for fmt, layers in pu.layer_groups(w):
        tables, dev, _, _, (starts, lens, cap, slots) = _run_group(w, fmt, layers)
        tfmt = pu.tq_format(fmt)
        Q = np.stack([wl.gen_q(w, layer) for layer in layers])
        n_layers, batch, hq, _ = Q.shape
        max_len = int(max(lens))
        qt = torch.from_numpy(Q).cuda().contiguous()
        st = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
        ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
        ws = tq.workspace_for(tfmt, dev, batch, hq, max_len)
        one = torch.full((n_layers, batch, hq, 128), float("nan"), device="cuda")
        staged = torch.full_like(one, float("nan"))
        tq.tq_decode_attention(tfmt, tables, dev, qt, st, ln, max_len, one, ws)
        ws.fill_(0xFF)  # NaN everywhere: the staged calls must rewrite what they read
        tq.tq_decode_prepare(tfmt, tables, dev, qt, max_len, ws)
        tq.tq_decode_partials(tfmt, tables, dev, batch, hq, st, ln, max_len, ws)
        tq.tq_decode_combine(tfmt, tables, dev, batch, hq, max_len, staged, ws)
        torch.cuda.synchronize()
        a, b = one.cpu().numpy(), staged.cpu().numpy()
        assert not np.isnan(a).any() and not np.isnan(b).any()
        scale = max(1.0, float(np.max(np.abs(a))))
        assert float(np.max(np.abs(a - b))) <= 1e-5 * scale


def test_stream_read_probe_reads_every_element_once():
    """The bandwidth reference reads each float4 exactly once: the per-workgroup
    sums of an all-ones buffer (with a ragged tail past the unrolled loop) add up to
    its length."""
    import kv_cache_quantization_norm_amd as tq
    _say("stream read probe")
    n = (1 << 20) + 4 * 37
    data = torch.ones(n, device="cuda")
    part = torch.zeros(96, device="cuda")
    tq.tq_stream_read_probe(data, part, 96)
    torch.cuda.synchronize()
    assert float(part.double().sum()) == n


@pytest.mark.parametrize("chunk", [None, 3])
def test_degenerate_vectors_and_nan(chunk):
    """Zero keys/values compress to zero norms and contribute nothing; a NaN key
    makes its sequence's outputs NaN and leaves other sequences finite.  chunk:
    tokens per compression call (None: one call; 3: the few-token kernel)."""
    import kv_cache_quantization_norm_amd as tq
    _say("degenerate", chunk)
    w = wl.Workload("degenerate", 1, 1, 2, (40, 40), 4, 4, "f32", 0.0, 0, 1.0)
    fmt = pu.layer_format(w, 0)
    starts, lens, cap, slots = pu.slots_of(w)
    K, V = _inputs(w, [0])
    K[0, 3] = 0.0
    V[0, 5] = 0.0
    K[0, 50, 0, 7] = np.nan       # second sequence (starts at slot 64 -> token index 40..79)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, [0])
    dev = tq.Cache.allocate(tfmt, 1, 1, cap)
    kt, vt, st = torch.from_numpy(K).cuda(), torch.from_numpy(V).cuda(), torch.from_numpy(slots).cuda()
    if chunk is None:
        tq.tq_compress_kv(tfmt, tables, dev, kt, vt, slots=st)
    else:
        for i in range(0, K.shape[1], chunk):
            tq.tq_compress_kv(tfmt, tables, dev, kt[:, i:i + chunk].contiguous(), vt[:, i:i + chunk].contiguous(),
                              slots=st[i:i + chunk].contiguous())
    torch.cuda.synchronize()
    g = pu.download_cache(dev, fmt)[0]
    s3 = slots[3]
    assert g["k_norm"][0, s3] == 0 and g["k_rnorm"][0, s3] == 0
    assert np.all(quant.unpack_bits(g["k_sign"][0, s3:s3 + 1], 1, 128) == 1)
    assert np.all(quant.unpack_bits(g["k_idx"][0, s3:s3 + 1], 3, 128) == 4)
    assert g["v_norm"][0, slots[5]] == 0
    s50 = slots[50]
    assert np.isnan(g["k_norm"][0, s50]) and np.isnan(g["k_rnorm"][0, s50])
    assert np.all(quant.unpack_bits(g["k_idx"][0, s50:s50 + 1], 3, 128) == 0)
    Q = wl.gen_q(w, 0)[None]
    out, _ = _decode_gpu(fmt, tables, dev, Q, starts, lens, want_logits=False)
    assert np.all(np.isfinite(out[0, 0])) and np.all(np.isnan(out[0, 1]))
    # matches the oracle on the finite sequence
    c, _ = pu.oracle_compress_layer(w, 0, fmt, K[0], V[0], slots, cap)
    pi, s, cbk, cbv = pu.oracle_tables(fmt, 0)
    ref = attention.decode_attention(c, Q[0][:1], starts[:1], lens[:1], pi, s, cbk, cbv)
    pu.check_outputs(out[0, :1], ref)


@pytest.mark.parametrize("k_bits,v_bits,dtype", [(4, 2, "bf16"), (3, 4, "f32"), (5, 1, "f16"), (2, 0, "f32"),
                                                 (8, 4, "bf16"), (4, 3, "bf16")])
def test_overwrite_slot_and_append(k_bits, v_bits, dtype):
    """Re-compressing into used slots replaces their records (value codes are
    rewritten inside shared 32-slot groups), one token at a time."""
    import kv_cache_quantization_norm_amd as tq
    _say("append", k_bits, v_bits, dtype)
    w = wl.Workload("append", 2, 2, 4, (70,), k_bits, v_bits, dtype, 0.5, 1, 10.0)
    fmt = pu.layer_format(w, 0)
    starts, lens, cap, slots = pu.slots_of(w)
    K, V = _inputs(w, [0, 1])
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, [0, 1])
    dev = tq.Cache.allocate(tfmt, 2, 2, cap)
    dt = _torch_dtype(w)
    # first fill with garbage (shifted tokens), then append the real tokens one by one
    kt = torch.from_numpy(np.roll(K, 3, axis=1)).to("cuda", dt).contiguous()
    vt = torch.from_numpy(np.roll(V, 5, axis=1)).to("cuda", dt).contiguous()
    tq.tq_compress_kv(tfmt, tables, dev, kt, vt, slot0=0)
    kr = torch.from_numpy(K).to("cuda", dt)
    vr = torch.from_numpy(V).to("cuda", dt)
    for i in range(70):
        tq.tq_compress_kv(tfmt, tables, dev, kr[:, i:i + 1].contiguous(), vr[:, i:i + 1].contiguous(), slot0=i)
    torch.cuda.synchronize()
    _say("appends done")
    gpu = pu.download_cache(dev, fmt)
    for layer in (0, 1):
        c, det = pu.oracle_compress_layer(w, layer, fmt, K[layer], V[layer], slots, cap)
        pu.compare_layer(gpu[layer], c, det, fmt, slots, layer)


@pytest.mark.parametrize("k_bits,v_bits,dtype,n_new", [(4, 4, "bf16", 1), (3, 2, "f32", 3), (0, 4, "bf16", 1),
                                                         (5, 1, "f16", 20), (3, 3, "bf16", 2)])
def test_append_prepare_matches_separate_calls(k_bits, v_bits, dtype, n_new):
    """tq_append_prepare leaves the same cache records and workspace, bit for
    bit, as tq_compress_kv followed by tq_decode_prepare (one kernel for a
    few tokens, the two calls for 16 or more)."""
    import kv_cache_quantization_norm_amd as tq
    _say("append_prepare", k_bits, v_bits, dtype, n_new)
    L, H, HQ, T = 3, 2, 14, 96
    tfmt = tq.make_format(128, k_bits, v_bits)
    tables = tq.Tables.create(tfmt, list(range(L)))
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    g = torch.Generator().manual_seed(11)
    K = torch.randn(L, T, H, 128, generator=g).to("cuda", tdt)
    V = torch.randn(L, T, H, 128, generator=g).to("cuda", tdt)
    kn = torch.randn(L, n_new, H, 128, generator=g).to("cuda", tdt)
    vn = torch.randn(L, n_new, H, 128, generator=g).to("cuda", tdt)
    Q = torch.randn(L, 2, HQ, 128, generator=g).cuda()
    base = tq.Cache.allocate(tfmt, L, H, T)
    tq.tq_compress_kv(tfmt, tables, base, K, V, slot0=0)
    copies = [tq.Cache(tfmt, L, H, T, {k: (None if t is None else t.clone()) for k, t in base.planes.items()})
              for _ in range(2)]
    ws = [tq.workspace_for(tfmt, base, 2, HQ, T) for _ in range(2)]
    for w in ws:
        w.zero_()
    slot0 = 40
    tq.tq_compress_kv(tfmt, tables, copies[0], kn, vn, slot0=slot0)
    tq.tq_decode_prepare(tfmt, tables, copies[0], Q, T, ws[0])
    tq.tq_append_prepare(tfmt, tables, copies[1], kn, vn, Q, T, ws[1], slot0=slot0)
    torch.cuda.synchronize()
    for name, t0 in copies[0].planes.items():
        if t0 is None:
            continue
        assert torch.equal(t0, copies[1].planes[name]), name
    assert torch.equal(ws[0], ws[1])


@pytest.mark.parametrize("k_bits,v_bits,HQ", [(4, 4, 14), (3, 2, 14), (0, 4, 14), (4, 4, 20), (8, 0, 16)])
def test_decode_with_fp16_tail(k_bits, v_bits, HQ):
    """Decode over a packed cache plus an fp16 tail of recent tokens (one
    softmax over both parts) against the oracle on the GPU's own caches, for
    ragged packed and tail lengths including empty parts."""
    import kv_cache_quantization_norm_amd as tq
    _say("tail", k_bits, v_bits, HQ)
    L, H = 2, 2
    lens, tlens = [300, 0, 97, 64], [40, 12, 0, 33]
    starts = [0, 320, 320, 448]
    tstarts = [0, 64, 128, 128]
    cap, tcap = 512, 192
    fmt = quant.Format(128, k_bits, v_bits)
    fmt16 = quant.Format(128, 0, 0)
    tfmt, tfmt16 = pu.tq_format(fmt), pu.tq_format(fmt16)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(21)
    dev = tq.Cache.allocate(tfmt, L, H, cap)
    tail = tq.Cache.allocate(tfmt16, L, H, tcap)
    for b in range(4):
        if lens[b]:
            k = torch.randn(L, lens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
            v = torch.randn(L, lens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
            tq.tq_compress_kv(tfmt, tables, dev, k, v, slot0=starts[b])
        if tlens[b]:
            k = torch.randn(L, tlens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
            v = torch.randn(L, tlens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
            tq.tq_compress_kv(tfmt16, tables, tail, k, v, slot0=tstarts[b])
    Q = torch.randn(L, 4, HQ, 128, generator=g).cuda()
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    tst = torch.tensor(tstarts, dtype=torch.int64, device="cuda")
    tln = torch.tensor(tlens, dtype=torch.int32, device="cuda")
    ws = tq.tail_workspace_for(tfmt, dev, 4, HQ, max(lens), max(tlens))
    out = torch.full((L, 4, HQ, 128), float("nan"), device="cuda")
    tq.tq_decode_attention_tail(tfmt, tables, dev, tail, Q, st, ln, max(lens), tst, tln, max(tlens), out, ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ora, ora_t = pu.download_cache(dev, fmt), pu.download_cache(tail, fmt16)
    qn = Q.cpu().numpy()
    worst = 0.0
    for layer in range(L):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        ref = attention.decode_attention_with_tail(ora[layer], ora_t[layer], qn[layer], starts, lens, tstarts, tlens,
                                                   pi, s, cbk, cbv)
        worst = max(worst, pu.check_outputs(out[layer], ref))
    _say("tail worst out abs", f"{worst:.2e}")
    # an empty tail gives tq_decode_attention's result (to the last bits that
    # the dynamic dealing of chunks may move)
    zero = torch.zeros(4, dtype=torch.int32, device="cuda")
    out2 = torch.empty(L, 4, HQ, 128, device="cuda")
    tq.tq_decode_attention_tail(tfmt, tables, dev, tail, Q, st, ln, max(lens), tst, zero, 0, out2, ws)
    ref2 = torch.empty_like(out2)
    tq.tq_decode_attention(tfmt, tables, dev, Q, st, ln, max(lens), ref2, tq.workspace_for(tfmt, dev, 4, HQ, max(lens)))
    torch.cuda.synchronize()
    assert float((out2 - ref2).abs().max()) <= 1e-5 * max(1.0, float(ref2.abs().max()))


@pytest.mark.parametrize("k_bits,v_bits,hq,lens", [(4, 4, 28, (300, 45, 0, 129)), (3, 0, 8, (70, 200)),
                                                     (5, 1, 40, (257, 31))])
def test_decode_steps_append_prepare_attend(k_bits, v_bits, hq, lens):
    """The decode step as two launches: tq_append_prepare (each sequence's new
    token into the packed cache, and the prepared queries), then
    tq_decode_attend (the pieces merged inside the decode kernel by the last
    workgroup of each problem).  The workspace starts as all-ones bytes (the
    preparation zeroes the piece counters); every step is checked against the
    oracle on the GPU's cache, and a second tq_decode_attend on the same
    prepared workspace (counters left at zero by the first) agrees with the
    first.  An empty sequence stays empty (its new token's slot is -1)."""
    import kv_cache_quantization_norm_amd as tq
    _say("append_prepare + attend", k_bits, v_bits, hq, lens)
    L, H, steps, stride = 2, 4, 3, 320
    B = len(lens)
    fmt = quant.Format(128, k_bits, v_bits)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(41)
    starts = [b * stride for b in range(B)]
    dev = tq.Cache.allocate(tfmt, L, H, B * stride)
    for b, n in enumerate(lens):
        if n:
            k = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
            v = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
            tq.tq_compress_kv(tfmt, tables, dev, k, v, slot0=starts[b])
    max_len = max(lens) + steps
    ws = tq.workspace_for(tfmt, dev, B, hq, max_len)
    ws.fill_(0xFF)
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    cur = list(lens)
    worst = 0.0
    for step in range(steps):
        slots = torch.tensor([starts[b] + cur[b] if cur[b] else -1 for b in range(B)], dtype=torch.int64,
                             device="cuda")
        cur = [n + 1 if n else 0 for n in cur]
        kn = torch.randn(L, B, H, 128, generator=g).to("cuda", torch.bfloat16)
        vn = torch.randn(L, B, H, 128, generator=g).to("cuda", torch.bfloat16)
        Q = torch.randn(L, B, hq, 128, generator=g).cuda()
        ln = torch.tensor(cur, dtype=torch.int32, device="cuda")
        out = torch.full((L, B, hq, 128), float("nan"), device="cuda")
        out2 = torch.full_like(out, float("nan"))
        tq.tq_append_prepare(tfmt, tables, dev, kn, vn, Q, max_len, ws, slots=slots)
        tq.tq_decode_attend(tfmt, tables, dev, B, hq, st, ln, max_len, out, ws)
        tq.tq_decode_attend(tfmt, tables, dev, B, hq, st, ln, max_len, out2, ws)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        ora = pu.download_cache(dev, fmt)
        qn = Q.cpu().numpy()
        for layer in range(L):
            pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
            ref = attention.decode_attention(ora[layer], qn[layer], starts, cur, pi, s, cbk, cbv)
            worst = max(worst, pu.check_outputs(o[layer], ref))
            for b, n in enumerate(cur):
                if n == 0:
                    assert np.all(o[layer, b] == 0)
        assert float((out2 - out).abs().max()) <= 1e-5 * max(1.0, float(out.abs().max()))
    _say("worst out abs", f"{worst:.2e}")


@pytest.mark.parametrize("mode,k_bits,v_bits,hq,lens,n_new,layer0", [
    ("slots", 4, 4, 28, (300, 45, 0, 129), 1, 0),
    ("slots", 3, 0, 8, (70, 200), 1, 0),
    ("slot0", 5, 1, 40, (31,), 1, 0),
    ("slot0", 2, 2, 12, (5,), 3, 0),
    ("slot0", 0, 4, 16, (100,), 2, 1),
    ("slots", 8, 4, 28, (300, 45, 0, 129), 1, 0),
    ("slot0", 4, 4, 28, (100,), 20, 0),   # 20 tokens: 10 append workgroups per layer, inside the decode launch
    ("slots", 4, 4, 16, (60, 33, 1, 0, 7, 300, 95, 64, 2, 18, 250, 77, 3, 40, 121, 9), 1, 0),   # 16 sequences
    ("slot0", 3, 2, 8, (100,), 40, 0),    # 40 appended workgroups: bulk compression, then the decode
    ("slots", 3, 3, 28, (300, 45, 0, 129), 1, 0),   # 3-bit values
    # listed slots inside the sequences: each sequence's middle token rewritten,
    # and sequence 0's first token too (its waits span several chunks)
    ("slots_mid", 4, 4, 28, (300, 45, 0, 129), 1, 0),
])
def test_decode_step_append_inside_decode_launch(mode, k_bits, v_bits, hq, lens, n_new, layer0):
    """tq_decode_step: the new tokens are compressed by the decode launch's
    first workgroups while the others attend, each decode wave waiting for its
    layer's append before it reads a chunk that may hold a new token.  Every
    step is checked against the oracle on the GPU's cache (which then holds the
    new tokens).  Cases: one token per sequence through a slots array (any
    slot may change), consecutive slots from slot0 (new tokens in the first
    chunk of a 5-token sequence, or crossing into a new chunk), fp16 keys or
    values, an append to layer 1 only of a 2-layer cache, and tokens rewritten
    inside the sequences (the middle one of each, and the first of sequence 0)."""
    import kv_cache_quantization_norm_amd as tq
    _say("decode step", mode, k_bits, v_bits, hq, lens, n_new, layer0)
    L, H, steps, stride = 2, 4, 3, 320
    B = len(lens)
    fmt = quant.Format(128, k_bits, v_bits)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(43)
    starts = [b * stride for b in range(B)]
    dev = tq.Cache.allocate(tfmt, L, H, B * stride)
    for b, n in enumerate(lens):
        if n:
            k = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
            v = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
            tq.tq_compress_kv(tfmt, tables, dev, k, v, slot0=starts[b])
    max_len = max(lens) + steps * n_new
    ws = tq.workspace_for(tfmt, dev, B, hq, max_len)
    ws.fill_(0xFF)
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    cur = list(lens)
    n_app_layers = L - layer0
    worst = 0.0
    for step in range(steps):
        Q = torch.randn(L, B, hq, 128, generator=g).cuda()
        if mode == "slots_mid":
            lst = [starts[b] + cur[b] // 2 if cur[b] else -1 for b in range(B)] + [starts[0] if cur[0] else -1]
            slots = torch.tensor(lst, dtype=torch.int64, device="cuda")
            kn = torch.randn(n_app_layers, len(lst), H, 128, generator=g).to("cuda", torch.bfloat16)
            vn = torch.randn(n_app_layers, len(lst), H, 128, generator=g).to("cuda", torch.bfloat16)
            extra = dict(slots=slots)
        elif mode == "slots":
            slots = torch.tensor([starts[b] + cur[b] if cur[b] else -1 for b in range(B)], dtype=torch.int64,
                                 device="cuda")
            kn = torch.randn(n_app_layers, B, H, 128, generator=g).to("cuda", torch.bfloat16)
            vn = torch.randn(n_app_layers, B, H, 128, generator=g).to("cuda", torch.bfloat16)
            extra = dict(slots=slots)
            cur = [n + 1 if n else 0 for n in cur]
        else:
            kn = torch.randn(n_app_layers, n_new, H, 128, generator=g).to("cuda", torch.bfloat16)
            vn = torch.randn(n_app_layers, n_new, H, 128, generator=g).to("cuda", torch.bfloat16)
            extra = dict(slot0=starts[0] + cur[0])
            cur = [cur[0] + n_new]
        ln = torch.tensor(cur, dtype=torch.int32, device="cuda")
        out = torch.full((L, B, hq, 128), float("nan"), device="cuda")
        tq.tq_decode_step(tfmt, tables, dev, kn, vn, Q, st, ln, max_len, out, ws, layer0=layer0, **extra)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        ora = pu.download_cache(dev, fmt)
        qn = Q.cpu().numpy()
        for layer in range(L):
            pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
            # (layers below layer0 get no new tokens: their new slots keep the
            # zero records of the allocation, read alike by both sides)
            ref = attention.decode_attention(ora[layer], qn[layer], starts, cur, pi, s, cbk, cbv)
            worst = max(worst, pu.check_outputs(o[layer], ref))
    _say("worst out abs", f"{worst:.2e}")


@pytest.mark.parametrize("formats,hq,lens,mode", [
    (((0, 4, 3), (0, 0, 2)), 28, (700,), "slot0"),                   # fp16 keys / 4-bit values beside fp16 layers
    (((4, 4, 2), (0, 0, 2)), 16, (300, 45, 0, 129), "slots"),        # ragged batch, packed keys
    (((3, 2, 1), (0, 0, 1)), 8, (100,), "slot0"),                     # one layer each
    (((3, 2, 2), (4, 4, 1)), 8, (70, 200), "slots"),                  # second part not fp16: one call per part
    (((0, 4, 1), (0, 0, 1), (4, 4, 1)), 8, (90,), "slot0"),           # three parts: one call per part
])
def test_decode_step_parts(formats, hq, lens, mode):
    """tq_decode_step_parts: a model whose layers use different formats, one
    cache per format sharing the batch and the new tokens' slots.  Two parts
    whose second is fp16 / fp16 run both appends and decodes in one launch;
    other layouts make one tq_decode_step per part.  Every step's outputs are
    checked against the oracle on the GPU's caches (which then hold the new
    tokens), and tq_decode_attend_parts on queries prepared per part likewise."""
    import kv_cache_quantization_norm_amd as tq
    _say("decode step parts", formats, hq, lens, mode)
    H, steps, stride = 4, 2, 1024
    B = len(lens)
    g = torch.Generator().manual_seed(47)
    starts = [b * stride for b in range(B)]
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    parts, fmts = [], []
    max_len = max(lens) + steps
    for kb, vb, L in formats:
        fmt = quant.Format(128, kb, vb)
        tfmt = pu.tq_format(fmt)
        tables = tq.Tables.create(tfmt, list(range(L)))
        dev = tq.Cache.allocate(tfmt, L, H, B * stride)
        for b, n in enumerate(lens):
            if n:
                k = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
                v = torch.randn(L, n, H, 128, generator=g).to("cuda", torch.bfloat16)
                tq.tq_compress_kv(tfmt, tables, dev, k, v, slot0=starts[b])
        ws = tq.workspace_for(tfmt, dev, B, hq, max_len)
        ws.fill_(0xFF)
        parts.append(tq.StepPart(tfmt, tables, dev, None, None, None, None, ws))
        fmts.append(fmt)
    cur = list(lens)
    worst = 0.0

    def check(outs, Qs):
        nonlocal worst
        for fmt, part, o, qn in zip(fmts, parts, outs, Qs):
            ora = pu.download_cache(part.cache, fmt)
            for layer in range(part.cache.n_layers):
                pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
                ref = attention.decode_attention(ora[layer], qn[layer], starts, cur, pi, s, cbk, cbv)
                worst = max(worst, pu.check_outputs(o[layer], ref))

    for step in range(steps):
        if mode == "slots":
            slots = torch.tensor([starts[b] + cur[b] if cur[b] else -1 for b in range(B)], dtype=torch.int64,
                                 device="cuda")
            extra = dict(slots=slots)
            n_new = B
            cur = [n + 1 if n else 0 for n in cur]
        else:
            extra = dict(slot0=starts[0] + cur[0])
            n_new = 1
            cur = [cur[0] + 1]
        Qs = []
        for part in parts:
            L = part.cache.n_layers
            part.k = torch.randn(L, n_new, H, 128, generator=g).to("cuda", torch.bfloat16)
            part.v = torch.randn(L, n_new, H, 128, generator=g).to("cuda", torch.bfloat16)
            part.q = torch.randn(L, B, hq, 128, generator=g).cuda()
            part.out = torch.full((L, B, hq, 128), float("nan"), device="cuda")
            Qs.append(part.q.cpu().numpy())
        ln = torch.tensor(cur, dtype=torch.int32, device="cuda")
        tq.tq_decode_step_parts(parts, st, ln, max_len, **extra)
        torch.cuda.synchronize()
        check([part.out.cpu().numpy() for part in parts], Qs)
    # the decode alone, on queries prepared per part
    for part in parts:
        tq.tq_decode_prepare(part.fmt, part.tables, part.cache, part.q, max_len, part.workspace)
        part.out = torch.full_like(part.out, float("nan"))
    tq.tq_decode_attend_parts(parts, st, ln, max_len)
    torch.cuda.synchronize()
    check([part.out.cpu().numpy() for part in parts], Qs)
    _say("worst out abs", f"{worst:.2e}")


def test_decode_step_append_wait_give_up_is_reported():
    """The decode waves' wait for the step's append is bounded; when it ends
    unmet the wave records it and tq_decode_step_check reports it.  The host
    makes the wait unmeetable (test hook: more append workgroups waited for
    than launched, 16 polls), so the waves give up and every kernel still
    exits normally; the flag is set for that call, and the next call (normal
    wait) clears it and matches the oracle."""
    import kv_cache_quantization_norm_amd as tq
    _say("append wait give-up")
    L, H, HQ, T = 2, 4, 16, 300
    fmt = quant.Format(128, 4, 4)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(47)
    dev = tq.Cache.allocate(tfmt, L, H, 320)
    k = torch.randn(L, T, H, 128, generator=g).to("cuda", torch.bfloat16)
    v = torch.randn(L, T, H, 128, generator=g).to("cuda", torch.bfloat16)
    tq.tq_compress_kv(tfmt, tables, dev, k[:, :T - 1].contiguous(), v[:, :T - 1].contiguous(), slot0=0)
    Q = torch.randn(L, 1, HQ, 128, generator=g).cuda()
    st = torch.zeros(1, dtype=torch.int64, device="cuda")
    ln = torch.full((1,), T, dtype=torch.int32, device="cuda")
    ws = tq.workspace_for(tfmt, dev, 1, HQ, T)
    out = torch.empty(L, 1, HQ, 128, device="cuda")
    kn, vn = k[:, T - 1:].contiguous(), v[:, T - 1:].contiguous()
    try:
        tq.tq_set_append_wait(16, 1000)
        tq.tq_decode_step(tfmt, tables, dev, kn, vn, Q, st, ln, T, out, ws, slot0=T - 1)
        with pytest.raises(tq.TQError) as e:
            tq.tq_decode_step_check(tfmt, dev, 1, HQ, T, ws)
        assert e.value.status == tq.TQ_ERR_APPEND_TIMEOUT
    finally:
        tq.tq_set_append_wait()
    tq.tq_decode_step(tfmt, tables, dev, kn, vn, Q, st, ln, T, out, ws, slot0=T - 1)
    tq.tq_decode_step_check(tfmt, dev, 1, HQ, T, ws)
    o = out.cpu().numpy()
    ora = pu.download_cache(dev, fmt)
    for layer in range(L):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        ref = attention.decode_attention(ora[layer], Q[layer].cpu().numpy(), [0], [T], pi, s, cbk, cbv)
        pu.check_outputs(o[layer], ref)


def test_serving_loop_with_fp16_tail_and_trigger():
    """The recent-token pattern of the pages, step by step: a compressed
    prefill; each decode step appends its token to an fp16 tail; once the
    tail holds `trigger` tokens they are compressed into the packed cache
    (from their fp16 values) and the tail is cleared.  At checkpoints the
    decode output over packed cache + tail is checked against the oracle on
    the GPU's caches; at the end the moved tokens' records are checked against
    the oracle's compression of the same fp16 values."""
    import kv_cache_quantization_norm_amd as tq
    _say("serving loop")
    L, H, HQ, P0, steps, trigger = 2, 2, 14, 200, 150, 64
    fmt, fmt16 = quant.Format(128, 4, 4), quant.Format(128, 0, 0)
    tfmt, tfmt16 = pu.tq_format(fmt), pu.tq_format(fmt16)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(31)
    K = torch.randn(L, P0 + steps, H, 128, generator=g).to("cuda", torch.float16)
    V = torch.randn(L, P0 + steps, H, 128, generator=g).to("cuda", torch.float16)
    Q = torch.randn(L, 1, HQ, 128, generator=g).cuda()
    packed = tq.Cache.allocate(tfmt, L, H, 512)
    tail = tq.Cache.allocate(tfmt16, L, H, trigger)
    tq.tq_compress_kv(tfmt, tables, packed, K[:, :P0].contiguous(), V[:, :P0].contiguous(), slot0=0)
    n_packed, n_tail = P0, 0
    zero64 = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = tq.tail_workspace_for(tfmt, packed, 1, HQ, 512, trigger)
    out = torch.empty(L, 1, HQ, 128, device="cuda")
    checks = 0
    for step in range(steps):
        tok = P0 + step
        tq.tq_compress_kv(tfmt16, tables, tail, K[:, tok:tok + 1].contiguous(), V[:, tok:tok + 1].contiguous(),
                          slot0=n_tail)
        n_tail += 1
        if n_tail == trigger:
            lo = tok + 1 - trigger
            tq.tq_compress_kv(tfmt, tables, packed, K[:, lo:tok + 1].contiguous(), V[:, lo:tok + 1].contiguous(),
                              slot0=n_packed)
            n_packed += trigger
            n_tail = 0
        if step % 37 == 0 or step == steps - 1:
            ln = torch.full((1,), n_packed, dtype=torch.int32, device="cuda")
            tln = torch.full((1,), n_tail, dtype=torch.int32, device="cuda")
            tq.tq_decode_attention_tail(tfmt, tables, packed, tail, Q, zero64, ln, 512, zero64, tln, trigger, out, ws)
            torch.cuda.synchronize()
            ora, ora_t = pu.download_cache(packed, fmt), pu.download_cache(tail, fmt16)
            for layer in range(L):
                pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
                ref = attention.decode_attention_with_tail(ora[layer], ora_t[layer], Q[layer].cpu().numpy(), [0],
                                                           [n_packed], [0], [n_tail], pi, s, cbk, cbv)
                pu.check_outputs(out[layer].cpu().numpy(), ref)
            checks += 1
    assert n_packed == P0 + 2 * trigger and checks >= 4
    # the moved tokens against the oracle's compression of the same fp16 values
    moved = np.arange(P0, n_packed)
    gpu = pu.download_cache(packed, fmt)
    kh, vh = K.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64)
    for layer in range(L):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        ora = quant.empty_cache(fmt, H, 512)
        det = quant.compress_into(ora, kh[layer, P0:n_packed], vh[layer, P0:n_packed], moved, pi, s, cbk, cbv)
        det["keys"] = kh[layer, P0:n_packed]
        pu.compare_layer(gpu[layer], ora, det, fmt, moved, layer)


def test_multi_query_scoring_as_query_rows():
    """Several queries per sequence (a prefill chunk scored against the cache)
    passed as n_q_heads * n_q query rows: logits and outputs against the
    oracle (which maps rows to KV heads the same way), and each query row
    equal to a single-query call (to the last bits of the dynamic dealing)."""
    import kv_cache_quantization_norm_amd as tq
    _say("multi-query")
    L, H, HQ, NQ = 2, 2, 14, 5
    lens, starts, cap = [300, 97], [0, 320], 448
    fmt = quant.Format(128, 4, 2)
    tfmt = pu.tq_format(fmt)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(41)
    dev = tq.Cache.allocate(tfmt, L, H, cap)
    for b in range(2):
        k = torch.randn(L, lens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
        v = torch.randn(L, lens[b], H, 128, generator=g).to("cuda", torch.bfloat16)
        tq.tq_compress_kv(tfmt, tables, dev, k, v, slot0=starts[b])
    Q5 = torch.randn(L, 2, HQ, NQ, 128, generator=g).cuda()
    Qr = Q5.reshape(L, 2, HQ * NQ, 128)
    st = torch.tensor(starts, dtype=torch.int64, device="cuda")
    ln = torch.tensor(lens, dtype=torch.int32, device="cuda")
    T = max(lens)
    ws = tq.workspace_for(tfmt, dev, 2, HQ * NQ, T)
    out = torch.empty(L, 2, HQ * NQ, 128, device="cuda")
    logits = torch.full((L, 2, HQ * NQ, T), float("nan"), device="cuda")
    tq.tq_decode_attention(tfmt, tables, dev, Qr, st, ln, T, out, ws)
    tq.tq_score(tfmt, tables, dev, Qr, st, ln, T, logits, ws)
    torch.cuda.synchronize()
    ora = pu.download_cache(dev, fmt)
    qn, on, lg = Qr.cpu().numpy(), out.cpu().numpy(), logits.cpu().numpy()
    for layer in range(L):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        ref, ref_logits = attention.decode_attention(ora[layer], qn[layer], starts, lens, pi, s, cbk, cbv,
                                                     return_logits=True)
        pu.check_logits(lg[layer], ref_logits, lens, HQ * NQ)
        pu.check_outputs(on[layer], ref)
    ws1 = tq.workspace_for(tfmt, dev, 2, HQ, T)
    o1 = torch.empty(L, 2, HQ, 128, device="cuda")
    for j in range(NQ):
        tq.tq_decode_attention(tfmt, tables, dev, Q5[:, :, :, j].contiguous(), st, ln, T, o1, ws1)
        torch.cuda.synchronize()
        oj = out.reshape(L, 2, HQ, NQ, 128)[:, :, :, j]
        assert float((oj - o1).abs().max()) <= 1e-5 * max(1.0, float(o1.abs().max()))


def test_background_recompression_on_second_stream():
    """Bulk compression on a second stream, concurrent with decode calls on
    the main stream: the compressed records are bit-identical to a compression
    made alone, and the decode outputs agree with a decode made alone (to the
    last bits that the dynamic dealing of chunks may move)."""
    import kv_cache_quantization_norm_amd as tq
    _say("background recompression")
    L, H, HQ, T, P = 2, 2, 14, 320, 600
    tfmt = tq.make_format(128, 4, 4)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(5)
    K = torch.randn(L, T, H, 128, generator=g).to("cuda", torch.bfloat16)
    V = torch.randn(L, T, H, 128, generator=g).to("cuda", torch.bfloat16)
    K2 = torch.randn(L, P, H, 128, generator=g).to("cuda", torch.bfloat16)
    V2 = torch.randn(L, P, H, 128, generator=g).to("cuda", torch.bfloat16)
    Q = torch.randn(L, 1, HQ, 128, generator=g).cuda()
    cache = tq.Cache.allocate(tfmt, L, H, T)
    tq.tq_compress_kv(tfmt, tables, cache, K, V, slot0=0)
    st = torch.zeros(1, dtype=torch.int64, device="cuda")
    ln = torch.full((1,), T, dtype=torch.int32, device="cuda")
    ws = tq.workspace_for(tfmt, cache, 1, HQ, T)
    ref_out = torch.empty(L, 1, HQ, 128, device="cuda")
    tq.tq_decode_attention(tfmt, tables, cache, Q, st, ln, T, ref_out, ws)
    ref_target = tq.Cache.allocate(tfmt, L, H, P + 32 - P % 32)
    tq.tq_compress_kv(tfmt, tables, ref_target, K2, V2, slot0=0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    target = tq.Cache.allocate(tfmt, L, H, P + 32 - P % 32)
    outs = [torch.empty_like(ref_out) for _ in range(4)]
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    # the bulk kernel on the CUs that the decode kernel leaves free
    free = max(1, 256 - tq.tq_decode_split(tfmt, L, 1, H, HQ, T)["n_workgroups"])
    tq.tq_compress_kv_bounded(tfmt, tables, target, K2, V2, free, slot0=0, stream=side)
    for o in outs:
        tq.tq_decode_attention(tfmt, tables, cache, Q, st, ln, T, o, ws, stream=main)
    torch.cuda.synchronize()
    for name, t0 in ref_target.planes.items():
        if t0 is not None:
            assert torch.equal(t0, target.planes[name]), name
    scale = float(ref_out.abs().max())
    for o in outs:
        assert float((o - ref_out).abs().max()) <= 1e-5 * scale


def _check_sampled_heads(w, fmt, layers, dev, samples, sampled_inputs, slots, cap, out, Q, starts, lens):
    """The oracle's compression and decode of sampled (layer, KV head) pairs
    against the device cache and decode outputs."""
    G = w.group
    for li, kvh in samples:
        layer = layers[li]
        k, v = sampled_inputs[li]
        one = w.with_(n_kv_heads=1, n_q_heads=G, name=w.name + "_one_head")
        c, det = pu.oracle_compress_layer(one, layer, fmt, k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], slots, cap)
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        gl = pu.download_cache(dev, fmt)[li]
        sub = {n: (a[kvh:kvh + 1] if isinstance(a, np.ndarray) else a) for n, a in gl.items()}
        sub["n_kv_heads"] = 1
        st = pu.compare_layer(sub, c, det, fmt, slots, layer)
        _say("sample", fmt, layer, kvh, st)
        if out is not None:
            qh = Q[li][:, kvh * G:(kvh + 1) * G]
            ref = attention.decode_attention(c, qh, starts, lens, pi, s, cbk, cbv)
            err = pu.check_outputs(out[li][:, kvh * G:(kvh + 1) * G], ref)
            _say("sample out err", f"{err:.2e}")


@pytest.mark.parametrize("short", ["w2", "w3", "w4", "w5"])
def test_full_size_sampled(short):
    """Full workload size in the benchmark's launch configuration (each
    storage format's layers in one cache; one format decoded by one call, the
    28-layer asymmetric workload's fp16-key / 4-bit-value layers and fp16
    boundary layers by one tq_decode_attend_parts launch; a ragged batch
    compressed through a slot list); the oracle recomputes sampled (layer, KV
    head) pairs end to end in every format.  The 16-sequence workload also
    compresses its 32768-token prefill of 8 KV heads in one bulk call, checked
    on sampled heads."""
    import kv_cache_quantization_norm_amd as tq
    w = wl.BY_SHORT[short]
    _say("full-size", w.name)
    starts, lens, cap, slots = pu.slots_of(w)
    dt = _torch_dtype(w)
    rs = np.random.default_rng(1)
    by_fmt = {}
    for f, layers in pu.layer_groups(w):
        by_fmt.setdefault(f, []).extend(layers)
    # the fp16 / fp16 layers last, as the benchmark orders its parts
    groups = sorted(by_fmt.items(), key=lambda fl: (fl[0].k_bits, fl[0].v_bits) == (0, 0))
    n_samples = 2 if len(groups) == 1 else 1
    st = torch.from_numpy(slots).cuda()
    built = []
    for fmt, layers in groups:
        tfmt = pu.tq_format(fmt)
        tables = tq.Tables.create(tfmt, layers)
        dev = tq.Cache.allocate(tfmt, len(layers), w.n_kv_heads, cap)
        samples = [(int(rs.integers(len(layers))), int(rs.integers(w.n_kv_heads))) for _ in range(n_samples)]
        sampled_inputs = {}
        for i, layer in enumerate(layers):
            k, v = wl.gen_kv(w, layer)
            heads = [kvh for li, kvh in samples if li == i]
            if heads:
                # sampled heads: no decision within 1e-6 of its threshold (see test_end_to_end)
                k, v, n = pu.sanitize_near_boundary(fmt, layer, k, v, heads=heads)
                _say("layer", layer, "heads", heads, "zeroed", n)
                sampled_inputs[i] = (k, v)
            kt = torch.from_numpy(k).to("cuda", dt)[None].contiguous()
            vt = torch.from_numpy(v).to("cuda", dt)[None].contiguous()
            if len(w.seq_lens) == 1:
                tq.tq_compress_kv(tfmt, tables, dev, kt, vt, layer0=i, slot0=int(starts[0]))
            else:
                tq.tq_compress_kv(tfmt, tables, dev, kt, vt, layer0=i, slots=st)
            del kt, vt
        Q = np.stack([wl.gen_q(w, layer) for layer in layers])
        built.append((fmt, tables, dev, layers, Q, samples, sampled_inputs))
    if len(built) == 2 and (built[1][0].k_bits, built[1][0].v_bits) == (0, 0):
        max_len = int(max(lens))
        sl = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
        ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
        parts = []
        for fmt, tables, dev, layers, Q, _, _ in built:
            tfmt = pu.tq_format(fmt)
            qt = torch.from_numpy(Q).cuda().contiguous()
            ws = tq.workspace_for(tfmt, dev, len(lens), w.n_q_heads, max_len)
            out = torch.full((len(layers), len(lens), w.n_q_heads, 128), float("nan"), device="cuda")
            tq.tq_decode_prepare(tfmt, tables, dev, qt, max_len, ws)
            parts.append(tq.StepPart(tfmt, tables, dev, None, None, qt, out, ws))
        tq.tq_decode_attend_parts(parts, sl, ln, max_len)
        torch.cuda.synchronize()
        outs = [p.out.cpu().numpy() for p in parts]
        del parts
    else:
        outs = [_decode_gpu(fmt, tables, dev, Q, starts, lens, want_logits=False)[0]
                for fmt, tables, dev, _, Q, _, _ in built]
    for (fmt, tables, dev, layers, Q, samples, sampled_inputs), out in zip(built, outs):
        _check_sampled_heads(w, fmt, layers, dev, samples, sampled_inputs, slots, cap, out, Q, starts, lens)
    del built
    if short == "w5":
        P = 32768
        pw = w.with_(seq_lens=(P,), name=w.name + "_prefill")
        fmt, layers = pu.layer_groups(pw)[0]
        tfmt = pu.tq_format(fmt)
        tables = tq.Tables.create(tfmt, layers)
        dev = tq.Cache.allocate(tfmt, 1, pw.n_kv_heads, P)
        k, v = wl.gen_kv(pw, 0, stream=2)
        heads = [int(h) for h in rs.choice(pw.n_kv_heads, 2, replace=False)]
        k, v, n = pu.sanitize_near_boundary(fmt, 0, k, v, heads=heads)
        _say("prefill heads", heads, "zeroed", n)
        tq.tq_compress_kv(tfmt, tables, dev, torch.from_numpy(k).to("cuda", dt)[None].contiguous(),
                          torch.from_numpy(v).to("cuda", dt)[None].contiguous(), slot0=0)
        torch.cuda.synchronize()
        pslots = np.arange(P, dtype=np.int64)
        _check_sampled_heads(pw, fmt, layers, dev, [(0, h) for h in heads], {0: (k, v)}, pslots, P, None, None,
                             None, None)


def test_tail_ring_policy_flush_and_decode():
    """The library's recent-token ring: tokens enter an fp16 ring (each at its
    ring slot and its mirror, tq_tail_append), tq_tail_policy decides when the
    oldest whole 32-token blocks move to the packed cache (min_compress_tokens,
    keep_recent) and tq_tail_flush moves them from their fp16 values.  Three
    sequences (prefills of 300, 40 and 0 tokens) run 150 steps, so the rings
    wrap; the decode over packed part + ring range (one contiguous range even
    when it wraps) is checked against the oracle on the GPU's caches, the ring
    ranges against the tokens they should hold, and at the end every moved
    token's record against the oracle's compression of its fp16 values."""
    import kv_cache_quantization_norm_amd as tq
    _say("tail ring")
    L, H, HQ, B, R, steps = 2, 2, 14, 3, 96, 150
    min_compress, keep = 64, 16
    P0 = (300, 40, 0)
    span = 1024                      # packed slots per sequence
    fmt, fmt16 = quant.Format(128, 4, 4), quant.Format(128, 0, 0)
    tfmt, tfmt16 = pu.tq_format(fmt), pu.tq_format(fmt16)
    tables = tq.Tables.create(tfmt, list(range(L)))
    g = torch.Generator().manual_seed(41)
    K = torch.randn(L, B, max(P0) + steps, H, 128, generator=g).to("cuda", torch.float16)
    V = torch.randn(L, B, max(P0) + steps, H, 128, generator=g).to("cuda", torch.float16)
    Q = torch.randn(L, B, HQ, 128, generator=g).cuda()
    packed = tq.Cache.allocate(tfmt, L, H, B * span)
    tails = [tq.Cache.allocate(tfmt16, L, H, 2 * R) for _ in range(B)]   # one ring per sequence
    n_packed, head, n_tail, n_seen = [0] * B, [0] * B, [0] * B, list(P0)
    # prefill: what the policy would move goes to the packed cache, the rest into the ring
    for b in range(B):
        m = int(tq.tq_tail_policy([0], [P0[b]], min_compress, keep)[0])
        if m:
            tq.tq_compress_kv(tfmt, tables, packed, K[:, b, :m].contiguous(), V[:, b, :m].contiguous(), slot0=b * span)
        n_packed[b] = m
        rest = P0[b] - m
        if rest:
            rs = torch.arange(rest, dtype=torch.int64, device="cuda") % R
            tq.tq_tail_append(tfmt16, tables, tails[b], K[:, b, m:P0[b]].contiguous(), V[:, b, m:P0[b]].contiguous(), rs, R)
        n_tail[b] = rest
    ws_flush = tq.tail_flush_workspace_for(tfmt, packed, 1, R)
    ws = tq.tail_workspace_for(tfmt, packed, 1, HQ, span, R)
    out = torch.empty(L, 1, HQ, 128, device="cuda")
    flushes, wraps, checks = 0, 0, 0
    for step in range(steps):
        for b in range(B):
            tok = n_seen[b]
            rs = torch.tensor([(head[b] + n_tail[b]) % R], dtype=torch.int64, device="cuda")
            tq.tq_tail_append(tfmt16, tables, tails[b], K[:, b, tok:tok + 1].contiguous(),
                              V[:, b, tok:tok + 1].contiguous(), rs, R)
            n_seen[b] += 1
            n_tail[b] += 1
        nf = tq.tq_tail_policy(n_packed, n_tail, min_compress, keep)
        for b in range(B):
            if nf[b] == 0:
                continue
            assert nf[b] % 32 == 0 and n_tail[b] - nf[b] >= keep
            one = lambda x, dt: torch.tensor([x], dtype=dt, device="cuda")
            tq.tq_tail_flush(tfmt, tables, packed, tails[b], R, one(head[b], torch.int64), one(int(nf[b]), torch.int32),
                             one(b * span + n_packed[b], torch.int64), ws_flush)
            n_packed[b] += int(nf[b])
            wraps += head[b] + int(nf[b]) >= R
            head[b] = (head[b] + int(nf[b])) % R
            n_tail[b] -= int(nf[b])
            flushes += 1
        if step % 29 == 0 or step == steps - 1:
            torch.cuda.synchronize()
            ora = pu.download_cache(packed, fmt)
            for b in range(B):
                ora_t = pu.download_cache(tails[b], fmt16)
                # the ring range holds the sequence's last n_tail tokens, in order
                got_k = np.stack([ora_t[layer]["k_f16"][:, head[b]:head[b] + n_tail[b]] for layer in range(L)])
                want_k = K[:, b, n_seen[b] - n_tail[b]:n_seen[b]].permute(0, 2, 1, 3).cpu().numpy()
                assert np.array_equal(got_k, want_k)
                st = torch.tensor([b * span], dtype=torch.int64, device="cuda")
                ln = torch.tensor([n_packed[b]], dtype=torch.int32, device="cuda")
                tst = torch.tensor([head[b]], dtype=torch.int64, device="cuda")
                tln = torch.tensor([n_tail[b]], dtype=torch.int32, device="cuda")
                tq.tq_decode_attention_tail(tfmt, tables, packed, tails[b], Q[:, b:b + 1].contiguous(), st, ln, span,
                                            tst, tln, R, out, ws)
                torch.cuda.synchronize()
                for layer in range(L):
                    pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
                    ref = attention.decode_attention_with_tail(ora[layer], ora_t[layer], Q[layer, b:b + 1].cpu().numpy(),
                                                               [b * span], [n_packed[b]], [head[b]], [n_tail[b]],
                                                               pi, s, cbk, cbv)
                    pu.check_outputs(out[layer].cpu().numpy(), ref)
            checks += 1
    _say("flushes", flushes, "wraps", wraps, "packed", n_packed, "tail", n_tail)
    assert flushes >= 8 and wraps >= 2 and checks >= 5
    # every moved token's record against the oracle's compression of its fp16 values
    gpu = pu.download_cache(packed, fmt)
    kh, vh = K.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64)
    for layer in range(L):
        pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
        ora = quant.empty_cache(fmt, H, B * span)
        slots = np.concatenate([b * span + np.arange(n_packed[b]) for b in range(B)])
        kk = np.concatenate([kh[layer, b, :n_packed[b]] for b in range(B)])
        vv = np.concatenate([vh[layer, b, :n_packed[b]] for b in range(B)])
        det = quant.compress_into(ora, kk, vv, slots, pi, s, cbk, cbv)
        det["keys"] = kk
        pu.compare_layer(gpu[layer], ora, det, fmt, slots, layer)


MULTI_CASES = {
    # 64 query rows per KV head (8 heads x 8 query tokens), two sequences
    "k4v4_g64": wl.Workload("k4v4_g64", 1, 2, 128, (700, 333), 4, 4, "bf16", 0.5, 2, 10.0),
    # 128 rows per KV head: two passes over the codes
    "k3v2_g128": wl.Workload("k3v2_g128", 1, 1, 128, (500,), 3, 2, "bf16", 0.5, 0, 1.0),
    # 72 rows: a full pass and a pass of one column block
    "k2v2_g72": wl.Workload("k2v2_g72", 1, 1, 72, (129, 0), 2, 2, "f32", 0.0, 0, 1.0),
    # fp16 keys, 20 rows (partly filled column blocks), ragged
    "k0v4_g20": wl.Workload("k0v4_g20", 2, 2, 40, (257, 31), 0, 4, "bf16", 0.5, 1, 10.0),
    # the wide key codes
    "k8v4_g64": wl.Workload("k8v4_g64", 1, 1, 64, (300,), 8, 4, "bf16", 0.5, 1, 10.0),
    "k5v1_g64": wl.Workload("k5v1_g64", 1, 1, 64, (96,), 5, 1, "f16", 0.3, 1, 5.0),
}


@pytest.mark.parametrize("case", list(MULTI_CASES))
def test_score_multi_on_oracle_cache(case):
    """tq_score_multi (64 query rows per pass over a KV head's codes) against
    the oracle's logits on the oracle's own packed cache, and against
    tq_score's kernel (8 rows per pass) on the same inputs."""
    import kv_cache_quantization_norm_amd as tq
    w = MULTI_CASES[case]
    _say("multi-query scores", case)
    for fmt, layers in pu.layer_groups(w):
        tables, _, ora_caches, _, (starts, lens, cap, slots) = _run_group(w, fmt, layers, dev_compress=False)
        dev = pu.upload_cache(ora_caches, fmt)
        Q = np.stack([wl.gen_q(w, layer) for layer in layers])
        tfmt = pu.tq_format(fmt)
        n_layers, batch, hq, _ = Q.shape
        max_len = int(max(lens))
        qt = torch.from_numpy(Q).cuda().contiguous()
        st = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
        ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
        ws = tq.workspace_for(tfmt, dev, batch, hq, max_len)
        multi = torch.full((n_layers, batch, hq, max_len), float("nan"), device="cuda")
        tq.tq_score_multi(tfmt, tables, dev, qt, st, ln, max_len, multi, ws)
        single = torch.full_like(multi, float("nan"))
        tq.tq_score(tfmt, tables, dev, qt, st, ln, max_len, single, ws)
        torch.cuda.synchronize()
        multi, single = multi.cpu().numpy(), single.cpu().numpy()
        for i, layer in enumerate(layers):
            pi, s, cbk, cbv = pu.oracle_tables(fmt, layer)
            _, ref_logits = attention.decode_attention(ora_caches[i], Q[i], starts, lens, pi, s, cbk, cbv,
                                                       return_logits=True)
            worst = pu.check_logits(multi[i], ref_logits, lens, hq)
            for b, n in enumerate(lens):
                assert np.all(np.isnan(multi[i, b, :, n:])), "positions past the sequence are left untouched"
                if n:
                    scale = np.max(np.abs(single[i, b, :, :n]))
                    assert np.max(np.abs(multi[i, b, :, :n] - single[i, b, :, :n])) <= 1e-5 * scale
            _say("format", fmt, "layer", layer, "worst logit rel", f"{worst:.2e}")
