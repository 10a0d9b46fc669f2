"""Pins for the oracle's decode attention over a packed cache."""
import math

import numpy as np
import pytest

from oracle import attention, codebook, quant, rotation


def _build(fmt, n_kv, lens, seed=0, g=2, scale_k=1.0, d=None):
    d = d or fmt.d
    pi, s = rotation.make_rotations(d, 42 + seed)
    cbk = codebook.codebook(d, fmt.k_mse_bits) if fmt.k_bits else None
    cbv = codebook.codebook(d, fmt.v_bits) if fmt.v_bits else None
    starts = []
    pos = 0
    for n in lens:
        starts.append(pos)
        pos += (n + 31) // 32 * 32
    cache = quant.empty_cache(fmt, n_kv, max(pos, 32))
    rs = np.random.default_rng(seed)
    kv = []
    for b, n in enumerate(lens):
        k = rs.standard_normal((n, n_kv, d)) * scale_k
        v = rs.standard_normal((n, n_kv, d))
        quant.compress_into(cache, k, v, np.arange(starts[b], starts[b] + n), pi, s, cbk, cbv)
        kv.append((k, v))
    q = rs.standard_normal((len(lens), n_kv * g, d))
    return cache, q, np.array(starts), np.array(lens), pi, s, cbk, cbv, kv


@pytest.mark.parametrize("kb,vb", [(3, 2), (4, 4), (2, 1), (5, 3)])
def test_rotated_online_form_equals_plain_definition(kb, vb):
    fmt = quant.Format(128, kb, vb)
    cache, q, st, ln, pi, s, cbk, cbv, _ = _build(fmt, 2, [200, 77, 1], seed=kb, g=3)
    a = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    b = attention.decode_attention_rotated(cache, q, st, ln, pi, s, cbk, cbv, chunk=48)
    assert np.max(np.abs(a - b)) < 1e-12 * max(1.0, np.max(np.abs(a)))


def test_brute_force_tiny():
    # d = 8, T <= 8: recompute de-quantisation, logits, softmax and the
    # weighted sum with explicit Python loops over scalars.
    d = 8
    fmt = quant.Format(d, 3, 2)
    cache, q, st, ln, pi, s, cbk, cbv, _ = _build(fmt, 1, [7], seed=3, g=2, d=d)
    out = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    ck, cv = cbk[0], cbv[0]
    kidx = quant.unpack_bits(cache["k_idx"][0, :7], 2, d)
    sgn = quant.unpack_bits(cache["k_sign"][0, :7], 1, d)
    vidx = quant.unpack_v_blocks(cache["v_idx"][0], 2)[:7]
    kap = math.sqrt(math.pi / 2) / d
    scale = 1 / math.sqrt(d)
    for h in range(2):
        qq = [float(x) for x in q[0, h]]
        logits, vals = [], []
        for t in range(7):
            xt = [sum(float(pi[j][i]) * float(ck[kidx[t][j]]) for j in range(d)) * float(cache["k_norm"][0, t])
                  for i in range(d)]
            sq = [sum(float(s[i][j]) * qq[j] for j in range(d)) for i in range(d)]
            qjl = sum(sq[i] * (1.0 if sgn[t][i] else -1.0) for i in range(d))
            logits.append(scale * (sum(qq[i] * xt[i] for i in range(d))
                                   + kap * float(cache["k_rnorm"][0, t]) * qjl))
            vals.append([sum(float(pi[j][i]) * float(cv[vidx[t][j]]) for j in range(d)) * float(cache["v_norm"][0, t])
                         for i in range(d)])
        mx = max(logits)
        e = [math.exp(l - mx) for l in logits]
        z = sum(e)
        ref = [sum(e[t] / z * vals[t][i] for t in range(7)) for i in range(d)]
        assert np.max(np.abs(np.array(ref) - out[0, h])) < 1e-12


def test_fp16_keys_and_values_reduce_to_textbook_attention():
    fmt = quant.Format(128, 0, 0)
    cache, q, st, ln, pi, s, cbk, cbv, kv = _build(fmt, 2, [150, 40], seed=1, g=2)
    out = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    for b in range(2):
        k, v = kv[b]
        for h in range(4):
            kvh = h // 2
            kk = k[:, kvh].astype(np.float16).astype(np.float64)
            vv = v[:, kvh].astype(np.float16).astype(np.float64)
            ref = attention.attention_exact(q[b, h], kk, vv)
            assert np.max(np.abs(ref - out[b, h])) < 1e-12


def test_fine_value_codebook_approaches_exact_attention():
    # K fp16 (asymmetric mode) and a 6-bit MSE value code: the output is
    # textbook attention up to the value quantisation error.
    fmt = quant.Format(128, 0, 6)
    cache, q, st, ln, pi, s, cbk, cbv, kv = _build(fmt, 1, [300], seed=2, g=1)
    out = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    k, v = kv[0]
    ref = attention.attention_exact(q[0, 0], k[:, 0].astype(np.float16), v[:, 0])
    err = np.max(np.abs(ref - out[0, 0]))
    assert err < 2e-2 * np.max(np.abs(ref)) and err > 0


def _logit_bias_z(n_draws=1500, n_keys=8, seed=4):
    """z-scores of the mean TurboQuant logit over independent sketches S
    against the exact scale * <q, x>, per key: the keys, the query and Pi are
    fixed; every draw compresses the keys with its own Gaussian S into a
    packed cache and scores them through the decode path's logits."""
    d = 128
    fmt = quant.Format(d, 3, 2)
    pi, _ = rotation.make_rotations(d, 42 + seed)
    cbk, cbv = codebook.codebook(d, 2), codebook.codebook(d, 2)
    rs = np.random.default_rng(seed)
    k = rs.standard_normal((n_keys, 1, d)) * 2.0
    v = rs.standard_normal((n_keys, 1, d))
    q = rs.standard_normal((1, 1, d))
    scale = 1.0 / math.sqrt(d)
    truth = scale * (k[:, 0] @ q[0, 0])
    lg = np.empty((n_draws, n_keys))
    for i in range(n_draws):
        s = rs.standard_normal((d, d))
        cache = quant.empty_cache(fmt, 1, 32)
        quant.compress_into(cache, k, v, np.arange(n_keys), pi, s, cbk, cbv)
        _, logits = attention.decode_attention(cache, q, [0], [n_keys], pi, s, cbk, cbv, return_logits=True)
        lg[i] = logits[(0, 0)]
    return (lg.mean(axis=0) - truth) / (lg.std(axis=0) / math.sqrt(n_draws))


def test_turboquant_logits_are_unbiased_estimates(monkeypatch):
    """QJL page §五: over independent sketches the decode logits average to
    the exact scale * <q, x> for every key; with the QJL constant scaled by
    0.5 or 1.5 they do not (the residual's part <q, r> is then missed or
    overcounted)."""
    z = _logit_bias_z()
    assert np.max(np.abs(z)) < 4.5, z
    kappa = quant.kappa
    for f in (0.5, 1.5):
        monkeypatch.setattr(quant, "kappa", lambda d, f=f: f * kappa(d))
        z = _logit_bias_z(n_draws=800)
        assert np.max(np.abs(z)) > 10, (f, z)
    monkeypatch.setattr(quant, "kappa", kappa)


def test_mse_only_logits_are_biased_by_the_distortion():
    # the MSE-only part is biased toward zero by the factor 1 - D
    fmt = quant.Format(128, 3, 2)
    cache, q, st, ln, pi, s, cbk, cbv, kv = _build(fmt, 1, [4000], seed=4, g=1, scale_k=1.0)
    k = kv[0][0][:, 0]
    true = (k @ q[0, 0]) / math.sqrt(128)
    kp, _ = quant.dequantize_cache(cache, pi, cbk, cbv, 0, np.arange(4000))
    mse_only = (kp["xt"] @ q[0, 0]) / math.sqrt(128)
    slope = np.sum(mse_only * true) / np.sum(true * true)
    c, t = cbk
    assert abs(slope - (1 - 128 * codebook.coordinate_mse(c, t, 128))) < 0.01


def test_gqa_mapping_ragged_batch_and_empty_sequence():
    fmt = quant.Format(128, 4, 4)
    cache, q, st, ln, pi, s, cbk, cbv, _ = _build(fmt, 2, [33, 0, 64], seed=5, g=3)
    out = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    assert np.all(out[1] == 0)
    # sequence 2 alone gives the same rows
    o2 = attention.decode_attention(cache, q[2:3], st[2:3], ln[2:3], pi, s, cbk, cbv)
    assert np.array_equal(o2[0], out[2])
    # query heads 0..2 read KV head 0: swapping KV head 1's records changes
    # only heads 3..5
    c2 = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    for key in ("k_idx", "k_sign", "k_norm", "k_rnorm", "v_idx", "v_norm"):
        c2[key][1] = np.roll(c2[key][1], 1, axis=0)
    o3 = attention.decode_attention(c2, q, st, ln, pi, s, cbk, cbv)
    assert np.array_equal(o3[:, :3], out[:, :3])
    assert not np.allclose(o3[0, 3:], out[0, 3:])


def _fp16_cache(n_kv, lens, starts, kv_list, pi, s):
    fmt16 = quant.Format(128, 0, 0)
    cap = max(32, max((st + (n + 31) // 32 * 32 for st, n in zip(starts, lens)), default=32))
    tail = quant.empty_cache(fmt16, n_kv, cap)
    for st, n, (k, v) in zip(starts, lens, kv_list):
        if n:
            quant.compress_into(tail, k, v, np.arange(st, st + n), pi, s, None, None)
    return tail


def test_tail_empty_equals_packed_decode():
    fmt = quant.Format(128, 4, 4)
    cache, q, st, ln, pi, s, cbk, cbv, _ = _build(fmt, 2, [120, 33], seed=6, g=3)
    tail = _fp16_cache(2, [0, 0], [0, 0], [], pi, s)
    a = attention.decode_attention(cache, q, st, ln, pi, s, cbk, cbv)
    b = attention.decode_attention_with_tail(cache, tail, q, st, ln, [0, 0], [0, 0], pi, s, cbk, cbv)
    assert np.array_equal(a, b)


def test_tail_only_equals_textbook_attention():
    # no packed tokens: softmax(q K^T / sqrt(d)) V over the fp16 tail
    fmt = quant.Format(128, 3, 2)
    cache, q, _, _, pi, s, cbk, cbv, _ = _build(fmt, 2, [40], seed=7, g=2)
    rs = np.random.default_rng(70)
    k, v = rs.standard_normal((57, 2, 128)), rs.standard_normal((57, 2, 128))
    tail = _fp16_cache(2, [57], [0], [(k, v)], pi, s)
    out = attention.decode_attention_with_tail(cache, tail, q, [0], [0], [0], [57], pi, s, cbk, cbv)
    for h in range(4):
        kk = k[:, h // 2].astype(np.float16).astype(np.float64)
        vv = v[:, h // 2].astype(np.float16).astype(np.float64)
        assert np.max(np.abs(attention.attention_exact(q[0, h], kk, vv) - out[0, h])) < 1e-12


def test_tail_split_equals_one_softmax():
    # an fp16 sequence split between a cache (older tokens) and a tail (recent
    # ones) gives the single-cache result: one softmax over the union
    fmt16 = quant.Format(128, 0, 0)
    cache, q, st, ln, pi, s, _, _, kv = _build(fmt16, 2, [150], seed=8, g=2)
    k, v = kv[0]
    older = _fp16_cache(2, [100], [0], [(k[:100], v[:100])], pi, s)
    recent = _fp16_cache(2, [50], [32], [(k[100:], v[100:])], pi, s)
    full = attention.decode_attention(cache, q, st, ln, pi, s, None, None)
    split = attention.decode_attention_with_tail(older, recent, q, [0], [100], [32], [50], pi, s, None, None)
    assert np.max(np.abs(full - split)) < 1e-12
