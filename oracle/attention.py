"""Single-query decode attention over a packed TurboQuant cache.

Pages:
  * "TurboQuant QJL投影深度剖析" §六: the score of a cached key is the MSE part
    (the query rotated forward, dotted with the looked-up centroids, never
    materialising the de-quantised key) plus the QJL part (the pre-sketched
    query dotted with the unpacked +-1 signs, times sqrt(pi/2)/d * ||r||); the
    logits then go through a softmax, and the fused kernel does the whole
    decode attention with an online softmax in one pass.
  * MLX write-up, 背景: values are reconstructed from the MSE-only code, so the
    output is softmax(logits) @ V~.

This module computes that result by its plain definition: de-quantise every
key and value of the sequence (x~ = ||x|| Pi^T c[idx], v~ = ||v|| Pi^T c_v[idx]),
form l_t = scale * (<q, x~_t> + ||r_t|| sqrt(pi/2)/d <S q, 2 s_t - 1>), take a
two-pass softmax and the weighted sum, all in float64.  Fp16 keys (asymmetric
mode) score as scale * <q, k_t>; fp16 values are used as stored.

Readings: the softmax scale defaults to 1/sqrt(d) (standard scaled dot-product
attention; the pages only say "logits -> softmax").  Query head h reads KV
head h // G (contiguous grouping; the pages do not discuss GQA).

`decode_attention_rotated` is a second, independent formulation used to pin
the first: it scores with Pi q and S q directly against codes, runs an online
(one-pass, running max and sum) softmax in chunks and applies Pi^T once at the
end to the accumulated rotated-domain values.
"""
import math

import numpy as np

from . import quant


def softmax_two_pass(logits: np.ndarray) -> np.ndarray:
    m = np.max(logits)
    e = np.exp(logits - m)
    return e / np.sum(e)


def key_logits(q: np.ndarray, kp: dict, s: np.ndarray, scale: float) -> np.ndarray:
    """Logits of one query q [d] against key parts from quant.dequantize_cache."""
    q = np.asarray(q, np.float64)
    if "k" in kp:
        return scale * (kp["k"] @ q)
    d = q.shape[0]
    qs = s @ q
    return scale * (kp["xt"] @ q + quant.kappa(d) * kp["rnorm"] * (kp["sign_pm"] @ qs))


def decode_attention(cache: dict, q: np.ndarray, seq_start, seq_len, pi, s, cb_k, cb_v,
                     scale: float = 0.0, return_logits: bool = False):
    """q [B][Hq][d] float -> out [B][Hq][d] float64 (and logits per (b, h))."""
    fmt = cache["fmt"]
    d = fmt.d
    if scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    b_, hq, _ = q.shape
    hkv = cache["n_kv_heads"]
    g = hq // hkv
    out = np.zeros((b_, hq, d))
    logits_all = {}
    for b in range(b_):
        slots = np.arange(int(seq_start[b]), int(seq_start[b]) + int(seq_len[b]))
        for kvh in range(hkv):
            kp, vals = quant.dequantize_cache(cache, pi, cb_k, cb_v, kvh, slots)
            for h in range(kvh * g, (kvh + 1) * g):
                if len(slots) == 0:
                    out[b, h] = 0.0
                    logits_all[(b, h)] = np.zeros(0)
                    continue
                lg = key_logits(q[b, h], kp, s, scale)
                p = softmax_two_pass(lg)
                out[b, h] = p @ vals
                logits_all[(b, h)] = lg
    return (out, logits_all) if return_logits else out


def decode_attention_rotated(cache: dict, q: np.ndarray, seq_start, seq_len, pi, s, cb_k, cb_v,
                             scale: float = 0.0, chunk: int = 64):
    """Same result as decode_attention for TurboQuant K and MSE V, computed as
    rotated-query scoring against codes + online softmax + deferred Pi^T."""
    fmt = cache["fmt"]
    assert fmt.k_bits > 0 and fmt.v_bits > 0
    d = fmt.d
    if scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    ck = np.asarray(cb_k[0])
    cv = np.asarray(cb_v[0])
    kap = quant.kappa(d)
    b_, hq, _ = q.shape
    hkv = cache["n_kv_heads"]
    g = hq // hkv
    out = np.zeros((b_, hq, d))
    for b in range(b_):
        lo, n = int(seq_start[b]), int(seq_len[b])
        for kvh in range(hkv):
            kidx = quant.unpack_bits(cache["k_idx"][kvh, lo:lo + n], fmt.k_mse_bits, d)
            sgn = quant.unpack_bits(cache["k_sign"][kvh, lo:lo + n], 1, d).astype(np.float64) * 2 - 1
            kn = cache["k_norm"][kvh, lo:lo + n].astype(np.float64)
            rn = cache["k_rnorm"][kvh, lo:lo + n].astype(np.float64)
            vidx = quant.unpack_v_blocks(cache["v_idx"][kvh], fmt.v_bits)[lo:lo + n]
            vn = cache["v_norm"][kvh, lo:lo + n].astype(np.float64)
            for h in range(kvh * g, (kvh + 1) * g):
                qr = pi @ q[b, h].astype(np.float64)
                qs = s @ q[b, h].astype(np.float64)
                m, l, acc = -np.inf, 0.0, np.zeros(d)
                for c0 in range(0, n, chunk):
                    sl = slice(c0, min(n, c0 + chunk))
                    lg = scale * (kn[sl] * (ck[kidx[sl]] @ qr) + kap * rn[sl] * (sgn[sl] @ qs))
                    m_new = max(m, float(np.max(lg)))
                    alpha = math.exp(m - m_new) if np.isfinite(m) else 0.0
                    p = np.exp(lg - m_new)
                    l = l * alpha + float(np.sum(p))
                    acc = acc * alpha + (p * vn[sl]) @ cv[vidx[sl]]
                    m = m_new
                out[b, h] = (pi.T @ acc) / l if n > 0 else 0.0
    return out


def decode_attention_with_tail(cache: dict, tail: dict, q: np.ndarray, seq_start, seq_len, tail_start, tail_len,
                               pi, s, cb_k, cb_v, scale: float = 0.0):
    """Decode attention over a sequence held in two parts: its older tokens in
    the packed cache (slots [seq_start[b], + seq_len[b])) and its recent ones
    in `tail`, a cache of the fp16 format (slots [tail_start[b],
    + tail_len[b])), with one softmax over all of them.

    Pages: the MLX write-up (直接构造缓存, 限制) keeps the most recent tokens in
    full precision and compresses the older ones; the QJL deep-dive (§六) has
    the same recent-token buffer.  The plain definition: the logits and values
    of both parts, concatenated (packed tokens first), then the two-pass
    softmax and the weighted sum, in float64.  q [B][Hq][d] -> [B][Hq][d]."""
    fmt = cache["fmt"]
    d = fmt.d
    assert tail["fmt"].k_bits == 0 and tail["fmt"].v_bits == 0 and tail["fmt"].d == d
    if scale == 0.0:
        scale = 1.0 / math.sqrt(d)
    b_, hq, _ = q.shape
    hkv = cache["n_kv_heads"]
    g = hq // hkv
    out = np.zeros((b_, hq, d))
    for b in range(b_):
        slots = np.arange(int(seq_start[b]), int(seq_start[b]) + int(seq_len[b]))
        tslots = np.arange(int(tail_start[b]), int(tail_start[b]) + int(tail_len[b]))
        for kvh in range(hkv):
            kp, vals = quant.dequantize_cache(cache, pi, cb_k, cb_v, kvh, slots)
            tkp, tvals = quant.dequantize_cache(tail, pi, cb_k, cb_v, kvh, tslots)
            allv = np.concatenate([vals.reshape(-1, d), tvals.reshape(-1, d)])
            for h in range(kvh * g, (kvh + 1) * g):
                if len(allv) == 0:
                    continue
                lg = np.concatenate([key_logits(q[b, h], kp, s, scale) if len(slots) else np.zeros(0),
                                     key_logits(q[b, h], tkp, s, scale) if len(tslots) else np.zeros(0)])
                out[b, h] = softmax_two_pass(lg) @ allv
    return out


def attention_exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float = 0.0):
    """Textbook softmax(q K^T * scale) V for one query q [d], K, V [T, d]."""
    q = np.asarray(q, np.float64)
    if scale == 0.0:
        scale = 1.0 / math.sqrt(q.shape[0])
    p = softmax_two_pass(scale * (np.asarray(k, np.float64) @ q))
    return p @ np.asarray(v, np.float64)
