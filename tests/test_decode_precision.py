"""The decode kernel's centroid operands, bounded with the oracle alone.

Compression applies the fp32 table centroids.  Decode attention feeds the
centroids to fp16 MFMA operands:

* values, and keys with at most 2 Lloyd-Max bits: one fp16 value per
  centroid, alpha * c rounded to fp16, with alpha in [1, 2) chosen per
  codebook so that the largest relative rounding error over the centroid
  magnitudes is smallest; the query operand (keys) or the output (values)
  carries 1 / alpha;
* keys with 3 or more Lloyd-Max bits: an fp16 high part and an fp16
  remainder per centroid (about 22 significant bits).

Plain fp16 rounding (alpha = 1) is not enough on these data laws: the keys'
norms and the outlier channels make the softmax sharp (logits up to about 40),
and it moves outputs by up to 1e-2, five times the 2e-3 tolerance.  This test
computes, in float64 with the oracle, what the scaled fp16 operands alone do
to the logits and outputs on the workload laws and holds it to a third of the
parity tolerances (logits 1e-3 of the row's largest magnitude, outputs 2e-3
max-abs), leaving the rest to the kernel's own rounding.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import attention, codebook, quant, rotation


def fp16_scale(c):
    """alpha in [1, 2) minimising max_k |fp16(alpha m_k) - alpha m_k| / (alpha m_k)
    over the nonzero centroid magnitudes m_k (fp32), among the candidates that
    put one magnitude exactly on an fp16 value.  Returns (alpha, error)."""
    m = np.unique(np.abs(np.asarray(c, np.float32)[np.asarray(c) != 0]).astype(np.float64))
    best = (np.inf, 1.0)
    for mk in m:
        e = np.floor(np.log2(mk))
        grid = 2.0 ** e * (1 + np.arange(2048) / 1024.0)    # fp16 values of the two binades from mk's
        a = grid / mk
        a = a[(a >= 1) & (a < 2)]
        v = a[:, None] * m[None, :]
        err = np.max(np.abs(v.astype(np.float16).astype(np.float64) - v) / v, axis=1)
        j = int(np.argmin(err))
        if err[j] < best[0]:
            best = (float(err[j]), float(a[j]))
    return best[1], best[0]


def operand_codebook(cb):
    """The centroids as the decode operands represent them."""
    c, t = cb
    alpha, _ = fp16_scale(c)
    return (np.asarray(c) * alpha).astype(np.float16).astype(np.float64) / alpha, t


@pytest.mark.parametrize("bits,expect", [(1, 0.0), (2, 2e-6), (4, 1e-4)])
def test_fp16_scale_search(bits, expect):
    c, _ = codebook.table_codebook(128, bits)
    alpha, err = fp16_scale(c)
    assert 1.0 <= alpha < 2.0 and err <= expect
    # plain rounding is worse by an order of magnitude or more
    m = np.abs(c)
    plain = np.max(np.abs(m.astype(np.float16).astype(np.float64) - m) / m)
    assert plain > 2e-4 and (err == 0 or plain / err > 3)


@pytest.mark.parametrize("k_bits,v_bits", [(4, 4), (3, 2), (8, 4), (5, 1), (2, 2), (0, 4), (3, 1)])
def test_decode_operands_stay_within_a_third_of_the_tolerances(k_bits, v_bits):
    w = wl.Workload("precision", 1, 2, 16, (3000,), k_bits, v_bits, "bf16", 0.5, 2, 10.0)
    fmt = quant.Format(128, k_bits, v_bits)
    pi, s = rotation.layer_rotations(128, 3)
    cbk = codebook.table_codebook(128, fmt.k_mse_bits) if k_bits else None
    cbv = codebook.table_codebook(128, v_bits) if v_bits else None
    k, v = wl.gen_kv(w, 0)
    q = wl.gen_q(w, 0)
    cache = quant.empty_cache(fmt, 2, 3008)
    quant.compress_into(cache, k.astype(np.float64), v.astype(np.float64), np.arange(3000), pi, s, cbk, cbv)
    ref, ref_lg = attention.decode_attention(cache, q, [0], [3000], pi, s, cbk, cbv, return_logits=True)
    # keys of >= 3 Lloyd-Max bits: high part + remainder, exact to about 2^-22 (taken as exact here)
    ok = operand_codebook(cbk) if (k_bits and fmt.k_mse_bits <= 2) else cbk
    ov = operand_codebook(cbv) if v_bits else None
    got, got_lg = attention.decode_attention(cache, q, [0], [3000], pi, s, ok, ov, return_logits=True)
    worst_l = max(np.max(np.abs(got_lg[key] - ref_lg[key])) / np.max(np.abs(ref_lg[key])) for key in ref_lg)
    worst_o = float(np.max(np.abs(got - ref)))
    print(f"K{k_bits}/V{v_bits}: logit {worst_l:.2e} of the row maximum, output {worst_o:.2e} max-abs")
    assert worst_l <= 1e-3 / 3
    assert worst_o <= 2e-3 / 3


def test_plain_fp16_centroids_are_not_enough():
    """The reason for the scaled / split operands: with every centroid simply
    rounded to fp16 the 4-bit keys move outputs beyond the tolerance."""
    w = wl.Workload("precision", 1, 2, 16, (3000,), 4, 4, "bf16", 0.5, 2, 10.0)
    fmt = quant.Format(128, 4, 4)
    pi, s = rotation.layer_rotations(128, 3)
    cbk, cbv = codebook.table_codebook(128, 3), codebook.table_codebook(128, 4)
    k, v = wl.gen_kv(w, 0)
    q = wl.gen_q(w, 0)
    cache = quant.empty_cache(fmt, 2, 3008)
    quant.compress_into(cache, k.astype(np.float64), v.astype(np.float64), np.arange(3000), pi, s, cbk, cbv)
    ref = attention.decode_attention(cache, q, [0], [3000], pi, s, cbk, cbv)
    f16 = (cbk[0].astype(np.float16).astype(np.float64), cbk[1])
    got = attention.decode_attention(cache, q, [0], [3000], pi, s, f16, cbv)
    assert np.max(np.abs(got - ref)) > 2e-3
