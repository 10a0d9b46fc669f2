"""Pins for the oracle's compression, packing and inner-product estimator."""
import math

import numpy as np
import pytest

from oracle import codebook, quant, rotation
from tests.conftest import load_golden

D = 128


def _tables(bits_mse, d=D, seed=42):
    pi, s = rotation.make_rotations(d, seed)
    return pi, s, codebook.codebook(d, bits_mse)


def _bigint_pack(codes, m):
    v = 0
    for j, c in enumerate(codes):
        v |= int(c) << (j * m)
    return list(v.to_bytes(len(codes) * m // 8, "little"))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 8])
def test_pack_matches_bit_position_definition(m):
    rs = np.random.default_rng(m)
    codes = rs.integers(0, 1 << m, size=(5, 64))
    packed = quant.pack_bits(codes, m)
    for row, prow in zip(codes, packed):
        assert list(prow) == _bigint_pack(row, m)
    assert np.array_equal(quant.unpack_bits(packed, m, 64), codes)


def test_pack_hand_example():
    # 3-bit codes 1..7,0: 1 + 2<<3 + 3<<6 + 4<<9 + 5<<12 + 6<<15 + 7<<18 = 0x1F58D1
    assert list(quant.pack_bits(np.array([1, 2, 3, 4, 5, 6, 7, 0]), 3)) == [0xD1, 0x58, 0x1F]
    # sign bits: coordinate j at bit j
    assert list(quant.pack_bits(np.array([1, 0, 0, 0, 0, 0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0]), 1)) == [0x81, 0x02]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_v_block_layout(b):
    rs = np.random.default_rng(b)
    idx = rs.integers(0, 1 << b, size=(96, 16))
    packed = quant.pack_v_blocks(idx, b)
    assert packed.shape == (3, 16, 4 * b)
    for blk in range(3):
        for j in range(16):
            assert list(packed[blk, j]) == _bigint_pack(idx[blk * 32:(blk + 1) * 32, j], b)
    assert np.array_equal(quant.unpack_v_blocks(packed, b), idx)


def test_record_sizes_and_page_constants():
    pc = load_golden("page_constants.json")
    assert quant.Format(D, 4, 4).k_record_bytes() == 48 + 16 + 8
    assert quant.Format(D, 3, 2).k_record_bytes() == 32 + 16 + 8
    assert quant.Format(D, 4, 4).v_record_bytes() == 64 + 4
    assert quant.Format(D, 3, 2).v_record_bytes() == 32 + 4
    c = quant.empty_cache(quant.Format(D, 3, 2), 1, 32)
    assert c["k_sign"].shape[-1] == pc["sign_bytes_per_key"]["bytes"]
    assert c["k_idx"].shape[-1] == D * 2 // 8
    # 3-bit key: (2 + 1) bits per coordinate = 0.375 bytes/dim before norms
    assert (c["k_idx"].shape[-1] + c["k_sign"].shape[-1]) / D == pc["key_bytes_per_dim_3bit"]["correct_value"]
    assert abs(quant.kappa(D) - math.sqrt(math.pi / 2) / D) == 0.0


def test_decision_is_nearest_centroid():
    c, t = codebook.codebook(D, 3)
    y = np.random.default_rng(0).normal(0, 1 / math.sqrt(D), size=20000)
    idx = quant.decide(y, t)
    nearest = np.argmin(np.abs(y[:, None] - c[None, :]), axis=1)
    assert np.array_equal(idx, nearest)
    # ties go to the upper cell
    assert np.array_equal(quant.decide(t.astype(np.float32).astype(np.float64), t), np.arange(1, 8))


def test_mse_only_bias_matches_codebook_distortion():
    # E <x/|x|, x~/|x|> = 1 - d * D_coord for an MSE-optimal (Lloyd-Max)
    # quantiser (QJL page, section 3: the MSE quantiser is biased).
    for bits in (2, 4):
        pi, _, (c, t) = _tables(bits)
        x = np.random.default_rng(bits).standard_normal((20000, D)) * 3.0
        idx, n = quant.compress_v(x, pi, c, t)
        xt = quant.dequantize_mse(idx, n, pi, c)
        ratio = np.sum(x * xt, axis=1) / np.sum(x * x, axis=1)
        expect = 1.0 - D * codebook.coordinate_mse(c, t, D)
        assert abs(ratio.mean() - expect) < 4 * ratio.std() / math.sqrt(len(ratio)) + 2e-4
        assert expect < 1.0


def test_v_cosine_two_bit_from_page():
    pc = load_golden("page_constants.json")["v_cosine"]
    pi, _, (c, t) = _tables(2)
    v = np.random.default_rng(5).standard_normal((20000, D))
    idx, n = quant.compress_v(v, pi, c, t)
    vt = quant.dequantize_mse(idx, n, pi, c)
    cos = np.sum(v * vt, 1) / (np.linalg.norm(v, axis=1) * np.linalg.norm(vt, axis=1))
    assert abs(cos.mean() - pc["2"]) < pc["tolerance_2bit"]
    # 4-bit: reported, the page's 0.997 is not reached on Gaussian data.
    pi4, _, (c4, t4) = _tables(4)
    idx4, n4 = quant.compress_v(v, pi4, c4, t4)
    vt4 = quant.dequantize_mse(idx4, n4, pi4, c4)
    cos4 = np.sum(v * vt4, 1) / (np.linalg.norm(v, axis=1) * np.linalg.norm(vt4, axis=1))
    assert abs(cos4.mean() - math.sqrt(1 - D * codebook.coordinate_mse(c4, t4, D))) < 2e-3


def _estimates_over_sketches(x, y, pi, c, t, n_draws, seed, d):
    """quant.estimate_inner over n_draws independent Gaussian sketches S, with
    Pi, x and y fixed: each draw compresses x with its own S
    (quant.compress_k) and estimates <y, x> from the record."""
    rs = np.random.default_rng(seed)
    out = np.empty(n_draws)
    rec = None
    for i in range(n_draws):
        s = rs.standard_normal((d, d))
        rec = quant.compress_k(x[None], pi, s, c, t)
        out[i] = quant.estimate_inner(y, rec, pi, s, c)[0]
    # the residual does not depend on S
    xt = quant.dequantize_mse(rec["idx"], rec["norm"], pi, c)[0]
    r = x - xt
    return out, r, float(np.linalg.norm(r))


def test_estimator_is_unbiased_with_closed_form_variance():
    d = D
    pi, _, (c, t) = _tables(2, d)
    rs = np.random.default_rng(11)
    x = rs.standard_normal(d) * 2.0
    y = rs.standard_normal(d)
    est, r, rho = _estimates_over_sketches(x, y, pi, c, t, 6000, 3, d)
    truth = float(x @ y)
    se = est.std() / math.sqrt(len(est))
    assert abs(est.mean() - truth) < 4 * se
    var_cf = (math.pi / 2 * rho ** 2 * (y @ y) - (y @ r) ** 2) / d
    assert abs(est.var() / var_cf - 1) < 0.08
    # and the MSE-only part alone is biased by exactly <y, r>
    xt = x - r
    assert abs((y @ xt) + (y @ r) - truth) < 1e-9


def _bias_in_standard_errors(d=D, n_draws=2000):
    """(mean estimate - <y, x>) / standard error, for a query with a large
    component along the key's residual, so that the QJL term carries the
    estimate."""
    pi, _, (c, t) = _tables(2, d)
    rs = np.random.default_rng(21)
    x = rs.standard_normal(d) * 2.0
    idx, n = quant.compress_v(x[None], pi, c, t)
    r = x - quant.dequantize_mse(idx, n, pi, c)[0]
    y = rs.standard_normal(d) + 3.0 * r / np.linalg.norm(r)
    est, _, _ = _estimates_over_sketches(x, y, pi, c, t, n_draws, 5, d)
    return (est.mean() - float(x @ y)) / (est.std() / math.sqrt(len(est)))


def test_estimator_pins_the_qjl_constant(monkeypatch):
    """Unbiasedness fixes sqrt(pi/2)/d: the estimator with the QJL constant
    scaled by 0.5 or 1.5 is biased by many standard errors."""
    assert abs(_bias_in_standard_errors()) < 4
    kappa = quant.kappa
    for f in (0.5, 1.5):
        monkeypatch.setattr(quant, "kappa", lambda d, f=f: f * kappa(d))
        assert abs(_bias_in_standard_errors()) > 20, f
    monkeypatch.setattr(quant, "kappa", kappa)


def test_estimator_variance_scales_as_one_over_d():
    vals = {}
    for d in (32, 64, 128, 256):
        pi, _, (c, t) = _tables(2, d, seed=100 + d)
        rs = np.random.default_rng(d)
        x = rs.standard_normal(d)
        y = rs.standard_normal(d)
        est, r, rho = _estimates_over_sketches(x, y, pi, c, t, 3000, d, d)
        # normalised by rho^2 |y|^2 the variance is (pi/2 - cos^2(y, r)) / d
        cos2 = (y @ r) ** 2 / (rho ** 2 * (y @ y))
        vals[d] = est.var() / (rho ** 2 * (y @ y)) * d / (math.pi / 2 - cos2)
    for d, v in vals.items():
        assert abs(v - 1) < 0.12, (d, v)


def test_compress_k_record_and_edge_cases():
    pi, s, (c, t) = _tables(2)
    x = np.random.default_rng(2).standard_normal((6, D))
    x[1] = 0.0
    x[2, 7] = np.nan
    rec = quant.compress_k(x, pi, s, c, t)
    # norms
    assert np.allclose(rec["norm"][[0, 3]], np.linalg.norm(x[[0, 3]], axis=1))
    # residual norm equals |x - x~|
    xt = quant.dequantize_mse(rec["idx"], rec["norm"], pi, c)
    assert abs(rec["rnorm"][0] - np.linalg.norm(x[0] - xt[0])) < 1e-12
    # residual is orthogonal-ish: |r|^2 = |x|^2 - 2<x,x~> + |x~|^2
    # zero vector: norm 0, upper-middle cell, all signs 1, residual 0
    assert rec["norm"][1] == 0 and rec["rnorm"][1] == 0
    assert np.all(rec["idx"][1] == len(c) // 2) and np.all(rec["sign"][1] == 1)
    # NaN propagates: NaN norms, codes 0, signs 0
    assert np.isnan(rec["norm"][2]) and np.isnan(rec["rnorm"][2])
    assert np.all(rec["idx"][2] == 0) and np.all(rec["sign"][2] == 0)
    # sign bits are the signs of S r
    r = x[0] - xt[0]
    assert np.array_equal(rec["sign"][0], (s @ r >= 0).astype(np.uint8))


def test_compress_into_cache_roundtrip():
    fmt = quant.Format(D, 3, 2)
    pi, s = rotation.make_rotations(D, 42)
    cbk, cbv = codebook.codebook(D, 2), codebook.codebook(D, 2)
    cache = quant.empty_cache(fmt, 2, 64)
    rs = np.random.default_rng(0)
    k = rs.standard_normal((40, 2, D))
    v = rs.standard_normal((40, 2, D))
    slots = np.arange(40) + 3
    out = quant.compress_into(cache, k, v, slots, pi, s, cbk, cbv)
    for h in range(2):
        kp, vals = quant.dequantize_cache(cache, pi, cbk, cbv, h, slots)
        assert np.allclose(kp["xt"], quant.dequantize_mse(out[("k", h)]["idx"], out[("k", h)]["norm"].astype(np.float32), pi, cbk[0]))
        assert np.allclose(vals, quant.dequantize_mse(out[("v", h)]["idx"], out[("v", h)]["norm"].astype(np.float32), pi, cbv[0]))
    # untouched slots stay zero
    assert np.all(cache["k_idx"][:, :3] == 0) and np.all(cache["k_norm"][:, 43:] == 0)
    vfull = quant.unpack_v_blocks(cache["v_idx"][0], 2)
    assert np.all(vfull[:3] == 0) and np.all(vfull[43:] == 0)
