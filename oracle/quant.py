"""TurboQuant compression of keys, MSE-only compression of values, the packed
cache layout, and the unbiased inner-product estimator.

Pages:
  * "TurboQuant QJL投影深度剖析" §二: a key x is compressed by (1) storing ||x||
    and rotating x/||x|| with Pi, (2) quantising every rotated coordinate with
    the (b-1)-bit Lloyd-Max codebook, (3) forming the residual r = x - x~
    against the original x, projecting it with the Gaussian S, keeping only
    the signs (d sign bits packed into d/8 bytes) plus ||r||.
    §五: the ProdQuantized record is (MSE indices, QJL sign bytes, ||r||, ||x||),
    all bit-packed; the inner product estimate is
    <y, x~> + ||r|| * sqrt(pi/2)/d * <S y, signs> with expectation <y, x>.
  * MLX write-up, 背景: K uses the full TurboQuant (Algorithm 2, b-1 MSE bits +
    1 QJL bit), V the MSE-only TurboQuantMSE (Algorithm 1, b bits).
    直接构造缓存: key_bits = 0 keeps K in fp16.

Readings (the pages are silent or loose):
  * The decision for a coordinate is idx = #{k : y >= t_k} (ties go to the
    upper cell), taken in fp32, the storage precision of the rotation and of
    the boundary table: y is computed in float64 and rounded to fp32 before the
    comparison with the fp32 boundaries.
  * x~ = ||x|| * Pi^T c[idx]; r = x - x~ in the original space.  The sign bit of
    coordinate j is 1 when (S r)_j >= 0 (a zero projection counts as +1).
  * A zero vector has norm 0, rotated coordinates 0 (so every index is the
    upper-middle cell), residual 0, all sign bits 1 and residual norm 0.
  * Norms are stored as fp32.
  * Packing (the pages only say "bit-packed"): codes are little-endian,
    least-significant-bit first.
      K codes  [head][slot][d*m/8 bytes]: coordinate j of a token occupies bits
               [j*m, (j+1)*m) of its record (m = k_bits - 1).
      K signs  [head][slot][d/8 bytes]: coordinate j at bit j.
      V codes  [head][slot/32][d][4*b bytes]: slots are grouped in blocks of 32;
               for each coordinate j of a block, the 32 codes of the block's
               slots are packed together, slot p of the block at bits
               [p*b, (p+1)*b).  (This coordinate-major grouping is a storage
               choice of this implementation; it carries the same bits.)
      fp16 K   [head][slot][d]; fp16 V [head][slot/32][d][32] (same grouping).
    Slots not written hold zero bytes.
"""
import math
from dataclasses import dataclass

import numpy as np

VBLOCK = 32  # slots per V block


@dataclass(frozen=True)
class Format:
    d: int = 128
    k_bits: int = 4   # 0 = fp16 keys; else (k_bits - 1) MSE bits + 1 QJL bit
    v_bits: int = 4   # 0 = fp16 values; else MSE-only bits

    @property
    def k_mse_bits(self) -> int:
        return self.k_bits - 1 if self.k_bits > 0 else 0

    def k_record_bytes(self) -> int:
        """Algorithmic bytes of one key record (codes + signs + two fp32 norms)."""
        if self.k_bits == 0:
            return 2 * self.d
        return self.d * self.k_mse_bits // 8 + self.d // 8 + 8

    def v_record_bytes(self) -> int:
        if self.v_bits == 0:
            return 2 * self.d
        return self.d * self.v_bits // 8 + 4


def kappa(d: int) -> float:
    """QJL constant sqrt(pi/2)/d (QJL page, §四 and §六)."""
    return math.sqrt(math.pi / 2.0) / d


def decide(y: np.ndarray, boundaries: np.ndarray) -> np.ndarray:
    """Lloyd-Max cell index #{k : y >= t_k}, decided in fp32."""
    y32 = np.asarray(y, np.float64).astype(np.float32)
    t32 = np.asarray(boundaries, np.float64).astype(np.float32)
    return np.sum(y32[..., None] >= t32, axis=-1).astype(np.uint8)


def _normalise(x: np.ndarray):
    x = np.asarray(x, np.float64)
    n = np.linalg.norm(x, axis=-1)
    safe = np.where(n > 0, n, 1.0)
    xhat = np.where((n > 0)[..., None], x / safe[..., None], 0.0)
    return n, xhat


def compress_v(x: np.ndarray, pi: np.ndarray, centroids, boundaries, return_y: bool = False):
    """MSE-only (PolarQuant) compression of rows of x [N, d].
    Returns (idx uint8 [N, d], norm float64 [N]) and, with return_y, the
    rotated unit vectors y (for locating coordinates near a boundary)."""
    n, xhat = _normalise(x)
    y = xhat @ pi.T                       # y = Pi x/||x||, one row per vector
    # NaN input: keep y NaN so the decision gives code 0 as in IEEE compares.
    y = np.where(np.isnan(n)[..., None], np.nan, y)
    if return_y:
        return decide(y, boundaries), n, y
    return decide(y, boundaries), n


def residual_sketch(x: np.ndarray, idx: np.ndarray, n: np.ndarray, pi: np.ndarray, s: np.ndarray, centroids):
    """QJL page §二 step 3 for rows of x [N, d] whose codes idx and norms n are
    given: x~ = ||x|| Pi^T c[idx], r = x - x~ (original space), the sign bits
    [(S r)_j >= 0] and ||r||.  Returns (sign uint8 [N, d], rnorm [N],
    S r / ||x|| [N, d])."""
    x = np.asarray(x, np.float64)
    xt = np.asarray(n, np.float64)[..., None] * (np.asarray(centroids)[idx] @ pi)   # ||x|| Pi^T c[idx]
    r = x - xt
    sr = r @ s.T                                                                    # S r
    sign = (sr >= 0).astype(np.uint8)
    rnorm = np.linalg.norm(r, axis=-1)
    # S r / ||x|| is returned for locating sign decisions near zero.
    with np.errstate(invalid="ignore", divide="ignore"):
        sr_rel = sr / np.where(n > 0, n, 1.0)[..., None]
    return sign, rnorm, sr_rel


def compress_k(x: np.ndarray, pi: np.ndarray, s: np.ndarray, centroids, boundaries):
    """TurboQuantProd compression of rows of x [N, d] with a (k_bits-1)-bit
    codebook.  Returns dict(idx, sign (0/1 uint8), norm, rnorm) and, for
    locating decisions near a boundary, y (the rotated unit vectors) and
    sr_rel (S r / ||x||)."""
    x = np.asarray(x, np.float64)
    idx, n, y = compress_v(x, pi, centroids, boundaries, return_y=True)
    sign, rnorm, sr_rel = residual_sketch(x, idx, n, pi, s, centroids)
    return dict(idx=idx, sign=sign, norm=n, rnorm=rnorm, y=y, sr_rel=sr_rel)


def dequantize_mse(idx, norm, pi, centroids):
    """||x|| Pi^T c[idx] for rows."""
    return np.asarray(norm, np.float64)[..., None] * (np.asarray(centroids)[idx] @ pi)


def estimate_inner(y: np.ndarray, rec: dict, pi, s, centroids) -> np.ndarray:
    """Unbiased estimate of <y, x> from a key record (QJL page, §五):
    <y, x~> + ||r|| sqrt(pi/2)/d <S y, 2*sign - 1>.  y: [d] or [M, d]; returns
    [..., N]."""
    d = pi.shape[0]
    xt = dequantize_mse(rec["idx"], rec["norm"], pi, centroids)
    signs = 2.0 * rec["sign"].astype(np.float64) - 1.0
    y = np.asarray(y, np.float64)
    sy = y @ s.T
    return y @ xt.T + kappa(d) * (sy @ signs.T) * rec["rnorm"]


# ----------------------------------------------------------------------------
# Packing


def pack_bits(codes: np.ndarray, m: int) -> np.ndarray:
    """Pack the last axis of `codes` (values < 2**m) LSB-first: element j at
    bits [j*m, (j+1)*m).  The last axis length times m must be a multiple of 8."""
    codes = np.asarray(codes, np.uint64)
    n = codes.shape[-1]
    assert (n * m) % 8 == 0
    bits = ((codes[..., :, None] >> np.arange(m, dtype=np.uint64)) & np.uint64(1)).astype(np.uint8)
    bits = bits.reshape(codes.shape[:-1] + (n * m,))
    return np.packbits(bits, axis=-1, bitorder="little")


def unpack_bits(packed: np.ndarray, m: int, n: int) -> np.ndarray:
    bits = np.unpackbits(np.asarray(packed, np.uint8), axis=-1, bitorder="little")
    bits = bits[..., : n * m].reshape(packed.shape[:-1] + (n, m)).astype(np.uint64)
    return np.sum(bits << np.arange(m, dtype=np.uint64), axis=-1).astype(np.uint8)


def pack_v_blocks(idx: np.ndarray, b: int) -> np.ndarray:
    """idx [S, d] (S a multiple of 32) -> [S/32, d, 4*b] bytes: the 32 codes of
    a block for one coordinate packed slot-by-slot."""
    s_, d = idx.shape
    assert s_ % VBLOCK == 0
    blk = idx.reshape(s_ // VBLOCK, VBLOCK, d).transpose(0, 2, 1)   # [blk][j][p]
    return pack_bits(blk, b)


def unpack_v_blocks(packed: np.ndarray, b: int) -> np.ndarray:
    nb, d, _ = packed.shape
    blk = unpack_bits(packed, b, VBLOCK)                              # [blk][j][p]
    return blk.transpose(0, 2, 1).reshape(nb * VBLOCK, d)


def f16_v_blocks(v: np.ndarray) -> np.ndarray:
    s_, d = v.shape
    return np.asarray(v, np.float16).reshape(s_ // VBLOCK, VBLOCK, d).transpose(0, 2, 1).copy()


def f16_v_unblock(vb: np.ndarray) -> np.ndarray:
    nb, d, _ = vb.shape
    return vb.transpose(0, 2, 1).reshape(nb * VBLOCK, d)


# ----------------------------------------------------------------------------
# The packed cache of one layer


def empty_cache(fmt: Format, n_kv_heads: int, capacity: int) -> dict:
    assert capacity % VBLOCK == 0
    d, h = fmt.d, n_kv_heads
    c = dict(fmt=fmt, n_kv_heads=h, capacity=capacity)
    if fmt.k_bits > 0:
        c["k_idx"] = np.zeros((h, capacity, d * fmt.k_mse_bits // 8), np.uint8)
        c["k_sign"] = np.zeros((h, capacity, d // 8), np.uint8)
        c["k_norm"] = np.zeros((h, capacity), np.float32)
        c["k_rnorm"] = np.zeros((h, capacity), np.float32)
    else:
        c["k_f16"] = np.zeros((h, capacity, d), np.float16)
    if fmt.v_bits > 0:
        c["v_idx"] = np.zeros((h, capacity // VBLOCK, d, 4 * fmt.v_bits), np.uint8)
        c["v_norm"] = np.zeros((h, capacity), np.float32)
    else:
        c["v_f16"] = np.zeros((h, capacity // VBLOCK, d, VBLOCK), np.float16)
    return c


def compress_into(cache: dict, k: np.ndarray, v: np.ndarray, slots: np.ndarray,
                  pi, s, cb_k, cb_v) -> dict:
    """Compress keys/values [n][H][d] and write them at `slots` (int [n]).
    cb_k / cb_v are (centroids, boundaries) pairs (ignored for fp16 planes).
    Returns the unpacked per-token results for inspection."""
    fmt: Format = cache["fmt"]
    n, h, d = k.shape
    slots = np.asarray(slots, np.int64)
    out = {}
    for hh in range(h):
        if fmt.k_bits > 0:
            rec = compress_k(k[:, hh], pi, s, *cb_k)
            cache["k_norm"][hh, slots] = rec["norm"].astype(np.float32)
            cache["k_rnorm"][hh, slots] = rec["rnorm"].astype(np.float32)
            cache["k_idx"][hh, slots] = pack_bits(rec["idx"], fmt.k_mse_bits)
            cache["k_sign"][hh, slots] = pack_bits(rec["sign"], 1)
            out[("k", hh)] = rec
        else:
            cache["k_f16"][hh, slots] = np.asarray(k[:, hh], np.float16)
        if fmt.v_bits > 0:
            idx, nv, yv = compress_v(v[:, hh], pi, *cb_v, return_y=True)
            cache["v_norm"][hh, slots] = nv.astype(np.float32)
            full = unpack_v_blocks(cache["v_idx"][hh], fmt.v_bits)
            full[slots] = idx
            cache["v_idx"][hh] = pack_v_blocks(full, fmt.v_bits)
            out[("v", hh)] = dict(idx=idx, norm=nv, y=yv)
        else:
            full = f16_v_unblock(cache["v_f16"][hh]).copy()
            full[slots] = np.asarray(v[:, hh], np.float16)
            cache["v_f16"][hh] = f16_v_blocks(full)
    return out


def dequantize_cache(cache: dict, pi, cb_k, cb_v, head: int, slots: np.ndarray):
    """Return (key parts, values) for the given slots of one KV head:
    keys as dict(xt, rnorm, sign_pm) for TurboQuant keys or dict(k) for fp16
    keys; values [n, d] float64."""
    fmt: Format = cache["fmt"]
    d = fmt.d
    slots = np.asarray(slots, np.int64)
    if fmt.k_bits > 0:
        idx = unpack_bits(cache["k_idx"][head, slots], fmt.k_mse_bits, d)
        sign = unpack_bits(cache["k_sign"][head, slots], 1, d)
        norm = cache["k_norm"][head, slots].astype(np.float64)
        kp = dict(xt=dequantize_mse(idx, norm, pi, cb_k[0]),
                  rnorm=cache["k_rnorm"][head, slots].astype(np.float64),
                  sign_pm=2.0 * sign.astype(np.float64) - 1.0)
    else:
        kp = dict(k=cache["k_f16"][head, slots].astype(np.float64))
    if fmt.v_bits > 0:
        vidx = unpack_v_blocks(cache["v_idx"][head], fmt.v_bits)[slots]
        vals = dequantize_mse(vidx, cache["v_norm"][head, slots].astype(np.float64), pi, cb_v[0])
    else:
        vals = f16_v_unblock(cache["v_f16"][head])[slots].astype(np.float64)
    return kp, vals
