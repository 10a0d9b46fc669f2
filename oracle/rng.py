"""Seeded normal stream for the rotation and sketch matrices.

The pages fix only that the rotation comes from the QR decomposition of a
random Gaussian matrix, that the QJL sketch matrix S is Gaussian, and that
each layer uses seed = 42 + 7 * layer ("TurboQuant QJL投影深度剖析", §二 step 1
and step 3, §六 on store.py).  They do not name a generator, so this oracle
uses one counter-based generator from its published definition:

  * SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): output n (n = 0, 1, ...) of seed s is
    mix64(s + (n + 1) * 0x9E3779B97F4A7C15 mod 2^64), where mix64 is the
    variant-13 finaliser z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
    z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31.
  * uniform u_n = ((z_n >> 11) + 0.5) * 2^-53, strictly inside (0, 1);
  * normal N_i = sqrt(-2 ln u_{2i}) * cos(2 pi u_{2i+1})  (Box & Muller 1958,
    cosine branch only; two uniforms per normal).

The matrix of normals for the rotation takes normals 0 .. d*d-1 in row-major
order; the sketch S continues with normals d*d .. 2*d*d-1.
"""
import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def layer_seed(layer: int) -> int:
    """Per-layer seed from the pages (§六, store.py): 42 + 7 * layer."""
    return 42 + 7 * int(layer)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs start .. start+n-1 of SplitMix64 seeded with `seed` (uint64)."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + ctr * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniforms(seed: int, n: int, start: int = 0) -> np.ndarray:
    z = splitmix64(seed, n, start)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normals(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Normals start .. start+n-1 of the stream (float64)."""
    u = uniforms(seed, 2 * n, 2 * start)
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
