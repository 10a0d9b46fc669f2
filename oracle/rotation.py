"""Random rotation Pi and QJL sketch matrix S for one layer.

"TurboQuant QJL投影深度剖析" §二 step 1: the unit vector x/||x|| is multiplied
by a random orthogonal matrix Pi obtained from a QR decomposition; a 128x128
matrix takes 64 KB, so it is stored in fp32.  §二 step 3: the residual is
projected with a random Gaussian matrix S.  §六: each layer seeds its own
Pi/S with 42 + 7 * layer.

Readings (the pages are silent):
  * Pi = Q * diag(sign(R_ii)) for the QR decomposition G = Q R of the d x d
    matrix of normals 0 .. d*d-1 (Mezzadri 2007: this makes Pi Haar-distributed
    and the decomposition unique).  Convention y = Pi x, so the forward-rotated
    query of §六 ("q @ Pi^T" for row vectors) is Pi q.
  * S[i][j] = normal d*d + i*d + j of the same stream, N(0, 1) entries, d rows.
    The MLX write-up calls the QJL projection "orthogonal", the QJL page says
    Gaussian; only Gaussian rows make sqrt(pi/2)/d the unbiased constant.
  * Both are stored as fp32 (the 64 KB figure); the oracle keeps the float64
    originals for its own checks and computes with the fp32-stored values
    widened to float64.
"""
import numpy as np

from . import rng


def gaussian_matrices(d: int, seed: int):
    g = rng.normals(seed, d * d, 0).reshape(d, d)
    s = rng.normals(seed, d * d, d * d).reshape(d, d)
    return g, s


def haar_from_gaussian(g: np.ndarray) -> np.ndarray:
    """Q * diag(sign(diag R)) for G = QR (numpy/LAPACK Householder QR)."""
    q, r = np.linalg.qr(g)
    sgn = np.sign(np.diag(r))
    sgn[sgn == 0] = 1.0
    return q * sgn[None, :]


def make_rotations(d: int, seed: int, as_stored: bool = True):
    """Return (Pi, S) for dimension d and seed.  With as_stored=True both are
    rounded to fp32 (the stored precision) and returned as float64 arrays."""
    g, s = gaussian_matrices(d, seed)
    pi = haar_from_gaussian(g)
    if as_stored:
        return (pi.astype(np.float32).astype(np.float64),
                s.astype(np.float32).astype(np.float64))
    return pi, s


def layer_rotations(d: int, layer: int, as_stored: bool = True):
    return make_rotations(d, rng.layer_seed(layer), as_stored)
