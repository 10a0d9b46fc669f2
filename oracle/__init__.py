"""Float64 CPU oracle for TurboQuant KV-cache compression and decode attention
on the packed cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in the graft entry
module and the benchmark's CPU-baseline leg may import anything from this
package.  The product path (the HIP library and its Python binding) never
imports, links or calls it, and it shares no code, tables or constants with
that library: it re-derives the rotation, the sketch matrix, the codebooks
and the packed layout on its own, from the method as the TurboQuant pages
describe it.

Sources (pages, by title and section):
  * "TurboQuant QJL投影深度剖析" (bjdmk.com.cn): §二 three-stage pipeline
    (norm + rotation, Lloyd-Max, QJL residual sketch), §四 the QJL identity,
    §五 the combined unbiased estimator and the ProdQuantized record,
    §六 attention scoring with a forward-rotated query and a pre-sketched query,
    per-layer seed 42 + 7*layer.
  * "TurboQuant MLX 移植" write-up of docs/mlx-port.md (cf-1.com): 背景 —
    PolarQuant (b-1 bits) + QJL (1 bit) for K, MSE-only TurboQuantMSE for V;
    直接构造缓存 — key_bits = 0 keeps K in fp16 (asymmetric mode).

Modules
  rng        SplitMix64 + Box-Muller normal stream (our reading: the pages do
             not name a generator).
  rotation   Pi = Haar orthogonal from QR of a Gaussian; S Gaussian sketch.
  codebook   Lloyd-Max quantiser for the exact coordinate law of a rotated
             unit vector.
  quant      compression of K (TurboQuantProd) and V (MSE-only), the packed
             cache layout, and the inner-product estimator.
  attention  decode attention over a packed cache, by its plain definition
             (dequantise, two-pass softmax) and in the rotated online form.

Every function is pinned by tests under tests/ that check it against what
the pages and mathematics fix; none is "parity unpinned".
"""
from . import rng, rotation, codebook, quant, attention  # noqa: F401
