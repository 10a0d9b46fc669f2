"""Seeded synthetic KV-cache workloads shared by the oracle tests, the GPU
parity tests and the benchmark.

This module only draws random inputs (keys, values, queries, sequence
lengths) and describes the workload shapes.  It holds none of the TurboQuant
arithmetic: no rotation, codebook, quantiser, packing or attention.  Both the
oracle and the HIP library consume what it produces, so the two sides see
identical arrays.

Workload shapes follow the decode settings discussed on the TurboQuant pages:
head_dim 128, K at b bits = (b-1) Lloyd-Max bits + 1 QJL bit, V MSE-only,
a dense 28-layer GQA-7 model shape, an asymmetric (K fp16, V 4-bit) variant
with the first and last two layers uncompressed, a 262,144-token long-context
scan, and a ragged 16-sequence serving batch plus a 32,768-token prefill.
Where the pages measure on real models and datasets (NIAH, KLD text,
MM-NIAH), these Gaussian generators with per-channel log-normal scales and
outlier channels stand in for real K/V activations.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

HEAD_DIM = 128

# Per-layer storage modes.
MODE_TQ = "tq"        # K TurboQuant (b-1 MSE bits + 1 QJL bit), V MSE-only
MODE_KF16 = "kf16"    # K kept fp16, V MSE-only (asymmetric mode)
MODE_F16 = "f16"      # K and V kept fp16 (uncompressed boundary layers)


@dataclass(frozen=True)
class Workload:
    name: str
    n_layers: int
    n_kv_heads: int
    n_q_heads: int
    seq_lens: Tuple[int, ...]          # one entry per sequence in the batch
    k_bits: int                        # total K bits per coordinate (0 = fp16 K)
    v_bits: int                        # V bits per coordinate (0 = fp16 V)
    dtype: str                         # "f32" | "bf16" | "f16" element type of K/V
    channel_lognormal_sigma: float     # 0 -> unit channel scales
    n_outlier_channels: int            # per (layer, head, K/V)
    outlier_scale: float
    data_seed: int = 0
    head_dim: int = HEAD_DIM
    layer_modes: Tuple[str, ...] = ()  # empty -> all MODE_TQ (or derived from bits)
    prefill_tokens: int = 0            # bulk-compress prefill measured with the decode
    single_stream: bool = False        # draw K, V, q from one default_rng(data_seed) stream

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    def modes(self) -> Tuple[str, ...]:
        if self.layer_modes:
            return self.layer_modes
        mode = MODE_TQ if self.k_bits > 0 else (MODE_KF16 if self.v_bits > 0 else MODE_F16)
        return tuple(mode for _ in range(self.n_layers))

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def _asym_modes(n_layers: int, n_edge: int = 2) -> Tuple[str, ...]:
    return tuple(MODE_F16 if (l < n_edge or l >= n_layers - n_edge) else MODE_KF16
                 for l in range(n_layers))


def ragged_lengths(n_seq: int, lo: int, hi: int, seed: int = 0) -> Tuple[int, ...]:
    """Sequence lengths uniform on the integers [lo, hi] (inclusive)."""
    rng = np.random.default_rng(seed)
    return tuple(int(v) for v in rng.integers(lo, hi, size=n_seq, endpoint=True))


# The five workloads.  W1 is small enough for the oracle to finish in seconds.
W1 = Workload("w1_single_head_t1024", n_layers=1, n_kv_heads=1, n_q_heads=1,
              seq_lens=(1024,), k_bits=3, v_bits=2, dtype="f32",
              channel_lognormal_sigma=0.0, n_outlier_channels=0, outlier_scale=1.0,
              single_stream=True)
W2 = Workload("w2_dense28L_gqa7_t8192_k4v4", n_layers=28, n_kv_heads=4, n_q_heads=28,
              seq_lens=(8192,), k_bits=4, v_bits=4, dtype="bf16",
              channel_lognormal_sigma=0.5, n_outlier_channels=2, outlier_scale=10.0)
W3 = Workload("w3_dense28L_asym_kf16_v4_t32768", n_layers=28, n_kv_heads=4, n_q_heads=28,
              seq_lens=(32768,), k_bits=0, v_bits=4, dtype="bf16",
              channel_lognormal_sigma=0.5, n_outlier_channels=2, outlier_scale=10.0,
              layer_modes=_asym_modes(28))
W4 = Workload("w4_longctx_h8_gqa8_t262144_k3v2", n_layers=1, n_kv_heads=8, n_q_heads=64,
              seq_lens=(262144,), k_bits=3, v_bits=2, dtype="bf16",
              channel_lognormal_sigma=0.5, n_outlier_channels=0, outlier_scale=1.0)
W5 = Workload("w5_ragged16_h8_gqa8_k4v4_prefill32768", n_layers=1, n_kv_heads=8, n_q_heads=64,
              seq_lens=ragged_lengths(16, 4096, 32768, seed=0), k_bits=4, v_bits=4,
              dtype="bf16", channel_lognormal_sigma=0.5, n_outlier_channels=0,
              outlier_scale=1.0, prefill_tokens=32768)

WORKLOADS = {w.name: w for w in (W1, W2, W3, W4, W5)}
BY_SHORT = {"w1": W1, "w2": W2, "w3": W3, "w4": W4, "w5": W5}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32 so both sides can upload identical values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # 32-bit arithmetic: only NaN / Inf bit patterns can wrap, and those are
    # restored below.
    with np.errstate(over="ignore"):
        rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)) << np.uint32(16)
    out = rounded.view(np.float32)
    # Leave NaN/Inf untouched.
    bad = ~np.isfinite(a)
    if bad.any():
        out = out.copy()
        out[bad] = a[bad]
    return out


def round_to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float32).astype(np.float16).astype(np.float32)
    raise ValueError(dtype)


def _layer_rng(w: Workload, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([w.data_seed, layer, stream])


def channel_scales(w: Workload, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-(head, channel) standard deviations for K and V of one layer:
    log-normal(0, sigma) with n_outlier_channels distinct channels per head
    multiplied by outlier_scale."""
    rng = _layer_rng(w, layer, 0)
    out = []
    for _ in range(2):  # K then V
        if w.channel_lognormal_sigma > 0:
            s = rng.lognormal(0.0, w.channel_lognormal_sigma, size=(w.n_kv_heads, w.head_dim))
        else:
            s = np.ones((w.n_kv_heads, w.head_dim))
        for h in range(w.n_kv_heads):
            if w.n_outlier_channels:
                ch = rng.choice(w.head_dim, size=w.n_outlier_channels, replace=False)
                s[h, ch] *= w.outlier_scale
        out.append(s.astype(np.float64))
    return out[0], out[1]


def gen_kv(w: Workload, layer: int, n_tokens: Optional[int] = None, token0: int = 0,
           stream: int = 1) -> Tuple[np.ndarray, np.ndarray]:
    """Keys and values [n_tokens][n_kv_heads][head_dim] (float32 holding values
    exactly representable in the workload dtype).

    W1 draws K, V (then q, see gen_q) from default_rng(0) in that order.  The
    other workloads draw N(0,1) per token block from a stream keyed on
    (data_seed, layer, stream, block) so that any token range can be drawn
    without drawing the tokens before it, then scale by channel_scales."""
    total = sum(w.seq_lens)
    if n_tokens is None:
        n_tokens = total - token0
    if w.single_stream:
        rng = np.random.default_rng(w.data_seed)
        k = rng.standard_normal((total, w.n_kv_heads, w.head_dim)).astype(np.float32)
        v = rng.standard_normal((total, w.n_kv_heads, w.head_dim)).astype(np.float32)
        return k[token0:token0 + n_tokens].copy(), v[token0:token0 + n_tokens].copy()
    ks, vs = channel_scales(w, layer)
    blk = 4096
    k = np.empty((n_tokens, w.n_kv_heads, w.head_dim), np.float32)
    v = np.empty_like(k)
    b0, b1 = token0 // blk, (token0 + n_tokens - 1) // blk
    for b in range(b0, b1 + 1):
        rng = np.random.default_rng([w.data_seed, layer, stream, b])
        kb = rng.standard_normal((blk, w.n_kv_heads, w.head_dim), dtype=np.float32)
        vb = rng.standard_normal((blk, w.n_kv_heads, w.head_dim), dtype=np.float32)
        lo = max(token0, b * blk)
        hi = min(token0 + n_tokens, (b + 1) * blk)
        k[lo - token0:hi - token0] = kb[lo - b * blk:hi - b * blk]
        v[lo - token0:hi - token0] = vb[lo - b * blk:hi - b * blk]
    k *= ks[None].astype(np.float32)
    v *= vs[None].astype(np.float32)
    return round_to_dtype(k, w.dtype), round_to_dtype(v, w.dtype)


def gen_q(w: Workload, layer: int) -> np.ndarray:
    """Decode queries [batch][n_q_heads][head_dim], float32 N(0,1)."""
    if w.single_stream:
        rng = np.random.default_rng(w.data_seed)
        total = sum(w.seq_lens)
        rng.standard_normal((total, w.n_kv_heads, w.head_dim))
        rng.standard_normal((total, w.n_kv_heads, w.head_dim))
        return rng.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32)
    rng = _layer_rng(w, layer, 2)
    return rng.standard_normal((w.batch, w.n_q_heads, w.head_dim)).astype(np.float32)


def gen_prefill(w: Workload, layer: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The bulk-compression prefill [prefill_tokens][n_kv_heads][head_dim]."""
    assert w.prefill_tokens > 0
    return gen_kv(w, layer, n_tokens=w.prefill_tokens, token0=0, stream=3)


def seq_layout(w: Workload, align: int = 32) -> Tuple[np.ndarray, np.ndarray, int]:
    """Slot ranges of the sequences inside one layer's cache: each sequence
    starts on a multiple of `align` slots.  Returns (seq_start int64,
    seq_len int32, capacity)."""
    starts, lens = [], []
    pos = 0
    for n in w.seq_lens:
        starts.append(pos)
        lens.append(n)
        pos += (n + align - 1) // align * align
    return np.asarray(starts, np.int64), np.asarray(lens, np.int32), pos


def reduced(w: Workload, seq_lens: Tuple[int, ...], n_layers: Optional[int] = None) -> Workload:
    """The same workload law at a smaller size (for tests the oracle finishes
    in seconds)."""
    nl = n_layers or w.n_layers
    modes = w.layer_modes
    if modes and nl != w.n_layers:
        modes = _asym_modes(nl, min(2, nl // 2)) if nl >= 4 else tuple(modes[:nl])
    return w.with_(seq_lens=tuple(seq_lens), n_layers=nl, layer_modes=modes,
                   name=w.name + f"_reduced_{nl}L_" + "_".join(map(str, seq_lens)))
