"""Helpers shared by the GPU parity tests: build oracle caches for a workload,
move packed planes between the oracle layout and the device, and compare
codes with the near-boundary allowance.

Test infrastructure: it calls the oracle and the HIP library side by side.
Every expected value comes from the oracle on the seeded inputs.  The one
place where the device's output selects what is expected: a key code that
differs from the oracle's is first checked to be a valid alternative (its
coordinate lies within 1e-6 of the boundary between the two codes); the
oracle then computes that token's residual, signs and residual norm from the
codes with the alternative taken (both records are correct encodings of the
key, and the residual of each is unique).
"""
import math
from typing import Dict, List, Tuple

import numpy as np

import workloads as wl
from oracle import attention, codebook, quant, rotation

D = 128
NEAR = 1e-6          # a decision within this distance of its threshold may differ
MAX_MISMATCH_RATE = 1e-5


def layer_format(w: wl.Workload, layer: int) -> quant.Format:
    mode = w.modes()[layer]
    if mode == wl.MODE_TQ:
        return quant.Format(D, w.k_bits, w.v_bits)
    if mode == wl.MODE_KF16:
        return quant.Format(D, 0, w.v_bits)
    return quant.Format(D, 0, 0)


def layer_groups(w: wl.Workload) -> List[Tuple[quant.Format, List[int]]]:
    """Consecutive layers that share a storage format."""
    groups: List[Tuple[quant.Format, List[int]]] = []
    for layer in range(w.n_layers):
        f = layer_format(w, layer)
        if groups and groups[-1][0] == f:
            groups[-1][1].append(layer)
        else:
            groups.append((f, [layer]))
    return groups


def tq_format(f: quant.Format):
    import kv_cache_quantization_norm_amd as tq
    return tq.make_format(f.d, f.k_bits, f.v_bits)


def slots_of(w: wl.Workload):
    starts, lens, cap = wl.seq_layout(w)
    slots = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lens)]).astype(np.int64)
    return starts, lens, max(cap, 32), slots


def oracle_tables(fmt: quant.Format, layer: int):
    pi, s = rotation.layer_rotations(D, layer)
    cbk = codebook.table_codebook(D, fmt.k_mse_bits) if fmt.k_bits else None
    cbv = codebook.table_codebook(D, fmt.v_bits) if fmt.v_bits else None
    return pi, s, cbk, cbv


def oracle_compress_layer(w: wl.Workload, layer: int, fmt: quant.Format, k, v, slots, capacity):
    pi, s, cbk, cbv = oracle_tables(fmt, layer)
    cache = quant.empty_cache(fmt, w.n_kv_heads, capacity)
    details = quant.compress_into(cache, k.astype(np.float64), v.astype(np.float64), slots, pi, s, cbk, cbv)
    details["keys"] = np.asarray(k, np.float64)
    return cache, details


PLANE_DTYPES = {"k_idx": np.uint8, "k_sign": np.uint8, "k_norm": np.float32, "k_rnorm": np.float32,
                "k_f16": np.float16, "v_idx": np.uint8, "v_norm": np.float32, "v_f16": np.float16}


def upload_cache(caches: List[dict], fmt: quant.Format, device="cuda"):
    """Device cache holding the given per-layer oracle caches."""
    import torch
    import kv_cache_quantization_norm_amd as tq
    h, cap = caches[0]["n_kv_heads"], caches[0]["capacity"]
    dev = tq.Cache.allocate(tq_format(fmt), len(caches), h, cap, device)
    for name, t in dev.planes.items():
        if t is None:
            continue
        host = np.stack([c[name] for c in caches]).reshape(-1)
        if host.dtype == np.float16:
            t.copy_(torch.from_numpy(host.view(np.int16)).view(torch.float16))
        else:
            t.copy_(torch.from_numpy(np.ascontiguousarray(host)))
    return dev


def download_cache(dev, fmt: quant.Format) -> List[dict]:
    """Per-layer oracle-layout copies of a device cache."""
    out = []
    shapes = quant.empty_cache(fmt, dev.n_kv_heads, dev.capacity)
    host = {}
    for name, t in dev.planes.items():
        if t is None:
            continue
        a = t.cpu().numpy()
        host[name] = a.reshape((dev.n_layers,) + shapes[name].shape)
    for l in range(dev.n_layers):
        c = dict(fmt=fmt, n_kv_heads=dev.n_kv_heads, capacity=dev.capacity)
        for name, a in host.items():
            c[name] = a[l]
        out.append(c)
    return out


def near_boundary(y: np.ndarray, boundaries) -> np.ndarray:
    t = np.asarray(boundaries, np.float64)
    return np.min(np.abs(np.asarray(y, np.float64)[..., None] - t), axis=-1) < NEAR


def alternative_codes(ora_idx: np.ndarray, gpu_idx: np.ndarray, y: np.ndarray, boundaries) -> np.ndarray:
    """Codes of the tokens whose device codes differ from the oracle's, with
    every differing coordinate checked to be a valid alternative: the two
    codes are neighbours and the rotated coordinate lies within NEAR of the
    boundary between them.  Returns the codes with the alternatives taken."""
    t = np.asarray(boundaries, np.float64)
    bad = gpu_idx != ora_idx
    lo = np.minimum(gpu_idx, ora_idx).astype(np.int64)
    assert np.all(np.abs(gpu_idx[bad].astype(np.int64) - ora_idx[bad].astype(np.int64)) == 1), \
        "a code differs from the oracle's by more than one cell"
    # boundary between cells lo and lo + 1 is t[lo]
    assert np.all(np.abs(np.asarray(y, np.float64)[bad] - t[lo[bad]]) < NEAR), "code mismatch away from a boundary"
    alt = ora_idx.copy()
    alt[bad] = gpu_idx[bad]
    return alt


def compare_layer(gpu: dict, ora: dict, details: Dict, fmt: quant.Format, slots: np.ndarray,
                  layer: int) -> Dict[str, int]:
    """Checks one layer's device planes against the oracle's compression of
    the same inputs.  details: the per-head results of quant.compress_into
    plus "keys", the inputs [n][H][d] (float64, row i at slot slots[i]), used
    for the records of tokens with an alternative key code.  Returns counts:
    decisions compared (key codes, sign bits, value codes) and mismatches of
    each."""
    pi, s, cbk, cbv = oracle_tables(fmt, layer)
    keys = details.get("keys")
    stats = dict(coords=0, k_mismatch=0, s_mismatch=0, v_mismatch=0, tokens_alt_codes=0)
    h_n = ora["n_kv_heads"]
    for h in range(h_n):
        if fmt.k_bits > 0:
            det = details[("k", h)]
            gi = quant.unpack_bits(gpu["k_idx"][h, slots], fmt.k_mse_bits, D)
            bad = gi != det["idx"]
            idx = det["idx"]
            sign, rnorm, sr_rel = det["sign"], det["rnorm"], det["sr_rel"]
            if bad.any():
                idx = alternative_codes(det["idx"], gi, det["y"], cbk[1])
                rows = np.nonzero(bad.any(axis=1))[0]
                assert keys is not None, "tokens with alternative codes need the keys"
                a_sign, a_rnorm, a_sr = quant.residual_sketch(keys[rows, h], idx[rows], det["norm"][rows], pi, s,
                                                              cbk[0])
                sign, rnorm, sr_rel = sign.copy(), rnorm.copy(), sr_rel.copy()
                sign[rows], rnorm[rows], sr_rel[rows] = a_sign, a_rnorm, a_sr
                stats["tokens_alt_codes"] += len(rows)
            stats["k_mismatch"] += int(bad.sum())
            stats["coords"] += 2 * bad.size   # codes and sign bits
            # norms
            np.testing.assert_allclose(gpu["k_norm"][h, slots], det["norm"], rtol=1e-6, atol=1e-30)
            # residual norm: the oracle's, for the codes compared
            np.testing.assert_allclose(gpu["k_rnorm"][h, slots], rnorm, rtol=2e-6, atol=1e-6 * det["norm"].max())
            # sign bits: exact except where (S r)_j / ||x|| is within NEAR of zero
            gs = quant.unpack_bits(gpu["k_sign"][h, slots], 1, D)
            sbad = gs != sign
            if sbad.any():
                assert np.all(np.abs(sr_rel[sbad]) < NEAR), "sign mismatch away from zero"
            stats["s_mismatch"] += int(sbad.sum())
            if not bad.any() and not sbad.any():
                assert np.array_equal(gpu["k_idx"][h, slots], ora["k_idx"][h, slots])
                assert np.array_equal(gpu["k_sign"][h, slots], ora["k_sign"][h, slots])
        else:
            assert np.array_equal(gpu["k_f16"][h, slots].view(np.uint16), ora["k_f16"][h, slots].view(np.uint16))
        if fmt.v_bits > 0:
            det = details[("v", h)]
            gv = quant.unpack_v_blocks(gpu["v_idx"][h], fmt.v_bits)[slots]
            bad = gv != det["idx"]
            if bad.any():
                alternative_codes(det["idx"], gv, det["y"], cbv[1])
            stats["v_mismatch"] += int(bad.sum())
            stats["coords"] += bad.size
            np.testing.assert_allclose(gpu["v_norm"][h, slots], det["norm"], rtol=1e-6, atol=1e-30)
        else:
            gv = quant.f16_v_unblock(gpu["v_f16"][h])[slots].view(np.uint16)
            ov = quant.f16_v_unblock(ora["v_f16"][h])[slots].view(np.uint16)
            assert np.array_equal(gv, ov)
    return stats


def mismatch_rate(stats: Dict[str, int]) -> float:
    """(key code + sign bit + value code mismatches) / decisions compared."""
    if not stats["coords"]:
        return 0.0
    return (stats["k_mismatch"] + stats["s_mismatch"] + stats["v_mismatch"]) / stats["coords"]


def check_logits(gpu_logits: np.ndarray, ora_logits: Dict, lens, hq, tol=1e-3):
    """|dl_t| <= tol * max_t |l_t| per query row.  Returns the worst ratio."""
    worst, where = 0.0, None
    for b, n in enumerate(lens):
        for h in range(hq):
            ref = ora_logits[(b, h)]
            if n == 0:
                continue
            got = gpu_logits[b, h, :n]
            scale = np.max(np.abs(ref))
            err = np.max(np.abs(got - ref))
            if err / scale > worst:
                worst, where = err / scale, (b, h, n, float(scale), float(err))
    assert worst <= tol, f"logit error {worst:.3e} of the row maximum exceeds {tol} at (b, h, len, max, err) {where}"
    return worst


def check_outputs(gpu_out: np.ndarray, ora_out: np.ndarray, tol=2e-3):
    err = float(np.max(np.abs(gpu_out.astype(np.float64) - ora_out)))
    assert err <= tol, f"output max-abs error {err:.3e} exceeds {tol}"
    return err


def sanitize_near_boundary(fmt: quant.Format, layer: int, k: np.ndarray, v: np.ndarray,
                           heads=None) -> Tuple[np.ndarray, np.ndarray, int]:
    """Zero the key and value of every (token, head) whose oracle compression
    has a decision within NEAR of its threshold (a code, or a QJL sign).

    Such a decision may legitimately go either way, and one flipped key code
    changes that token's whole residual sketch, so end-to-end outputs are only
    unique away from these inputs.  The flags come from the oracle alone; a zero
    vector compresses deterministically on both sides.  Returns the new arrays
    and the number of (token, head) pairs zeroed."""
    pi, s, cbk, cbv = oracle_tables(fmt, layer)
    k = k.copy()
    v = v.copy()
    zeroed = 0
    for h in (range(k.shape[1]) if heads is None else heads):
        flag = np.zeros(k.shape[0], bool)
        if fmt.k_bits > 0:
            rec = quant.compress_k(k[:, h].astype(np.float64), pi, s, *cbk)
            flag |= near_boundary(rec["y"], cbk[1]).any(axis=1)
            flag |= (np.abs(rec["sr_rel"]) < NEAR).any(axis=1)
        if fmt.v_bits > 0:
            _, _, y = quant.compress_v(v[:, h].astype(np.float64), pi, *cbv, return_y=True)
            flag |= near_boundary(y, cbv[1]).any(axis=1)
        k[flag, h] = 0.0
        v[flag, h] = 0.0
        zeroed += int(flag.sum())
    return k, v, zeroed
