"""Python binding of libtq, the TurboQuant KV-cache library for MI355X.

Argument marshalling only: every step of compression and decode attention
runs in libtq's HIP kernels (or, for the table generators, its host C++).
PyTorch supplies device memory and the current stream.  The entry points
keep the C names (tq_make_rotations, tq_make_codebook, tq_compress_kv,
tq_decode_attention, tq_score, ...); `Tables` and `Cache` allocate the device
arrays those calls take.

Importing this package fails loudly if libtq.so has not been built; there is
no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_HIP, TQ_ERR_APPEND_TIMEOUT = range(6)
TQ_DTYPE_F32, TQ_DTYPE_BF16, TQ_DTYPE_F16 = 0, 1, 2
VBLOCK = 32


class TQError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {status_name(status)}: {detail}")
        self.status = status


class tq_format(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32)]


class tq_tables(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("pi", "s", "pi_s", "k_centroids", "k_boundaries", "v_centroids", "v_boundaries")] + \
               [("k_operand_scale", ctypes.c_float), ("v_operand_scale", ctypes.c_float)]


class tq_cache(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("capacity", ctypes.c_int64)] + \
               [(n, ctypes.c_void_p) for n in
                ("k_idx", "k_sign", "k_norm", "k_rnorm", "k_f16", "v_idx", "v_norm", "v_f16")]


class tq_step_part(ctypes.Structure):
    _fields_ = [("fmt", ctypes.POINTER(tq_format)), ("tables", ctypes.POINTER(tq_tables)),
                ("cache", ctypes.POINTER(tq_cache)), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("layer0", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("q", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"libtq.so is not built ({path}); run __graft_entry__.build() or "
                          "python -m kv_cache_quantization_norm_amd.build")
    # libtq.so needs libamdhip64.so.7.  PyTorch ships its own copy of that
    # runtime under a file name the dynamic loader does not match to the
    # soname, so whichever loads first decides: if libtq.so came first the
    # process would hold two HIP runtimes and the second to start sees no
    # device.  Loading torch first makes libtq.so bind to torch's runtime, the
    # one that owns the tensors and streams handed to it.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    fmtp = ctypes.POINTER(tq_format)
    tabp = ctypes.POINTER(tq_tables)
    cachep = ctypes.POINTER(tq_cache)
    sig = {
        "tq_layer_seed": (ctypes.c_uint64, [I32]),
        "tq_make_rotations": (I32, [I32, ctypes.c_uint64, P, P, P]),
        "tq_make_codebook": (I32, [I32, I32, P, P]),
        "tq_fp16_operand_scale": (F32, [P, I32]),
        "tq_cache_plane_bytes": (I32, [fmtp, I32, I32, I64, P]),
        "tq_decode_workspace_bytes": (SZ, [fmtp, I32, I32, I32, I32, I64]),
        "tq_decode_split": (I32, [fmtp, I32, I32, I32, I32, I64, P]),
        "tq_compress_kv": (I32, [fmtp, tabp, cachep, P, P, I32, I32, I32, I64, P, I64, P]),
        "tq_compress_kv_bounded": (I32, [fmtp, tabp, cachep, P, P, I32, I32, I32, I64, P, I64, I32, P]),
        "tq_decode_attention_tail": (I32, [fmtp, tabp, cachep, cachep, P, I32, I32, P, P, I64, P, P, I64, F32, P, P,
                                           SZ, P]),
        "tq_decode_tail_workspace_bytes": (SZ, [fmtp, I32, I32, I32, I32, I64, I64]),
        "tq_decode_attention": (I32, [fmtp, tabp, cachep, P, I32, I32, P, P, I64, F32, P, P, SZ, P]),
        "tq_decode_attention_noalloc": (I32, [fmtp, tabp, cachep, P, I32, I32, P, P, I64, F32, P, P]),
        "tq_score": (I32, [fmtp, tabp, cachep, P, I32, I32, P, P, I64, F32, P, P, SZ, P]),
        "tq_score_multi": (I32, [fmtp, tabp, cachep, P, I32, I32, P, P, I64, F32, P, P, SZ, P]),
        "tq_decode_prepare": (I32, [fmtp, tabp, cachep, P, I32, I32, I64, P, SZ, P]),
        "tq_append_prepare": (I32, [fmtp, tabp, cachep, P, P, I32, I32, I32, I64, P, I64, P, I32, I32, I64, P, SZ,
                                    P]),
        "tq_decode_partials": (I32, [fmtp, tabp, cachep, I32, I32, P, P, I64, F32, P, SZ, P]),
        "tq_decode_combine": (I32, [fmtp, tabp, cachep, I32, I32, I64, P, P, SZ, P]),
        "tq_decode_attend": (I32, [fmtp, tabp, cachep, I32, I32, P, P, I64, F32, P, P, SZ, P]),
        "tq_stream_read_probe": (I32, [P, SZ, P, I32, P]),
        "tq_decode_step": (I32, [fmtp, tabp, cachep, P, P, I32, I32, I32, I64, P, I64, P, I32, I32, P, P, I64, F32, P,
                                 P, SZ, P]),
        "tq_decode_step_parts": (I32, [ctypes.POINTER(tq_step_part), I32, I32, I64, P, I64, I32, I32, P, P, I64,
                                       F32, P]),
        "tq_decode_attend_parts": (I32, [ctypes.POINTER(tq_step_part), I32, I32, I32, P, P, I64, F32, P]),
        "tq_decode_step_check": (I32, [fmtp, I32, I32, I32, I32, I64, P, SZ, P]),
        "tq_set_append_wait": (I32, [ctypes.c_uint32, I32]),
        "tq_tail_policy": (I32, [I32, P, P, I32, I32, P]),
        "tq_tail_append": (I32, [fmtp, tabp, cachep, P, P, I32, I32, I32, I64, P, I64, P]),
        "tq_tail_flush_workspace_bytes": (SZ, [fmtp, cachep, I32, I32]),
        "tq_tail_flush": (I32, [fmtp, tabp, cachep, cachep, I32, I32, P, P, P, P, SZ, P]),
        "tq_status_string": (ctypes.c_char_p, [I32]),
        "tq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("tq_layer_seed", "tq_make_rotations", "tq_make_codebook", "tq_cache_plane_bytes",
            "tq_decode_workspace_bytes", "tq_decode_split", "tq_compress_kv", "tq_decode_attention", "tq_score",
            "tq_decode_prepare", "tq_decode_partials", "tq_decode_combine", "tq_decode_attend", "tq_decode_step",
            "tq_stream_read_probe",
            "tq_append_prepare",
            "tq_compress_kv_bounded", "tq_decode_attention_tail", "tq_decode_tail_workspace_bytes",
            "tq_decode_attention_noalloc", "tq_decode_step_check", "tq_set_append_wait", "tq_fp16_operand_scale",
            "tq_tail_policy", "tq_tail_append", "tq_tail_flush_workspace_bytes", "tq_tail_flush", "tq_score_multi",
            "tq_decode_step_parts", "tq_decode_attend_parts", "tq_status_string", "tq_last_error")


def status_name(st: int) -> str:
    return _lib.tq_status_string(st).decode()


def _check(st: int, what: str):
    if st != TQ_OK:
        raise TQError(st, what, _lib.tq_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor the binding itself allocated (Tables, Cache),
    a raw integer address, or None; host arrays are refused."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        raise TypeError("a host (numpy) array was passed where the library expects device memory")
    if not t.is_cuda:
        raise ValueError("a host tensor was passed where the library expects device memory")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ----------------------------------------------------------------------------
# Host calls


def tq_layer_seed(layer: int) -> int:
    return int(_lib.tq_layer_seed(layer))


def tq_make_rotations(d: int, seed: int, with_pi_s: bool = True):
    """Returns (pi, s, pi_s) as float32 numpy arrays [d, d] (pi_s None if not asked)."""
    pi = np.empty((d, d), np.float32)
    s = np.empty((d, d), np.float32)
    m = np.empty((d, d), np.float32) if with_pi_s else None
    _check(_lib.tq_make_rotations(d, seed, pi.ctypes.data, s.ctypes.data, m.ctypes.data if m is not None else None),
           "tq_make_rotations")
    return pi, s, m


def tq_make_codebook(d: int, bits: int):
    """Returns (centroids [2^bits], boundaries [2^bits - 1]) float64."""
    c = np.empty(1 << bits, np.float64)
    t = np.empty(max(1, (1 << bits) - 1), np.float64)
    _check(_lib.tq_make_codebook(d, bits, c.ctypes.data, t.ctypes.data), "tq_make_codebook")
    return c, t[: (1 << bits) - 1]


def tq_fp16_operand_scale(centroids) -> float:
    """Scale of a codebook's fp16 decode operands (fp32 centroids, host)."""
    c = np.ascontiguousarray(np.asarray(centroids, np.float32))
    return float(_lib.tq_fp16_operand_scale(c.ctypes.data, len(c)))


def make_format(d: int = 128, k_bits: int = 4, v_bits: int = 4) -> tq_format:
    return tq_format(d, k_bits, v_bits)


PLANES = ("k_idx", "k_sign", "k_norm", "k_rnorm", "k_f16", "v_idx", "v_norm", "v_f16")


def tq_cache_plane_bytes(fmt: tq_format, n_layers: int, n_kv_heads: int, capacity: int) -> List[int]:
    out = (ctypes.c_size_t * 8)()
    _check(_lib.tq_cache_plane_bytes(ctypes.byref(fmt), n_layers, n_kv_heads, capacity, out),
           "tq_cache_plane_bytes")
    return list(out)


def tq_decode_split(fmt: tq_format, n_layers: int, batch: int, n_kv_heads: int, n_q_heads: int,
                    max_seq_len: int) -> dict:
    """The decode work split (see include/tq.h)."""
    out = (ctypes.c_int64 * 5)()
    _check(_lib.tq_decode_split(ctypes.byref(fmt), n_layers, batch, n_kv_heads, n_q_heads, max_seq_len, out),
           "tq_decode_split")
    return dict(zip(("problems", "chunks_per_problem", "chunks_per_wg", "n_workgroups", "pieces_max"), out))


def tq_decode_workspace_bytes(fmt: tq_format, n_layers: int, batch: int, n_kv_heads: int, n_q_heads: int,
                              max_seq_len: int) -> int:
    return int(_lib.tq_decode_workspace_bytes(ctypes.byref(fmt), n_layers, batch, n_kv_heads, n_q_heads,
                                              max_seq_len))


# ----------------------------------------------------------------------------
# Device arrays


@dataclass
class Tables:
    """Device tables for n_layers layers: Pi, S, S Pi^T per layer (fp32) and the
    key / value codebooks (fp32)."""
    fmt: tq_format
    pi: object
    s: object
    pi_s: object
    k_centroids: object
    k_boundaries: object
    v_centroids: object
    v_boundaries: object
    host: dict
    k_operand_scale: float = 1.0
    v_operand_scale: float = 1.0

    @classmethod
    def create(cls, fmt: tq_format, layers: Sequence[int], device="cuda"):
        import torch
        d = fmt.d
        pis, ss, ms = [], [], []
        for layer in layers:
            pi, s, m = tq_make_rotations(d, tq_layer_seed(layer))
            pis.append(pi)
            ss.append(s)
            ms.append(m)
        host = dict(pi=np.stack(pis), s=np.stack(ss), pi_s=np.stack(ms))
        dev = {k: torch.from_numpy(v).to(device) for k, v in host.items()}

        def cb(bits):
            if bits <= 0:
                return None, None
            c, t = tq_make_codebook(d, bits)
            host[f"c{bits}"] = (c, t)
            return (torch.from_numpy(c.astype(np.float32)).to(device),
                    torch.from_numpy(t.astype(np.float32)).to(device) if len(t) else
                    torch.zeros(1, dtype=torch.float32, device=device))

        kc, kb = cb(fmt.k_bits - 1 if fmt.k_bits > 0 else 0)
        vc, vb = cb(fmt.v_bits)
        ks = tq_fp16_operand_scale(host[f"c{fmt.k_bits - 1}"][0]) if fmt.k_bits > 0 else 1.0
        vs = tq_fp16_operand_scale(host[f"c{fmt.v_bits}"][0]) if fmt.v_bits > 0 else 1.0
        return cls(fmt, dev["pi"], dev["s"], dev["pi_s"], kc, kb, vc, vb, host, ks, vs)

    def struct(self) -> tq_tables:
        return tq_tables(*[_ptr(x) for x in (self.pi, self.s, self.pi_s, self.k_centroids, self.k_boundaries,
                                             self.v_centroids, self.v_boundaries)],
                         self.k_operand_scale, self.v_operand_scale)


@dataclass
class Cache:
    """Zero-initialised device planes of a packed cache."""
    fmt: tq_format
    n_layers: int
    n_kv_heads: int
    capacity: int
    planes: dict

    @classmethod
    def allocate(cls, fmt: tq_format, n_layers: int, n_kv_heads: int, capacity: int, device="cuda"):
        import torch
        sizes = tq_cache_plane_bytes(fmt, n_layers, n_kv_heads, capacity)
        planes = {}
        for name, nbytes in zip(PLANES, sizes):
            if nbytes == 0:
                planes[name] = None
                continue
            if name in ("k_norm", "k_rnorm", "v_norm"):
                planes[name] = torch.zeros(nbytes // 4, dtype=torch.float32, device=device)
            elif name in ("k_f16", "v_f16"):
                planes[name] = torch.zeros(nbytes // 2, dtype=torch.float16, device=device)
            else:
                planes[name] = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        return cls(fmt, n_layers, n_kv_heads, capacity, planes)

    def struct(self) -> tq_cache:
        return tq_cache(self.n_layers, self.n_kv_heads, self.capacity,
                        *[_ptr(self.planes[n]) for n in PLANES])

    def nbytes(self) -> int:
        return sum(p.numel() * p.element_size() for p in self.planes.values() if p is not None)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_DTYPE_F32, torch.bfloat16: TQ_DTYPE_BF16, torch.float16: TQ_DTYPE_F16}[t.dtype]


# ----------------------------------------------------------------------------
# Argument checks: the C side takes raw device pointers, so every tensor is
# checked here for being a contiguous device tensor of the dtype and shape the
# call reads or writes (a wrong one would make the kernels read or write out of
# bounds).


def _dev(t, dtypes, shape, name: str) -> int:
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a device torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device (cuda) tensor, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    return t.data_ptr()


def _f32():
    import torch
    return (torch.float32,)


def _kv_types():
    import torch
    return (torch.float32, torch.bfloat16, torch.float16)


def _i64():
    import torch
    return (torch.int64,)


def _i32():
    import torch
    return (torch.int32,)


def _u8():
    import torch
    return (torch.uint8,)


def _kv(fmt: tq_format, cache: Cache, k, v):
    """k, v [n_layers][n_tokens][n_kv_heads][d], same shape and dtype."""
    import torch
    if not isinstance(k, torch.Tensor):
        raise TypeError(f"k: expected a device torch.Tensor, got {type(k).__name__}")
    if k.dim() != 4:
        raise ValueError("k: expected a 4-d tensor [n_layers][n_tokens][n_kv_heads][d]")
    n_layers, n_tokens = int(k.shape[0]), int(k.shape[1])
    shape = (n_layers, n_tokens, cache.n_kv_heads, fmt.d)
    pk = _dev(k, _kv_types(), shape, "k")
    pv = _dev(v, (k.dtype,), shape, "v")
    return pk, pv, n_layers, n_tokens


def _slots(slots, n_tokens: int):
    return None if slots is None else _dev(slots, _i64(), (n_tokens,), "slots")


def _q(fmt: tq_format, cache: Cache, q, name="q"):
    """q [n_layers][batch][n_q_heads][d] float32 with n_layers = cache's."""
    import torch
    if not isinstance(q, torch.Tensor):
        raise TypeError(f"{name}: expected a device torch.Tensor, got {type(q).__name__}")
    if q.dim() != 4:
        raise ValueError(f"{name}: expected a 4-d tensor [n_layers][batch][n_q_heads][d]")
    _, batch, hq, _ = q.shape
    return _dev(q, _f32(), (cache.n_layers, batch, hq, fmt.d), name), int(batch), int(hq)


def _seq(seq_start, seq_len, batch: int, a="seq_start", b="seq_len"):
    return _dev(seq_start, _i64(), (batch,), a), _dev(seq_len, _i32(), (batch,), b)


def _out(fmt: tq_format, cache: Cache, out, batch: int, hq: int):
    return _dev(out, _f32(), (cache.n_layers, batch, hq, fmt.d), "out")


def _ws(workspace):
    p = _dev(workspace, _u8(), None, "workspace")
    return p, workspace.numel()


# ----------------------------------------------------------------------------
# Device calls


def tq_compress_kv(fmt: tq_format, tables: Tables, cache: Cache, k, v, layer0: int = 0, slots=None,
                   slot0: int = 0, stream=None):
    """k, v: contiguous device tensors [n_layers][n_tokens][n_kv_heads][d]
    (float32, bfloat16 or float16); slots: optional device int64 [n_tokens]."""
    pk, pv, n_layers, n_tokens = _kv(fmt, cache, k, v)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_compress_kv(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pk, pv, _dtype_code(k), layer0,
                               n_layers, n_tokens, _slots(slots, n_tokens), slot0, _stream(stream)), "tq_compress_kv")


def tq_compress_kv_bounded(fmt: tq_format, tables: Tables, cache: Cache, k, v, max_workgroups: int, layer0: int = 0,
                           slots=None, slot0: int = 0, stream=None):
    """tq_compress_kv with the bulk kernel held to at most max_workgroups CUs."""
    pk, pv, n_layers, n_tokens = _kv(fmt, cache, k, v)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_compress_kv_bounded(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pk, pv, _dtype_code(k),
                                       layer0, n_layers, n_tokens, _slots(slots, n_tokens), slot0, max_workgroups,
                                       _stream(stream)), "tq_compress_kv_bounded")


def workspace_for(fmt: tq_format, cache: Cache, batch: int, n_q_heads: int, max_seq_len: int, device="cuda"):
    import torch
    nbytes = tq_decode_workspace_bytes(fmt, cache.n_layers, batch, cache.n_kv_heads, n_q_heads, max_seq_len)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def tq_decode_attention(fmt: tq_format, tables: Tables, cache: Cache, q, seq_start, seq_len, max_seq_len: int,
                        out, workspace, scale: float = 0.0, stream=None):
    """q, out: device float32 [n_layers][batch][n_q_heads][d]; seq_start int64 and
    seq_len int32 device tensors [batch]."""
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    po = _out(fmt, cache, out, batch, hq)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_attention(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pq, batch, hq, ps, pl,
                                    max_seq_len, scale, po, pw, nw, _stream(stream)), "tq_decode_attention")


NOALLOC_SCRATCH_BYTES = 64 << 20


def tq_decode_attention_noalloc(fmt: tq_format, tables: Tables, cache: Cache, q, seq_start, seq_len, max_seq_len: int,
                                out, scale: float = 0.0, stream=None):
    """tq_decode_attention with its workspace in the library's static device
    scratch (nothing is allocated; calls that overlap on one GPU race)."""
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    po = _out(fmt, cache, out, batch, hq)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_attention_noalloc(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pq, batch, hq, ps,
                                            pl, max_seq_len, scale, po, _stream(stream)),
           "tq_decode_attention_noalloc")


def tq_decode_prepare(fmt: tq_format, tables: Tables, cache: Cache, q, max_seq_len: int, workspace, stream=None):
    pq, batch, hq = _q(fmt, cache, q)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_prepare(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pq, batch, hq, max_seq_len,
                                  pw, nw, _stream(stream)), "tq_decode_prepare")


def tq_append_prepare(fmt: tq_format, tables: Tables, cache: Cache, k, v, q, max_seq_len: int, workspace,
                      layer0: int = 0, slots=None, slot0: int = 0, stream=None):
    """tq_compress_kv(k, v, ...) then tq_decode_prepare(q, ...), in one launch
    for fewer than 16 tokens."""
    pk, pv, n_layers, n_tokens = _kv(fmt, cache, k, v)
    pq, batch, hq = _q(fmt, cache, q)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_append_prepare(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pk, pv, _dtype_code(k),
                                  layer0, n_layers, n_tokens, _slots(slots, n_tokens), slot0, pq, batch, hq,
                                  max_seq_len, pw, nw, _stream(stream)), "tq_append_prepare")


def tq_decode_step(fmt: tq_format, tables: Tables, cache: Cache, k, v, q, seq_start, seq_len, max_seq_len: int, out,
                   workspace, layer0: int = 0, slots=None, slot0: int = 0, scale: float = 0.0, stream=None):
    """tq_compress_kv(k, v, ...) then tq_decode_attention(q, ...): for a small
    append two launches, the append inside the decode launch."""
    pk, pv, n_layers, n_tokens = _kv(fmt, cache, k, v)
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    po = _out(fmt, cache, out, batch, hq)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_step(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pk, pv, _dtype_code(k), layer0,
                               n_layers, n_tokens, _slots(slots, n_tokens), slot0, pq, batch, hq, ps, pl, max_seq_len,
                               scale, po, pw, nw, _stream(stream)), "tq_decode_step")


@dataclass
class StepPart:
    """One part of tq_decode_step_parts: a cache of one format (its layers),
    the new tokens of its layers [layer0, layer0 + k.shape[0]), its queries,
    outputs and workspace."""
    fmt: tq_format
    tables: "Tables"
    cache: "Cache"
    k: object
    v: object
    q: object
    out: object
    workspace: object
    layer0: int = 0


def tq_decode_step_parts(parts: Sequence[StepPart], seq_start, seq_len, max_seq_len: int, slots=None, slot0: int = 0,
                         scale: float = 0.0, stream=None):
    """tq_decode_step over each part in order, the parts sharing the batch, its
    sequences and the new tokens' slots; two parts whose second is fp16 / fp16
    run their decodes in one launch."""
    if not parts:
        raise ValueError("no parts")
    arr = (tq_step_part * len(parts))()
    keep = []
    shared = None
    for i, p in enumerate(parts):
        pk, pv, n_layers, n_tokens = _kv(p.fmt, p.cache, p.k, p.v)
        pq, batch, hq = _q(p.fmt, p.cache, p.q)
        po = _out(p.fmt, p.cache, p.out, batch, hq)
        pw, nw = _ws(p.workspace)
        mine = (n_tokens, batch, hq, _dtype_code(p.k))
        if shared is None:
            shared = mine
        elif mine != shared:
            raise ValueError(f"part {i}: (tokens, batch, q heads, dtype) {mine} differ from part 0's {shared}")
        tb, cs = p.tables.struct(), p.cache.struct()
        keep += [tb, cs]
        arr[i] = tq_step_part(ctypes.pointer(p.fmt), ctypes.pointer(tb), ctypes.pointer(cs), pk, pv, p.layer0, n_layers,
                              pq, po, pw, nw)
    n_tokens, batch, hq, dtype = shared
    ps, pl = _seq(seq_start, seq_len, batch)
    _check(_lib.tq_decode_step_parts(arr, len(parts), dtype, n_tokens, _slots(slots, n_tokens), slot0, batch, hq, ps, pl,
                                     max_seq_len, scale, _stream(stream)), "tq_decode_step_parts")
    del keep


def tq_decode_attend_parts(parts: Sequence[StepPart], seq_start, seq_len, max_seq_len: int, scale: float = 0.0,
                           stream=None):
    """The decode of tq_decode_step_parts alone, on queries prepared in each
    part's workspace (the parts' k and v are not read and may be None)."""
    if not parts:
        raise ValueError("no parts")
    arr = (tq_step_part * len(parts))()
    keep = []
    shared = None
    for i, p in enumerate(parts):
        pq, batch, hq = _q(p.fmt, p.cache, p.q)
        po = _out(p.fmt, p.cache, p.out, batch, hq)
        pw, nw = _ws(p.workspace)
        if shared is None:
            shared = (batch, hq)
        elif (batch, hq) != shared:
            raise ValueError(f"part {i}: (batch, q heads) {(batch, hq)} differ from part 0's {shared}")
        tb, cs = p.tables.struct(), p.cache.struct()
        keep += [tb, cs]
        arr[i] = tq_step_part(ctypes.pointer(p.fmt), ctypes.pointer(tb), ctypes.pointer(cs), None, None, 0, 0, pq, po,
                              pw, nw)
    batch, hq = shared
    ps, pl = _seq(seq_start, seq_len, batch)
    _check(_lib.tq_decode_attend_parts(arr, len(parts), batch, hq, ps, pl, max_seq_len, scale, _stream(stream)),
           "tq_decode_attend_parts")
    del keep


def tq_decode_step_check(fmt: tq_format, cache: Cache, batch: int, n_q_heads: int, max_seq_len: int, workspace,
                         stream=None):
    """Raises TQError(TQ_ERR_APPEND_TIMEOUT) if a decode wave of the last
    tq_decode_step on `workspace` gave up waiting for the step's append
    (synchronizes the stream)."""
    pw, nw = _ws(workspace)
    _check(_lib.tq_decode_step_check(ctypes.byref(fmt), cache.n_layers, batch, cache.n_kv_heads, n_q_heads,
                                     max_seq_len, pw, nw, _stream(stream)), "tq_decode_step_check")


def tq_set_append_wait(max_polls: int = 1 << 20, extra_groups: int = 0):
    """Test hook: the bounded wait of later tq_decode_step launches."""
    _check(_lib.tq_set_append_wait(max_polls, extra_groups), "tq_set_append_wait")


def tq_stream_read_probe(data, partial, n_workgroups: int, stream=None):
    """Plain streaming read of the device tensor `data` (measurement reference)."""
    import torch
    pd = _dev(data, (data.dtype,) if isinstance(data, torch.Tensor) else (), None, "data")
    pp = _dev(partial, _f32(), (n_workgroups,), "partial")
    _check(_lib.tq_stream_read_probe(pd, data.numel() * data.element_size(), pp, n_workgroups, _stream(stream)),
           "tq_stream_read_probe")


def tail_workspace_for(fmt: tq_format, cache: Cache, batch: int, n_q_heads: int, max_seq_len: int,
                       max_tail_len: int, device="cuda"):
    import torch
    nbytes = int(_lib.tq_decode_tail_workspace_bytes(ctypes.byref(fmt), cache.n_layers, batch, cache.n_kv_heads,
                                                     n_q_heads, max_seq_len, max_tail_len))
    if nbytes == 0:
        raise TQError(TQ_ERR_INVALID_ARG, "tq_decode_tail_workspace_bytes", "invalid sizes")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def tq_tail_policy(packed_len, tail_len, min_compress_tokens: int = 256, keep_recent: int = 16):
    """Host: tokens each sequence moves from its fp16 tail ring into the
    packed cache (multiples of 32), from host int sequences of lengths."""
    pl = np.ascontiguousarray(packed_len, dtype=np.int32)
    tl = np.ascontiguousarray(tail_len, dtype=np.int32)
    if pl.shape != tl.shape or pl.ndim != 1:
        raise ValueError("packed_len and tail_len: 1-d of the same length")
    out = np.zeros(pl.shape, np.int32)
    _check(_lib.tq_tail_policy(len(pl), pl.ctypes.data, tl.ctypes.data, min_compress_tokens, keep_recent,
                               out.ctypes.data), "tq_tail_policy")
    return out


def tq_tail_append(fmt: tq_format, tables: Tables, tail: Cache, k, v, ring_slots, ring_cap: int, layer0: int = 0,
                   stream=None):
    """New tokens into the tail ring (slot p and its mirror p + ring_cap):
    k, v [n_layers][n_tokens][n_kv_heads][d]; ring_slots device int64 [n_tokens]."""
    pk, pv, n_layers, n_tokens = _kv(fmt, tail, k, v)
    ps = _dev(ring_slots, _i64(), (n_tokens,), "ring_slots")
    tb, ts = tables.struct(), tail.struct()
    _check(_lib.tq_tail_append(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(ts), pk, pv, _dtype_code(k), layer0,
                               n_layers, n_tokens, ps, ring_cap, _stream(stream)), "tq_tail_append")


def tail_flush_workspace_for(fmt: tq_format, packed: Cache, batch: int, max_flush: int, device="cuda"):
    import torch
    nbytes = int(_lib.tq_tail_flush_workspace_bytes(ctypes.byref(fmt), ctypes.byref(packed.struct()), batch, max_flush))
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def tq_tail_flush(fmt: tq_format, tables: Tables, packed: Cache, tail: Cache, max_flush: int, tail_pos, n_flush,
                  dst_slot, workspace, stream=None):
    """Moves n_flush[b] tail tokens (from tail slot tail_pos[b]) of each
    sequence into packed slots dst_slot[b] ..; device int64 / int32 / int64 [batch]."""
    import torch
    if not isinstance(tail_pos, torch.Tensor) or tail_pos.dim() != 1:
        raise TypeError("tail_pos: expected a 1-d device int64 tensor")
    batch = int(tail_pos.shape[0])
    pp = _dev(tail_pos, _i64(), (batch,), "tail_pos")
    pn = _dev(n_flush, _i32(), (batch,), "n_flush")
    pd = _dev(dst_slot, _i64(), (batch,), "dst_slot")
    pw, nw = _ws(workspace)
    if tail.n_layers != packed.n_layers or tail.n_kv_heads != packed.n_kv_heads:
        raise ValueError("tail: must have the packed cache's layers and KV heads")
    tb, cs, ts = tables.struct(), packed.struct(), tail.struct()
    _check(_lib.tq_tail_flush(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), ctypes.byref(ts), batch,
                              max_flush, pp, pn, pd, pw, nw, _stream(stream)), "tq_tail_flush")


def tq_decode_attention_tail(fmt: tq_format, tables: Tables, cache: Cache, tail: Cache, q, seq_start, seq_len,
                             max_seq_len: int, tail_start, tail_len, max_tail_len: int, out, workspace,
                             scale: float = 0.0, stream=None):
    """Decode over a packed cache plus an fp16-format tail (one softmax)."""
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    pts, ptl = _seq(tail_start, tail_len, batch, "tail_start", "tail_len")
    po = _out(fmt, cache, out, batch, hq)
    pw, nw = _ws(workspace)
    if tail.n_layers != cache.n_layers or tail.n_kv_heads != cache.n_kv_heads:
        raise ValueError("tail: must have the cache's layers and KV heads")
    tb, cs, ts = tables.struct(), cache.struct(), tail.struct()
    _check(_lib.tq_decode_attention_tail(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), ctypes.byref(ts), pq,
                                         batch, hq, ps, pl, max_seq_len, pts, ptl, max_tail_len, scale, po, pw, nw,
                                         _stream(stream)), "tq_decode_attention_tail")


def tq_decode_partials(fmt: tq_format, tables: Tables, cache: Cache, batch: int, n_q_heads: int, seq_start, seq_len,
                       max_seq_len: int, workspace, scale: float = 0.0, stream=None):
    ps, pl = _seq(seq_start, seq_len, batch)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_partials(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), batch, n_q_heads, ps, pl,
                                   max_seq_len, scale, pw, nw, _stream(stream)), "tq_decode_partials")


def tq_decode_combine(fmt: tq_format, tables: Tables, cache: Cache, batch: int, n_q_heads: int, max_seq_len: int,
                      out, workspace, stream=None):
    po = _out(fmt, cache, out, batch, n_q_heads)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_combine(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), batch, n_q_heads, max_seq_len,
                                  po, pw, nw, _stream(stream)), "tq_decode_combine")


def tq_decode_attend(fmt: tq_format, tables: Tables, cache: Cache, batch: int, n_q_heads: int, seq_start, seq_len,
                     max_seq_len: int, out, workspace, scale: float = 0.0, stream=None):
    """Partials and their merge in one launch, on queries prepared in `workspace`."""
    ps, pl = _seq(seq_start, seq_len, batch)
    po = _out(fmt, cache, out, batch, n_q_heads)
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_decode_attend(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), batch, n_q_heads, ps, pl,
                                 max_seq_len, scale, po, pw, nw, _stream(stream)), "tq_decode_attend")


def tq_score(fmt: tq_format, tables: Tables, cache: Cache, q, seq_start, seq_len, max_seq_len: int, logits,
             workspace, scale: float = 0.0, stream=None):
    """logits: device float32 [n_layers][batch][n_q_heads][max_seq_len]."""
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    plg = _dev(logits, _f32(), (cache.n_layers, batch, hq, max(max_seq_len, 1)), "logits")
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_score(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pq, batch, hq, ps, pl, max_seq_len,
                         scale, plg, pw, nw, _stream(stream)), "tq_score")


def tq_score_multi(fmt: tq_format, tables: Tables, cache: Cache, q, seq_start, seq_len, max_seq_len: int, logits,
                   workspace, scale: float = 0.0, stream=None):
    """tq_score with the multi-query kernel (64 query rows per pass over a KV
    head's codes); logits: device float32 [n_layers][batch][n_q_heads][max_seq_len]."""
    pq, batch, hq = _q(fmt, cache, q)
    ps, pl = _seq(seq_start, seq_len, batch)
    plg = _dev(logits, _f32(), (cache.n_layers, batch, hq, max(max_seq_len, 1)), "logits")
    pw, nw = _ws(workspace)
    tb, cs = tables.struct(), cache.struct()
    _check(_lib.tq_score_multi(ctypes.byref(fmt), ctypes.byref(tb), ctypes.byref(cs), pq, batch, hq, ps, pl,
                               max_seq_len, scale, plg, pw, nw, _stream(stream)), "tq_score_multi")


def raw_call(name: str, *args):
    """Calls a C entry point with raw arguments and returns its status (for
    argument-validation tests)."""
    return getattr(_lib, name)(*args)
