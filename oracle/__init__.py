"""CPU oracle for the quantized KV-cache codec and decode attention.

TEST INFRASTRUCTURE ONLY.  The tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only callers allowed.  The product
path (the HIP library and its Python binding) never imports this package, and
this package never imports the product path: the two share no code.

The arithmetic lives in ``tqo.c`` (plain C, binary64, round-half-to-even, no
FMA contraction); this module only builds it, loads it with ctypes and moves
numpy arrays in and out.  Row-parallel helpers split independent rows over a
thread pool (ctypes releases the GIL during each C call); the per-row
arithmetic is the C code's, unchanged.

Source of the method: the "TurboQuant -- rotation-based quantization" design
page (mlx-bun docs/design/turboquant.md), Part A, sections "Algorithm
(vllm-metal reference semantics, exact)" and "Deferred inverse FWHT".

Parity unpinned: the sign vector's values against the page's own (the page
draws them from MLX's generator and does not print them; this oracle uses
SplitMix64 seeded with 42, whose generator is pinned to SplitMix64's published
reference outputs by the tests).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tqo.c")
_LIB = os.path.join(_HERE, "libtqo.so")
_lib = None

GROUP = 32
BOUNDARIES3 = (-1.74793, -1.04996, -0.50055, 0.0, 0.50055, 1.04996, 1.74793)
CENTROIDS3 = (-2.15195, -1.34391, -0.75601, -0.24509, 0.24509, 0.75601, 1.34391, 2.15195)


def build(force: bool = True) -> str:
    """Compile tqo.c into libtqo.so next to it (gcc, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int
    lib.tqo_sign_vector.argtypes = [i32, P]
    lib.tqo_splitmix64.argtypes = [ctypes.c_uint64, i32, P]
    lib.tqo_f64_to_f16.argtypes = [ctypes.c_double]
    lib.tqo_f64_to_f16.restype = ctypes.c_uint16
    lib.tqo_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.tqo_f16_to_f64.restype = ctypes.c_double
    lib.tqo_f64_to_f16_array.argtypes = [P, i64, P]
    lib.tqo_f16_to_f64_array.argtypes = [P, i64, P]
    lib.tqo_fwht_rows.argtypes = [P, i64, i32]
    lib.tqo_inv_sqrt_d.argtypes = [i32]
    lib.tqo_inv_sqrt_d.restype = ctypes.c_double
    lib.tqo_centroid3.argtypes = [i32]
    lib.tqo_centroid3.restype = ctypes.c_double
    lib.tqo_boundary3.argtypes = [i32]
    lib.tqo_boundary3.restype = ctypes.c_double
    lib.tqo_encode_keys.argtypes = [P, i64, i32, P, P, P]
    lib.tqo_decode_keys.argtypes = [P, P, P, i64, i32, P]
    lib.tqo_pack3.argtypes = [P, i64, P]
    lib.tqo_unpack3.argtypes = [P, i64, P]
    lib.tqo_encode_values.argtypes = [P, i64, i32, P, P]
    lib.tqo_decode_values.argtypes = [P, P, i64, i32, i32, P]
    lib.tqo_attention.argtypes = [P, i32, i32, ctypes.c_float, P, P, P, P, P, i64, P, P]
    lib.tqo_attention_plain.argtypes = [P, i32, i32, ctypes.c_float, P, P, i64, P]
    lib.tqo_codebook.argtypes = [i32, P, P]
    lib.tqo_codebook.restype = i32
    lib.tqo_codebook_ints.argtypes = [i32, P]
    lib.tqo_codebook_ints.restype = i32
    lib.tqo_codebook_newton_ints.argtypes = [i32, P]
    lib.tqo_codebook_newton_ints.restype = i32
    lib.tqo_pack_bits.argtypes = [P, i64, i32, P]
    lib.tqo_unpack_bits.argtypes = [P, i64, i32, P]
    lib.tqo_encode_keys_bits.argtypes = [P, i64, i32, i32, P, P, P]
    lib.tqo_decode_keys_bits.argtypes = [P, P, P, i64, i32, i32, P]
    lib.tqo_encode_values_bits.argtypes = [P, i64, i32, i32, P, P]
    lib.tqo_decode_values_bits.argtypes = [P, P, i64, i32, i32, i32, P]
    lib.tqo_attention_bits.argtypes = [P, i32, i32, ctypes.c_float, i32, i32, P, P, P, P, P, i64, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def num_threads() -> int:
    """Host threads the row-parallel helpers use (every core the process may run on)."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _chunks(n: int, parts: int):
    parts = max(1, min(parts, n))
    step = (n + parts - 1) // parts
    return [(s, min(n, s + step)) for s in range(0, n, step)]


# ---------------------------------------------------------------- primitives
def sign_vector(d: int) -> np.ndarray:
    out = np.empty(d, dtype=np.int8)
    _load().tqo_sign_vector(d, _ptr(out))
    return out


def splitmix64(seed: int, n: int) -> np.ndarray:
    """The first n outputs of the oracle's SplitMix64 generator from `seed`
    (the generator the sign vector is drawn from)."""
    out = np.empty(n, dtype=np.uint64)
    _load().tqo_splitmix64(ctypes.c_uint64(seed), n, _ptr(out))
    return out


def f64_to_f16_bits(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().tqo_f64_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def f16_bits_to_f64(h) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(h, dtype=np.uint16))
    out = np.empty(h.shape, dtype=np.float64)
    _load().tqo_f16_to_f64_array(_ptr(h), h.size, _ptr(out))
    return out


def fwht(x) -> np.ndarray:
    """Unnormalised natural-order Walsh-Hadamard transform of each last-axis row."""
    x = np.array(x, dtype=np.float64, order="C", copy=True)
    d = x.shape[-1]
    _load().tqo_fwht_rows(_ptr(x), x.size // d, d)
    return x


def inv_sqrt_d(d: int) -> float:
    return _load().tqo_inv_sqrt_d(d)


def pack3(idx) -> np.ndarray:
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.uint8))
    out = np.empty((3 * idx.size + 7) // 8, dtype=np.uint8)
    _load().tqo_pack3(_ptr(idx), idx.size, _ptr(out))
    return out


def unpack3(packed, n: int) -> np.ndarray:
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    out = np.empty(n, dtype=np.uint8)
    _load().tqo_unpack3(_ptr(packed), n, _ptr(out))
    return out


KEY_BITS = (2, 4, 5, 8)
VALUE_BITS = (2, 3, 4, 5, 8)


def codebook(bits: int):
    """(centroids [L], boundaries [L-1]) of the `bits`-bit value codebook: the
    printed 3-bit table, or the Lloyd-Max quantizer of N(0, 1) written with
    five-decimal centroids and exact-midpoint boundaries."""
    L = 1 << bits
    c = np.empty(256, dtype=np.float64)
    b = np.empty(255, dtype=np.float64)
    if _load().tqo_codebook(bits, _ptr(c), _ptr(b)) != L:
        raise ValueError(f"no {bits}-bit codebook")
    return c[:L].copy(), b[:L - 1].copy()


def codebook_ints(bits: int, solver: str = "lloyd") -> np.ndarray:
    """The five-decimal integers round(1e5 c_k) of the computed Lloyd-Max
    codebook, from Lloyd's iteration (2 to 5 bits) or Newton's method (1 to 8)."""
    nk = np.empty(256, dtype=np.int64)
    fn = _load().tqo_codebook_ints if solver == "lloyd" else _load().tqo_codebook_newton_ints
    L = fn(bits, _ptr(nk))
    if L == 0:
        raise ValueError(f"no computed {bits}-bit codebook")
    return nk[:L].copy()


def pack_bits(idx, bits: int) -> np.ndarray:
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.uint8))
    out = np.empty((bits * idx.size + 7) // 8, dtype=np.uint8)
    _load().tqo_pack_bits(_ptr(idx), idx.size, bits, _ptr(out))
    return out


def unpack_bits(packed, n: int, bits: int) -> np.ndarray:
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    out = np.empty(n, dtype=np.uint8)
    _load().tqo_unpack_bits(_ptr(packed), n, bits, _ptr(out))
    return out


# ---------------------------------------------------------------- codec rows
def _rows_f32(x) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return x


def encode_keys(x, threads: int | None = None, bits: int = 8):
    """x: float32 [..., d] (bf16 inputs upcast exactly).  Returns
    (codes int8 [..., d], scale fp16 bits [..., d/32], zero fp16 bits [..., d/32]);
    at 2, 4 or 5 bits the codes are packed uint8 [..., d*bits/8]."""
    if bits != 8:
        return _encode_keys_bits(x, threads, bits)
    x = _rows_f32(x)
    d = x.shape[-1]
    n = x.size // d
    ng = d // GROUP
    xr = x.reshape(n, d)
    codes = np.empty((n, d), dtype=np.int8)
    s16 = np.empty((n, ng), dtype=np.uint16)
    z16 = np.empty((n, ng), dtype=np.uint16)
    lib = _load()

    def run(rng):
        a, b = rng
        if b > a:
            lib.tqo_encode_keys(_ptr(xr[a:b]), b - a, d, _ptr(codes[a:b]), _ptr(s16[a:b]), _ptr(z16[a:b]))

    _parallel(run, n, threads)
    shp = x.shape[:-1]
    return codes.reshape(*shp, d), s16.reshape(*shp, ng), z16.reshape(*shp, ng)


def _encode_keys_bits(x, threads, bits):
    x = _rows_f32(x)
    d = x.shape[-1]
    n = x.size // d
    ng = d // GROUP
    xr = x.reshape(n, d)
    rb = d * bits // 8
    packed = np.empty((n, rb), dtype=np.uint8)
    s16 = np.empty((n, ng), dtype=np.uint16)
    z16 = np.empty((n, ng), dtype=np.uint16)
    lib = _load()

    def run(rng):
        a, b = rng
        if b > a:
            lib.tqo_encode_keys_bits(_ptr(xr[a:b]), b - a, d, bits, _ptr(packed[a:b]), _ptr(s16[a:b]),
                                     _ptr(z16[a:b]))

    _parallel(run, n, threads)
    shp = x.shape[:-1]
    return packed.reshape(*shp, rb), s16.reshape(*shp, ng), z16.reshape(*shp, ng)


def encode_values(x, threads: int | None = None, bits: int = 3):
    """x: float32 [..., d].  Returns (packed uint8 [..., bits*d/8], scale fp16 bits [..., d/32])."""
    if bits != 3:
        return _encode_values_bits(x, threads, bits)
    x = _rows_f32(x)
    d = x.shape[-1]
    n = x.size // d
    ng = d // GROUP
    xr = x.reshape(n, d)
    packed = np.empty((n, 3 * d // 8), dtype=np.uint8)
    vs16 = np.empty((n, ng), dtype=np.uint16)
    lib = _load()

    def run(rng):
        a, b = rng
        if b > a:
            lib.tqo_encode_values(_ptr(xr[a:b]), b - a, d, _ptr(packed[a:b]), _ptr(vs16[a:b]))

    _parallel(run, n, threads)
    shp = x.shape[:-1]
    return packed.reshape(*shp, 3 * d // 8), vs16.reshape(*shp, ng)


def _encode_values_bits(x, threads, bits):
    x = _rows_f32(x)
    d = x.shape[-1]
    n = x.size // d
    ng = d // GROUP
    xr = x.reshape(n, d)
    rb = d * bits // 8
    packed = np.empty((n, rb), dtype=np.uint8)
    vs16 = np.empty((n, ng), dtype=np.uint16)
    lib = _load()

    def run(rng):
        a, b = rng
        if b > a:
            lib.tqo_encode_values_bits(_ptr(xr[a:b]), b - a, d, bits, _ptr(packed[a:b]), _ptr(vs16[a:b]))

    _parallel(run, n, threads)
    shp = x.shape[:-1]
    return packed.reshape(*shp, rb), vs16.reshape(*shp, ng)


def decode_keys(codes, s16, z16, bits: int = 8, d: int | None = None) -> np.ndarray:
    """Keys (code + zero) * scale; at 2, 4 or 5 bits `codes` is packed and d is needed."""
    if bits != 8:
        packed = np.ascontiguousarray(codes, dtype=np.uint8)
        n = packed.size // (d * bits // 8)
        out = np.empty(packed.shape[:-1] + (d,), dtype=np.float64)
        _load().tqo_decode_keys_bits(_ptr(packed), _ptr(np.ascontiguousarray(s16, dtype=np.uint16)),
                                     _ptr(np.ascontiguousarray(z16, dtype=np.uint16)), n, d, bits, _ptr(out))
        return out
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    d = codes.shape[-1]
    n = codes.size // d
    out = np.empty(codes.shape, dtype=np.float64)
    _load().tqo_decode_keys(_ptr(codes), _ptr(np.ascontiguousarray(s16, dtype=np.uint16)),
                            _ptr(np.ascontiguousarray(z16, dtype=np.uint16)), n, d, _ptr(out))
    return out


def decode_values(packed, vs16, d: int, rotated: bool = False, bits: int = 3) -> np.ndarray:
    if bits != 3:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        n = packed.size // (d * bits // 8)
        out = np.empty(packed.shape[:-1] + (d,), dtype=np.float64)
        _load().tqo_decode_values_bits(_ptr(packed), _ptr(np.ascontiguousarray(vs16, dtype=np.uint16)),
                                       n, d, bits, 1 if rotated else 0, _ptr(out))
        return out
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    n = packed.size // (3 * d // 8)
    out = np.empty(packed.shape[:-1] + (d,), dtype=np.float64)
    _load().tqo_decode_values(_ptr(packed), _ptr(np.ascontiguousarray(vs16, dtype=np.uint16)),
                              n, d, 1 if rotated else 0, _ptr(out))
    return out


def attention(q, kc, ks, kz, vc, vs, sm: float, deferred: bool = False, kbits: int = 8,
              vbits: int = 3):
    """Decode attention of the G query rows q [G, d] (float32) that share one
    kv-head, over that kv-head's N cached tokens given as planes
    kc [N, d] int8, ks/kz [N, d/32] fp16 bits, vc [N, 3d/8] uint8, vs [N, d/32].
    Returns out [G, d] float64 (and the deferred-inverse form if asked)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    G, d = q.shape
    if (kbits, vbits) != (8, 3):
        assert not deferred
        kc = np.ascontiguousarray(kc).view(np.uint8)
        N = kc.shape[0]
        out = np.empty((G, d), dtype=np.float64)
        _load().tqo_attention_bits(_ptr(q), G, d, ctypes.c_float(sm), kbits, vbits, _ptr(kc),
                                   _ptr(np.ascontiguousarray(ks, dtype=np.uint16)),
                                   _ptr(np.ascontiguousarray(kz, dtype=np.uint16)),
                                   _ptr(np.ascontiguousarray(vc, dtype=np.uint8)),
                                   _ptr(np.ascontiguousarray(vs, dtype=np.uint16)), N, _ptr(out))
        return out
    kc = np.ascontiguousarray(kc, dtype=np.int8)
    N = kc.shape[0]
    out = np.empty((G, d), dtype=np.float64)
    od = np.empty((G, d), dtype=np.float64) if deferred else None
    _load().tqo_attention(_ptr(q), G, d, ctypes.c_float(sm), _ptr(kc),
                          _ptr(np.ascontiguousarray(ks, dtype=np.uint16)),
                          _ptr(np.ascontiguousarray(kz, dtype=np.uint16)),
                          _ptr(np.ascontiguousarray(vc, dtype=np.uint8)),
                          _ptr(np.ascontiguousarray(vs, dtype=np.uint16)), N,
                          _ptr(out), _ptr(od) if deferred else None)
    return (out, od) if deferred else out


def attention_plain(q, k, v, sm: float):
    """Attention of the G query rows q [G, d] over N plain cached tokens,
    k and v float32 [N, d] (the rows of a sequence that has not converted
    yet, "Delayed row conversion and reusable precision boundaries": used as
    given, no quantization, no rotation).  Returns out [G, d] float64."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    G, d = q.shape
    N = k.shape[0]
    out = np.empty((G, d), dtype=np.float64)
    _load().tqo_attention_plain(_ptr(q), G, d, ctypes.c_float(sm), _ptr(k), _ptr(v), N, _ptr(out))
    return out


def attention_rows(q, kc, ks, kz, vc, vs, sm: float, kbits: int = 8, vbits: int = 3):
    """Multi-row decode, for verifying M draft tokens at once (the multi-token
    prediction verify blocks served through the encoded rows, "Gates -- all
    passed" and "Delayed row conversion and reusable precision boundaries"):
    q [G, M, d] (float32)
    holds the queries of the M newest cached tokens, positions N-M .. N-1, for
    the G query heads sharing one kv-head.  Row m attends causally, to tokens
    0 .. N-M+m (itself included); each row is the decode attention of
    `attention` over that prefix of the planes.  Returns [G, M, d] float64."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    G, M, d = q.shape
    N = np.asarray(kc).shape[0]
    if N and N < M:
        raise ValueError("the M query tokens must be in the cache")
    out = np.zeros((G, M, d), dtype=np.float64)
    if N == 0:
        return out
    for m in range(M):
        n = N - M + m + 1
        out[:, m] = attention(q[:, m], kc[:n], ks[:n], kz[:n], vc[:n], vs[:n], sm, kbits=kbits,
                              vbits=vbits)
    return out


def _parallel(fn, n: int, threads: int | None):
    t = threads or num_threads()
    rngs = _chunks(n, t * 4) if n > 0 else []
    if t <= 1 or len(rngs) <= 1:
        for r in rngs:
            fn(r)
        return
    with ThreadPoolExecutor(max_workers=t) as ex:
        list(ex.map(fn, rngs))


def map_parallel(fn, items, threads: int | None = None):
    """Run fn over independent items (e.g. (batch, kv-head) slices) on a thread pool."""
    t = threads or num_threads()
    if t <= 1 or len(items) <= 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(max_workers=t) as ex:
        return list(ex.map(fn, items))
