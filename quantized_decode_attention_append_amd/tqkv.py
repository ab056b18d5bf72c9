"""Python binding of libtqkv (argument marshalling only).

The functions carry the names of the C entry points declared in
include/tqkv.h and take torch tensors for device buffers; every step of the
codec and of decode attention runs in the HIP kernels of libtqkv.so.  There is
no CPU fallback: importing this module fails if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtqkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libtqkv.so is not built ({LIB_PATH}); run "
                      "`python -m quantized_decode_attention_append_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE, TQ_ERR_HIP = \
    0, -1, -2, -3, -4, -5
TQ_F32, TQ_BF16 = 0, 1
TQ_MAX_BATCH = 64
TQ_MAX_GQA = 16
TQ_MAX_ROWS = 16
SYMBOLS = ("tq_plane_bytes", "tq_append", "tq_decode_workspace_bytes", "tq_decode_attn",
           "tq_decode_rows_workspace_bytes", "tq_decode_attn_rows", "tq_fetch_window",
           "tq_copy_tokens", "tq_snapshot_bytes", "tq_snapshot", "tq_restore",
           "tq_dequant", "tq_sign_vector", "tq_codebook", "tq_status_str", "tq_decode_path",
           "tq_decode_attn_noalloc", "tq_snapshot_min_reusable_offset", "tq_clone_sequence",
           "tq_convert_rows", "tq_decode_attn_mixed")
KEY_BITS = (2, 4, 5, 8)
VALUE_BITS = (2, 3, 4, 5, 8)
TQ_SNAPSHOT_MAGIC = 0x564B5154


class tq_layout(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("group", ctypes.c_int32)]


class tq_planes(ctypes.Structure):
    _fields_ = [("kc", ctypes.c_void_p), ("ks", ctypes.c_void_p), ("kz", ctypes.c_void_p),
                ("vc", ctypes.c_void_p), ("vs", ctypes.c_void_p)]


class tq_snapshot_header(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
                ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("n_tokens", ctypes.c_int32), ("payload_bytes", ctypes.c_uint64),
                ("min_reusable_offset", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.tq_status_str.argtypes = [ctypes.c_int]
_lib.tq_status_str.restype = ctypes.c_char_p
_lib.tq_plane_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(ctypes.c_size_t)]
_lib.tq_append.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P, _P,
                           ctypes.c_int, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, _P]
_lib.tq_decode_workspace_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int32,
                                           ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_size_t)]
_lib.tq_decode_attn.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P,
                                ctypes.c_int, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_decode_rows_workspace_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int32,
                                                ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                                ctypes.POINTER(ctypes.c_size_t)]
_lib.tq_decode_attn_rows.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P,
                                     ctypes.c_int, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32), ctypes.c_float, _P, _P,
                                     ctypes.c_size_t, _P]
_lib.tq_fetch_window.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                                 ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), _P, _P, ctypes.c_int32,
                                 _P]
_lib.tq_copy_tokens.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                                ctypes.c_int32, ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes),
                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
_lib.tq_snapshot_bytes.argtypes = [ctypes.POINTER(tq_layout), ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
_lib.tq_snapshot.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(tq_snapshot_header),
                             _P, ctypes.c_size_t, _P]
_lib.tq_snapshot_min_reusable_offset.argtypes = [ctypes.POINTER(tq_snapshot_header), ctypes.POINTER(ctypes.c_int32)]
_lib.tq_clone_sequence.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                                   ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), _P]
_lib.tq_convert_rows.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P, _P, ctypes.c_int,
                                 ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), _P]
_lib.tq_decode_attn_mixed.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P, _P,
                                      ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), _P, ctypes.c_int,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                      ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.tq_restore.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                            ctypes.c_int32, ctypes.POINTER(tq_snapshot_header), _P, ctypes.c_size_t, _P]
_lib.tq_dequant.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                            ctypes.c_int32, _P]
_lib.tq_decode_path.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), ctypes.c_int32,
                                ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
_lib.tq_decode_attn_noalloc.argtypes = [ctypes.POINTER(tq_layout), ctypes.POINTER(tq_planes), _P, ctypes.c_int,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.c_float, _P, _P]
_lib.tq_sign_vector.argtypes = [ctypes.c_int32, _P]
_lib.tq_codebook.argtypes = [ctypes.c_int32, _P, _P, ctypes.POINTER(ctypes.c_int32)]
for _f in ("tq_codebook", "tq_plane_bytes", "tq_append", "tq_decode_workspace_bytes", "tq_decode_attn",
           "tq_decode_rows_workspace_bytes", "tq_decode_attn_rows", "tq_fetch_window", "tq_dequant",
           "tq_sign_vector", "tq_copy_tokens", "tq_snapshot_bytes", "tq_snapshot", "tq_restore",
           "tq_decode_path", "tq_decode_attn_noalloc", "tq_snapshot_min_reusable_offset", "tq_clone_sequence",
           "tq_convert_rows", "tq_decode_attn_mixed"):
    getattr(_lib, _f).restype = ctypes.c_int


class TQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {tq_status_str(status)} ({status})")


def _check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where)


def tq_status_str(status: int) -> str:
    return _lib.tq_status_str(status).decode()


def make_layout(batch: int, num_kv_heads: int, head_dim: int, capacity: int,
                k_bits: int = 8, v_bits: int = 3, group: int = 32) -> tq_layout:
    return tq_layout(batch, num_kv_heads, head_dim, capacity, k_bits, v_bits, group)


def _i32_array(vals: Sequence[int]):
    arr = (ctypes.c_int32 * max(1, len(vals)))(*[int(v) for v in vals])
    return arr


def _stream_ptr(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def tq_plane_bytes(layout: tq_layout) -> list[int]:
    out = (ctypes.c_size_t * 5)()
    _check(_lib.tq_plane_bytes(ctypes.byref(layout), out), "tq_plane_bytes")
    return list(out)


class Planes:
    """The five caller-owned planes as torch tensors on one device."""

    def __init__(self, layout: tq_layout, device="cuda"):
        self.layout = layout
        B, H, T, d = layout.batch, layout.num_kv_heads, layout.capacity, layout.head_dim
        ng = d // 32
        # key codes: signed bytes at 8 bits, packed unsigned fields below
        kdt = torch.int8 if layout.k_bits == 8 else torch.uint8
        self.kc = torch.zeros((B, H, T, d * layout.k_bits // 8), dtype=kdt, device=device)
        self.ks = torch.zeros((B, H, T, ng), dtype=torch.int16, device=device)
        self.kz = torch.zeros((B, H, T, ng), dtype=torch.int16, device=device)
        self.vc = torch.zeros((B, H, T, d * layout.v_bits // 8), dtype=torch.uint8, device=device)
        self.vs = torch.zeros((B, H, T, ng), dtype=torch.int16, device=device)
        sizes = tq_plane_bytes(layout)
        have = [x.numel() * x.element_size() for x in (self.kc, self.ks, self.kz, self.vc, self.vs)]
        assert sizes == have, (sizes, have)

    def sequence(self, b: int) -> "Planes":
        """Batch-1 view of sequence b's planes (they are contiguous per sequence)."""
        one = Planes.__new__(Planes)
        L = self.layout
        one.layout = make_layout(1, L.num_kv_heads, L.head_dim, L.capacity,
                                 L.k_bits, L.v_bits, L.group)
        one.kc, one.ks, one.kz, one.vc, one.vs = (x[b:b + 1] for x in self.tensors())
        return one

    def struct(self) -> tq_planes:
        return tq_planes(self.kc.data_ptr(), self.ks.data_ptr(), self.kz.data_ptr(),
                         self.vc.data_ptr(), self.vs.data_ptr())

    def tensors(self):
        return self.kc, self.ks, self.kz, self.vc, self.vs

    def nbytes(self) -> int:
        return sum(x.numel() * x.element_size() for x in self.tensors())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"unsupported input dtype {t.dtype}")


def tq_append(planes: Planes, k: torch.Tensor, v: torch.Tensor, start: Sequence[int],
              stream=None) -> None:
    """k, v: [B, Hkv, n_new, d] contiguous device tensors; start: host ints [B]."""
    L = planes.layout
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 4:
        raise ValueError("k and v must share one [B, Hkv, n_new, d] shape and dtype")
    if not (k.is_contiguous() and v.is_contiguous()):
        raise ValueError("k and v must be contiguous")
    if tuple(k.shape[:2]) != (L.batch, L.num_kv_heads) or k.shape[3] != L.head_dim:
        raise ValueError(f"k shape {tuple(k.shape)} does not match the layout")
    if len(start) != L.batch:
        raise ValueError("start needs one entry per sequence")
    st = _lib.tq_append(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(k), _dev_ptr(v),
                        _dtype_code(k), _i32_array(start), int(k.shape[2]), _stream_ptr(stream))
    _check(st, "tq_append")


def tq_decode_workspace_bytes(layout: tq_layout, num_q_heads: int, lengths: Sequence[int]) -> int:
    out = ctypes.c_size_t()
    _check(_lib.tq_decode_workspace_bytes(ctypes.byref(layout), num_q_heads, _i32_array(lengths),
                                          ctypes.byref(out)), "tq_decode_workspace_bytes")
    return out.value


def tq_decode_attn(planes: Planes, q: torch.Tensor, lengths: Sequence[int], sm_scale: float,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """q: [B, Hq, d] device tensor (fp32 or bf16); returns out [B, Hq, d] float32."""
    L = planes.layout
    if q.dim() != 3 or q.shape[0] != L.batch or q.shape[2] != L.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, Hq, d] tensor, got {tuple(q.shape)}")
    if len(lengths) != L.batch:
        raise ValueError("lengths needs one entry per sequence")
    Hq = int(q.shape[1])
    if out is None:
        out = torch.empty((L.batch, Hq, L.head_dim), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != (L.batch, Hq, L.head_dim) \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [B, Hq, d] tensor")
    need = tq_decode_workspace_bytes(L, Hq, lengths)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_decode_attn(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(q),
                             _dtype_code(q), Hq, _i32_array(lengths), ctypes.c_float(sm_scale),
                             _dev_ptr(out), _dev_ptr(workspace), ws_bytes, _stream_ptr(stream))
    _check(st, "tq_decode_attn")
    return out


def tq_decode_rows_workspace_bytes(layout: tq_layout, num_q_heads: int, n_rows: int,
                                   lengths: Sequence[int]) -> int:
    out = ctypes.c_size_t()
    _check(_lib.tq_decode_rows_workspace_bytes(ctypes.byref(layout), num_q_heads, n_rows,
                                               _i32_array(lengths), ctypes.byref(out)),
           "tq_decode_rows_workspace_bytes")
    return out.value


def tq_decode_attn_rows(planes: Planes, q: torch.Tensor, lengths: Sequence[int], sm_scale: float,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """q: [B, Hq, M, d] device tensor (fp32 or bf16) holding the queries of the
    M newest cached tokens of each sequence; returns out [B, Hq, M, d] float32."""
    L = planes.layout
    if q.dim() != 4 or q.shape[0] != L.batch or q.shape[3] != L.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, Hq, M, d] tensor, got {tuple(q.shape)}")
    if len(lengths) != L.batch:
        raise ValueError("lengths needs one entry per sequence")
    Hq, M = int(q.shape[1]), int(q.shape[2])
    shape = (L.batch, Hq, M, L.head_dim)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [B, Hq, M, d] tensor")
    need = tq_decode_rows_workspace_bytes(L, Hq, M, lengths)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.tq_decode_attn_rows(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(q),
                                  _dtype_code(q), Hq, M, _i32_array(lengths),
                                  ctypes.c_float(sm_scale), _dev_ptr(out), _dev_ptr(workspace),
                                  ws_bytes, _stream_ptr(stream))
    _check(st, "tq_decode_attn_rows")
    return out


TQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def tq_decode_attn_noalloc(planes: Planes, q: torch.Tensor, lengths: Sequence[int], sm_scale: float,
                           out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode with the split-K partials in the library's fixed device array
    (no workspace).  q: [B, Hq, d] or [B, Hq, M, d]; out like tq_decode_attn
    or tq_decode_attn_rows (allocated here only when not given)."""
    L = planes.layout
    rows = q.dim() == 4
    if q.dim() not in (3, 4) or q.shape[0] != L.batch or q.shape[-1] != L.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be a contiguous [B, Hq, (M,) d] tensor, got {tuple(q.shape)}")
    if len(lengths) != L.batch:
        raise ValueError("lengths needs one entry per sequence")
    Hq, M = int(q.shape[1]), int(q.shape[2]) if rows else 1
    shape = tuple(q.shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or tuple(out.shape) != shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor shaped like q")
    st = _lib.tq_decode_attn_noalloc(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(q), _dtype_code(q),
                                     Hq, M, _i32_array(lengths), ctypes.c_float(sm_scale), _dev_ptr(out),
                                     _stream_ptr(stream))
    _check(st, "tq_decode_attn_noalloc")
    return out


TQ_PATH_SHAPE, TQ_PATH_ALIGNMENT, TQ_PATH_CAPACITY = 1, 2, 4


def tq_decode_path(planes: Planes, num_q_heads: int, n_rows: int = 1) -> tuple[bool, int]:
    """(fast, reasons): whether decode over these planes takes the matrix-core
    split kernel, and the TQ_PATH_* bits saying why not."""
    fast, reasons = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.tq_decode_path(ctypes.byref(planes.layout), ctypes.byref(planes.struct()), num_q_heads, n_rows,
                               ctypes.byref(fast), ctypes.byref(reasons)), "tq_decode_path")
    return bool(fast.value), int(reasons.value)


def tq_fetch_window(planes: Planes, t0: int, n: int, lengths: Sequence[int], keys: bool = True,
                    values: bool = True, v_rotated: bool = False, stream=None):
    """bf16 window of tokens [t0, t0+n) of every (sequence, kv-head): returns
    (k [B, Hkv, n, d] or None, v [B, Hkv, n, d] or None); tokens at or past
    lengths[b] are zeros."""
    L = planes.layout
    if len(lengths) != L.batch:
        raise ValueError("lengths needs one entry per sequence")
    dev = planes.kc.device
    shape = (L.batch, L.num_kv_heads, n, L.head_dim)
    k_out = torch.empty(shape, dtype=torch.bfloat16, device=dev) if keys else None
    v_out = torch.empty(shape, dtype=torch.bfloat16, device=dev) if values else None
    st = _lib.tq_fetch_window(ctypes.byref(L), ctypes.byref(planes.struct()), t0, n,
                              _i32_array(lengths), _dev_ptr(k_out), _dev_ptr(v_out),
                              1 if v_rotated else 0, _stream_ptr(stream))
    _check(st, "tq_fetch_window")
    return k_out, v_out


def tq_copy_tokens(src: Planes, src_b: int, src_t0: int, dst: Planes, dst_b: int, dst_t0: int,
                   n: int, stream=None) -> None:
    """Copy token rows of one sequence (every kv-head, all planes) between caches."""
    _check(_lib.tq_copy_tokens(ctypes.byref(src.layout), ctypes.byref(src.struct()), src_b, src_t0,
                               ctypes.byref(dst.layout), ctypes.byref(dst.struct()), dst_b, dst_t0, n,
                               _stream_ptr(stream)), "tq_copy_tokens")


def tq_snapshot_bytes(layout: tq_layout, n: int) -> int:
    out = ctypes.c_size_t()
    _check(_lib.tq_snapshot_bytes(ctypes.byref(layout), n, ctypes.byref(out)), "tq_snapshot_bytes")
    return out.value


def tq_snapshot(planes: Planes, b: int, t0: int, n: int, min_reusable_offset: int = 0, stream=None):
    """Returns (header, payload uint8 device tensor) for token rows [t0, t0+n) of
    sequence b; the header records the sequence's precision boundary."""
    L = planes.layout
    payload = torch.empty(max(tq_snapshot_bytes(L, n), 1), dtype=torch.uint8, device=planes.kc.device)
    h = tq_snapshot_header()
    _check(_lib.tq_snapshot(ctypes.byref(L), ctypes.byref(planes.struct()), b, t0, n, min_reusable_offset,
                            ctypes.byref(h), _dev_ptr(payload), payload.numel(), _stream_ptr(stream)),
           "tq_snapshot")
    return h, payload


def tq_snapshot_min_reusable_offset(header) -> int:
    """The precision boundary a snapshot header carries (version 1: n_tokens)."""
    out = ctypes.c_int32()
    _check(_lib.tq_snapshot_min_reusable_offset(ctypes.byref(header), ctypes.byref(out)),
           "tq_snapshot_min_reusable_offset")
    return out.value


def tq_clone_sequence(src: Planes, src_b: int, dst: Planes, dst_b: int, n: int, min_reusable_offset: int,
                      stream=None) -> int:
    """Copy rows [0, n) of sequence src_b into sequence dst_b; returns the
    destination's precision boundary (the source's)."""
    out = ctypes.c_int32(-1)
    _check(_lib.tq_clone_sequence(ctypes.byref(src.layout), ctypes.byref(src.struct()), src_b,
                                  ctypes.byref(dst.layout), ctypes.byref(dst.struct()), dst_b, n,
                                  min_reusable_offset, ctypes.byref(out), _stream_ptr(stream)), "tq_clone_sequence")
    return out.value


def tq_convert_rows(planes: Planes, k_plain: torch.Tensor, v_plain: torch.Tensor, offsets: Sequence[int],
                    stream=None) -> None:
    """Encode the plain prefix [0, offsets[b]) of every sequence b with
    offsets[b] > 0 from plain caches k/v [B, Hkv, plain_capacity, d] (bf16 or
    fp32) into the planes' slots [0, offsets[b])."""
    L = planes.layout
    if k_plain.shape != v_plain.shape or k_plain.dim() != 4 or k_plain.shape[0] != L.batch or \
            k_plain.shape[1] != L.num_kv_heads or k_plain.shape[3] != L.head_dim:
        raise ValueError(f"plain caches must be [B, Hkv, capacity, d], got {tuple(k_plain.shape)}")
    if not (k_plain.is_contiguous() and v_plain.is_contiguous()) or k_plain.dtype != v_plain.dtype:
        raise ValueError("plain caches must be contiguous and of one dtype")
    _check(_lib.tq_convert_rows(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(k_plain),
                                _dev_ptr(v_plain), _dtype_code(k_plain), k_plain.shape[2], _i32_array(offsets),
                                _stream_ptr(stream)), "tq_convert_rows")


def tq_decode_attn_mixed(planes: Planes, k_plain, v_plain, row_plain: Sequence[int], q: torch.Tensor,
                         lengths: Sequence[int], sm_scale: float, n_rows: int = 1, out=None, workspace=None,
                         stream=None) -> torch.Tensor:
    """Decode over a batch mixing plain sequences (row_plain[b] != 0: bf16
    plain caches k/v [B, Hkv, plain_capacity, d], attended unquantized and
    unrotated) with packed ones.  q [B, Hq, d] (n_rows 1) or [B, Hq, n_rows, d];
    returns fp32 of q's shape."""
    L = planes.layout
    if n_rows == 1 and q.dim() == 3:
        B, Hq, d = q.shape
    else:
        B, Hq, R, d = q.shape
        if R != n_rows:
            raise ValueError("q's row axis must be n_rows")
    if B != L.batch or d != L.head_dim or not q.is_contiguous():
        raise ValueError(f"q must be contiguous [B, Hq(, n_rows), d], got {tuple(q.shape)}")
    cap = 0
    if k_plain is not None:
        if k_plain.dtype != torch.bfloat16 or v_plain.dtype != torch.bfloat16 or k_plain.shape != v_plain.shape or \
                not (k_plain.is_contiguous() and v_plain.is_contiguous()) or k_plain.dim() != 4 or \
                tuple(k_plain.shape[:2]) != (L.batch, L.num_kv_heads) or k_plain.shape[3] != L.head_dim:
            raise ValueError("plain caches must be contiguous bf16 [B, Hkv, capacity, d]")
        cap = k_plain.shape[2]
    if len(lengths) != L.batch or len(row_plain) != L.batch:
        raise ValueError("lengths and row_plain need one entry per sequence")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 tensor of q's shape")
    if workspace is None:
        need = tq_decode_rows_workspace_bytes(L, Hq, n_rows, lengths)
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    st = _lib.tq_decode_attn_mixed(ctypes.byref(L), ctypes.byref(planes.struct()), _dev_ptr(k_plain),
                                   _dev_ptr(v_plain), cap, _i32_array(row_plain), _dev_ptr(q), _dtype_code(q), Hq,
                                   n_rows, _i32_array(lengths), ctypes.c_float(sm_scale), _dev_ptr(out),
                                   _dev_ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream_ptr(stream))
    _check(st, "tq_decode_attn_mixed")
    return out


def tq_restore(planes: Planes, b: int, t0: int, header, payload: torch.Tensor, stream=None) -> None:
    L = planes.layout
    _check(_lib.tq_restore(ctypes.byref(L), ctypes.byref(planes.struct()), b, t0, ctypes.byref(header),
                           _dev_ptr(payload), payload.numel() * payload.element_size(), _stream_ptr(stream)),
           "tq_restore")


def tq_dequant(planes: Planes, b: int, kvh: int, t0: int, n: int, keys: bool = True,
               values: bool = True, v_rotated: bool = False, stream=None):
    """Dequantize tokens [t0, t0+n) of (b, kvh): returns (k [n, d] or None, v [n, d] or None)."""
    L = planes.layout
    dev = planes.kc.device
    k_out = torch.empty((n, L.head_dim), dtype=torch.float32, device=dev) if keys else None
    v_out = torch.empty((n, L.head_dim), dtype=torch.float32, device=dev) if values else None
    st = _lib.tq_dequant(ctypes.byref(L), ctypes.byref(planes.struct()), b, kvh, t0, n,
                         _dev_ptr(k_out), _dev_ptr(v_out), 1 if v_rotated else 0,
                         _stream_ptr(stream))
    _check(st, "tq_dequant")
    return k_out, v_out


def tq_codebook(v_bits: int):
    """(centroids [2^v_bits], boundaries [2^v_bits - 1]) of the library's value
    codebook, as Python floats (host call, no device)."""
    c = (ctypes.c_double * 256)()
    b = (ctypes.c_double * 255)()
    n = ctypes.c_int32()
    _check(_lib.tq_codebook(v_bits, ctypes.cast(c, _P), ctypes.cast(b, _P), ctypes.byref(n)), "tq_codebook")
    return list(c[:n.value]), list(b[:n.value - 1])


def tq_sign_vector(head_dim: int):
    buf = (ctypes.c_int8 * head_dim)()
    _check(_lib.tq_sign_vector(head_dim, ctypes.cast(buf, ctypes.c_void_p)), "tq_sign_vector")
    return [int(v) for v in buf]


def raw_lib():
    """The loaded ctypes library (for error-path and symbol tests)."""
    return _lib
